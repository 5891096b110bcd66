"""GPU checks of the absorb / project GEMMs (mla_absorb_q, mla_project_o) against
the oracle, and of the whole absorb -> latent decode -> project chain.

absorb: every product q*w of bf16 inputs is exact in fp32 and the 128-term sums
carry fp32 rounding only, then the result is rounded to bf16: |got - ref| <=
2^-8 |ref| + 1e-6.  project: O is rounded to bf16 for the MFMA (the kernel's
stated precision), so the tight check is against the oracle fed that rounded O,
within the fp32 accumulation bound 1e-5 * sum_c |O_c W_vc|; against the unrounded
O the output stays within 2e-2 * rms max and 2e-3 * rms mean."""
import math
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import absorb_q, bf16_bits_to_f64, mla_attention_folded, project_o  # noqa: E402
import mla_latent_kv_16_amd as mla  # noqa: E402
from mla_latent_kv_16_amd.workloads import f32_to_bf16_bits, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-proj]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(mla.LIB_PATH):
        pytest.fail("libmla.so is not built")
    torch.cuda.init()


def bf(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def weights(H, seed):
    rng = np.random.default_rng(seed)
    w_uk_t = bf(rng.standard_normal((H, 512, 128)) / math.sqrt(128))
    w_uv = bf(rng.standard_normal((H, 128, 512)) / math.sqrt(512))
    return w_uk_t, w_uv


@pytest.mark.parametrize("B,Sq,H", [(4, 4, 16), (3, 5, 7), (16, 16, 16), (1, 1, 128), (1, 4096, 16)])
def test_absorb_matches_oracle(B, Sq, H):
    rng = np.random.default_rng(B * 100 + Sq)
    q = bf(rng.standard_normal((B, Sq, H, 128)))
    w_uk_t, _ = weights(H, 3)
    got = mla.absorb_q(dev16(q), dev16(w_uk_t))
    torch.cuda.synchronize()
    got = bf16_bits_to_f64(got.cpu().numpy().view(np.uint16))
    ref = absorb_q(q, w_uk_t)
    err = np.abs(got - ref)
    say(f"absorb B={B} Sq={Sq} H={H}: max err {err.max():.2e}")
    assert (err <= 2.0 ** -8 * np.abs(ref) + 1e-6).all()


@pytest.mark.parametrize("B,Sq,H", [(4, 4, 16), (3, 5, 7), (16, 16, 16), (1, 4096, 16)])
def test_project_matches_oracle(B, Sq, H):
    rng = np.random.default_rng(B * 10 + H)
    O = (rng.standard_normal((B, Sq, H, 512)) * 0.3).astype(np.float32)
    _, w_uv = weights(H, 4)
    got = mla.project_o(torch.from_numpy(O).cuda(), dev16(w_uv))
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    O_bf = bf16_bits_to_f64(bf(O))                      # the kernel's rounding of O
    ref_bf = project_o(O_bf, w_uv)
    bound = 1e-5 * np.einsum("bthc,hvc->bthv", np.abs(O_bf), np.abs(bf16_bits_to_f64(w_uv)))
    assert (np.abs(got - ref_bf) <= bound + 1e-7).all()
    ref = project_o(O, w_uv)
    d = np.abs(got - ref)
    rms = math.sqrt(float((ref ** 2).mean()))
    say(f"project B={B} Sq={Sq} H={H}: max|d| {d.max():.2e} rms {rms:.3f}")
    assert d.max() <= 2e-2 * rms and d.mean() <= 2e-3 * rms


def test_absorb_decode_project_chain():
    """Per-head queries -> absorbed latent queries -> split-KV decode -> projected
    per-head outputs, all on the GPU, against the oracle's chain."""
    w = make_workload("tiny", seed=1201, B=3, Sq=4, H=16, lens=("uniform", 500, 1500))
    rng = np.random.default_rng(8)
    q_heads = bf(rng.standard_normal((w.B, w.Sq, w.H, 128)))
    w_uk_t, w_uv = weights(w.H, 9)
    q_lat = mla.absorb_q(dev16(q_heads), dev16(w_uk_t))
    O, lse = mla.decode(q_lat, dev16(w.q_rope), dev16(w.kv_pool),
                        torch.from_numpy(w.block_table).cuda(),
                        torch.from_numpy(w.seq_lens).cuda(), float(w.scale), True, 0)
    out = mla.project_o(O, dev16(w_uv))
    torch.cuda.synchronize()
    # the absorbed query is bf16 by definition of mla_absorb_q's output: the oracle's
    # fp64 result, rounded the same way (nearest, ties to even)
    q_ref = bf(absorb_q(q_heads, w_uk_t))
    O_ref, l_ref = mla_attention_folded(q_ref, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                                        w.scale, True)
    ref = project_o(O_ref, w_uv)
    got = out.cpu().numpy().astype(np.float64)
    d = np.abs(got - ref)
    rms = math.sqrt(float((ref ** 2).mean()))
    dl = np.abs(lse.cpu().numpy() - l_ref).max()
    say(f"chain: max|d| {d.max():.2e} mean|d| {d.mean():.2e} rms {rms:.3f} max|dLSE| {dl:.2e}")
    # the decode's bar, plus the projection's bf16 rounding of O (about 2^-9 relative)
    assert d.max() <= 3e-2 * rms and d.mean() <= 3e-3 * rms
    assert dl <= 1e-3
