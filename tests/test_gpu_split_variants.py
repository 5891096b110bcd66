"""GPU parity of the optional split-KV kernels for bf16 pools, which the library runs
when MLA_SPLITKV selects them (default: the four-wave kernel):
  8  eight waves, two per SIMD: each wave 32 query rows and a quarter of the
     contraction and of the output columns;
  q  four waves, each holding the whole 64-row M-tile with a quarter of the
     contraction and of the output columns.
Same bar as tests/test_gpu_parity.py."""
import math
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import mla_attention_folded, mla_attention_rows  # noqa: E402
import mla_latent_kv_16_amd as mla  # noqa: E402
from mla_latent_kv_16_amd.workloads import make_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-split-variant]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True, params=["8", "q"], ids=["eight-wave", "quarter"])
def _variant(request, monkeypatch):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(mla.LIB_PATH):
        pytest.fail("libmla.so is not built")
    monkeypatch.setenv("MLA_SPLITKV", request.param)
    say(f"MLA_SPLITKV={request.param}")


def run(w, parts=0, fn=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    fn = fn or mla.decode
    say(f"{fn.__name__} B={w.B} Sq={w.Sq} H={w.H} L={w.seq_lens.tolist()[:4]} parts={parts}")
    O, lse = fn(t(w.q_nope), t(w.q_rope), t(w.kv_pool), torch.from_numpy(w.block_table).cuda(),
                torch.from_numpy(w.seq_lens).cuda(), float(w.scale), causal=w.causal,
                num_partitions=parts)
    torch.cuda.synchronize()
    return O.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(O, lse, O_ref, lse_ref, what):
    assert np.isfinite(O).all() and np.isfinite(lse).all(), what
    d = np.abs(O - O_ref)
    rms = math.sqrt(float((O_ref ** 2).mean()))
    dl = float(np.abs(lse - lse_ref).max())
    say(f"{what}: max|dO|={d.max():.2e} mean|dO|={d.mean():.2e} rms(O)={rms:.3f} max|dLSE|={dl:.2e}")
    assert d.max() <= 2e-2 * rms and d.mean() <= 2e-3 * rms and dl <= 1e-3, what
    if rms <= 1.0:
        assert d.max() <= 2e-2 and d.mean() <= 2e-3, what


CASES = [
    ("spec4-short", dict(seed=201, B=3, Sq=4, H=16, lens=("uniform", 700, 3000)), 0),
    ("spec16-short", dict(seed=202, B=2, Sq=16, H=16, lens=("uniform", 1000, 2200)), 0),
    ("odd-M-split", dict(seed=203, B=2, Sq=3, H=5, lens=("uniform", 130, 700)), 7),
    ("tail-shorter-than-drafts", dict(seed=204, B=2, Sq=6, H=16, lens=("fixed", 64 * 9 + 2)), 3),
    ("non-causal", dict(seed=205, B=2, Sq=4, H=16, lens=("uniform", 300, 900), causal=False), 2),
    ("peaked-q4", dict(seed=206, B=2, Sq=4, H=16, lens=("uniform", 500, 1500), q_sigma=4.0), 0),
    ("one-page-per-part", dict(seed=207, B=1, Sq=2, H=16, lens=("fixed", 150)), 11),
]


@pytest.mark.parametrize("name,kw,parts", CASES, ids=[c[0] for c in CASES])
def test_matches_oracle(name, kw, parts):
    w = make_workload("tiny", **kw)
    O, lse = run(w, parts)
    check(O, lse, *mla_attention_folded(w.q_nope, w.q_rope, w.kv_pool, w.block_table,
                                        w.seq_lens, w.scale, w.causal), name)


def test_rescale_walks():
    """Keys x8 on later pages: the piece is walked again from the true maxima."""
    from mla_latent_kv_16_amd.workloads import f32_to_bf16_bits
    w = make_workload("tiny", seed=208, B=2, Sq=4, H=16, lens=("fixed", 64 * 12 + 5), q_sigma=4.0)
    f = (w.kv_pool.astype(np.uint32) << 16).view(np.float32)
    for b in range(w.B):
        for p in range(6, 13):
            f[w.block_table[b, p]] *= 8.0
    w.kv_pool = f32_to_bf16_bits(f)
    ref = mla_attention_folded(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                               w.scale, True)
    for parts in (1, 3):
        check(*run(w, parts), *ref, f"rescale parts={parts}")


def test_prefill_full_size_sampled():
    """The prefix-prefill configuration (1,024 M-tiles): both ends of every M-tile."""
    w = make_workload("prefill")
    O, lse = run(w, fn=mla.prefill_with_prefix)
    M = w.Sq * w.H
    rows = sorted({r for mt in range(M // 64) for r in (64 * mt, 64 * mt + 63)})
    for c0 in range(0, len(rows), 512):
        part = rows[c0:c0 + 512]
        o_ref, l_ref = mla_attention_rows(w.q_nope, w.q_rope, w.kv_pool, w.block_table,
                                          w.seq_lens, w.scale, True, 0, part)
        check(O[0].reshape(M, 512)[part], lse[0].reshape(M)[part], o_ref, l_ref,
              f"prefill rows {part[0]}..{part[-1]}")
