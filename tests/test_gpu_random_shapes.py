"""GPU parity over seeded random shapes: every compute entry point family (two-pass and
single-pass decode, E4M3 and NoPE pools, draft trees, per-request draft counts, prefix
prefill) at batch sizes, draft counts, head counts, context lengths and partition
counts drawn at random (fixed seed, so the list is the same on every run), against
the fp64 oracle.  Same bar as the other parity tests: |dLSE| <= 1e-3, max |dO| <=
2e-2 * rms(O_ref) and mean |dO| <= 2e-3 * rms(O_ref), absolute where rms <= 1; padding
query slots of per-request draft counts must come back as O = 0, LSE = -inf.
Unused pages and rows past each length hold NaN codes, so any stray read shows up."""
import math
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import (E4M3Pool, mla_attention_folded, mla_attention_nope,  # noqa: E402
                    mla_attention_tree, mla_attention_varlen)
import mla_latent_kv_16_amd as mla  # noqa: E402
from mla_latent_kv_16_amd.workloads import PAGE, make_tree_masks, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_ABS = 2e-2, 2e-3, 1e-3
KINDS = ["decode", "single", "e4m3", "nope", "tree", "varlen", "prefill"]


def say(*a):
    print("[gpu-random]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(mla.LIB_PATH):
        pytest.fail("libmla.so is not built")
    torch.cuda.init()


def _draw_cases(n=70, seed=2024):
    """n cases, each (kind, workload keywords, partitions, extra seed), ten per kind."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kind = KINDS[i % len(KINDS)]
        if kind == "prefill":
            B, Sq, H = 1, int(rng.integers(24, 97)), int(rng.choice([1, 2, 4]))
        else:
            B = int(rng.integers(1, 7))
            Sq = int(rng.integers(1, 10))
            H = int(rng.choice([1, 3, 8, 16, 20, 32]))
        lo = max(Sq, int(rng.integers(1, 600)))
        hi = lo + int(rng.integers(0, 1800))
        causal = bool(rng.integers(0, 2)) if kind in ("decode", "single", "e4m3", "nope") \
            else True
        pages = B * ((hi + PAGE - 1) // PAGE)
        r = rng.random()
        parts = 0 if r < 0.4 else (int(rng.integers(1, 2 * pages + 2)) if r < 0.9
                                   else int(pages + rng.integers(1, 40)))
        kw = dict(seed=int(rng.integers(1, 1 << 30)), B=B, Sq=Sq, H=H, lens=("uniform", lo, hi),
                  causal=causal)
        cases.append((f"{i:02d}-{kind}-B{B}-Sq{Sq}-H{H}-L{lo}..{hi}-G{parts}", kind, kw, parts,
                      int(rng.integers(1, 1 << 30))))
    return cases


CASES = _draw_cases()


def _t16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _check(O, lse, O_ref, lse_ref, what, real=None):
    if real is not None:
        assert (O[~real] == 0).all() and np.isneginf(lse[~real]).all(), f"{what}: padding rows"
        O, O_ref, lse, lse_ref = O[real], O_ref[real], lse[real], lse_ref[real]
    assert np.isfinite(O).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    d = np.abs(O - O_ref)
    rms = math.sqrt(float((O_ref ** 2).mean()))
    dl = float(np.abs(lse - lse_ref).max())
    say(f"{what}: max|dO|={d.max():.2e} mean|dO|={d.mean():.2e} rms(O)={rms:.3f} max|dLSE|={dl:.2e}")
    assert d.max() <= MAX_ABS * rms and d.mean() <= MEAN_ABS * rms, what
    if rms <= 1.0:
        assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, what
    assert dl <= LSE_ABS, what


def _np(O, lse):
    torch.cuda.synchronize()
    return O.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name,kind,kw,parts,seed2", CASES, ids=[c[0] for c in CASES])
def test_random_shape_matches_oracle(name, kind, kw, parts, seed2):
    fmt = "e4m3" if kind == "e4m3" else "bf16"
    w = make_workload("tiny", kv_format=fmt, rope=kind != "nope", **kw)
    say(name)
    bt = torch.from_numpy(w.block_table).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    real = None
    if kind == "nope":
        O, lse = _np(*mla.decode_nope(_t16(w.q_nope), _t16(w.kv_pool), bt, sl, float(w.scale),
                                      causal=w.causal, num_partitions=parts))
        ref = mla_attention_nope(w.q_nope, w.kv_pool, w.block_table, w.seq_lens, w.scale,
                                 w.causal)
    elif kind == "e4m3":
        pool = torch.from_numpy(np.ascontiguousarray(w.kv_pool)).cuda()
        O, lse = _np(*mla.decode_e4m3(_t16(w.q_nope), _t16(w.q_rope), pool, w.kv_scale, bt, sl,
                                      float(w.scale), causal=w.causal, num_partitions=parts))
        ref = mla_attention_folded(w.q_nope, w.q_rope, E4M3Pool(w.kv_pool, w.kv_scale),
                                   w.block_table, w.seq_lens, w.scale, w.causal)
    elif kind == "tree":
        masks = make_tree_masks(w.B, w.Sq, "random", seed=seed2)
        O, lse = _np(*mla.decode_tree(_t16(w.q_nope), _t16(w.q_rope), _t16(w.kv_pool), bt, sl,
                                      torch.from_numpy(masks.view(np.int64)).cuda(),
                                      float(w.scale), num_partitions=parts))
        ref = mla_attention_tree(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                                 w.scale, masks)
    elif kind == "varlen":
        rng = np.random.default_rng(seed2)
        q_lens = np.array([int(rng.integers(1, min(w.Sq, int(L)) + 1)) for L in w.seq_lens],
                          dtype=np.int32)
        O, lse = _np(*mla.decode_varlen(_t16(w.q_nope), _t16(w.q_rope), _t16(w.kv_pool), bt, sl,
                                        torch.from_numpy(q_lens).cuda(), float(w.scale),
                                        num_partitions=parts))
        ref = mla_attention_varlen(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                                   w.scale, q_lens)
        real = np.arange(w.Sq)[None, :] < q_lens[:, None]
    else:
        fn = {"decode": mla.decode, "single": mla.decode_single_pass,
              "prefill": mla.prefill_with_prefix}[kind]
        O, lse = _np(*fn(_t16(w.q_nope), _t16(w.q_rope), _t16(w.kv_pool), bt, sl, float(w.scale),
                         causal=w.causal, num_partitions=parts))
        ref = mla_attention_folded(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                                   w.scale, w.causal)
    _check(O, lse, *ref, name, real)
