"""GPU parity of the E4M3 latent-pool entry points against the fp64 CPU oracle.

The pool holds OCP E4M3 codes with one per-tensor scale; the oracle reads it through
E4M3Pool (code value times scale, exact in fp64), so the only differences left are
the kernel's bf16 P, fp32 accumulation and exp2 — the same bar as the bf16 pool:
|dLSE| <= 1e-3, max |dO| <= 2e-2 * rms(O_ref), mean |dO| <= 2e-3 * rms(O_ref), and
the absolute 2e-2 / 2e-3 where rms(O_ref) <= 1.  Unused pages and rows past each
request's length hold the E4M3 NaN code, so any stray read shows up.
"""
import math
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import E4M3Pool, e4m3_bits_to_f64, mla_attention_folded, mla_attention_rows  # noqa: E402
import mla_latent_kv_16_amd as mla  # noqa: E402
from mla_latent_kv_16_amd.workloads import E4M3_NAN, PAGE, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_ABS = 2e-2, 2e-3, 1e-3


def say(*a):
    print("[gpu-e4m3]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(mla.LIB_PATH):
        pytest.fail("libmla.so is not built")
    torch.cuda.init()


def e4m3(name="tiny", **kw):
    return make_workload(name, kv_format="e4m3", **kw)


def to_dev(w):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return dict(q_nope=t(w.q_nope), q_rope=t(w.q_rope),
                kv_pool=torch.from_numpy(np.ascontiguousarray(w.kv_pool)).cuda(),
                block_table=torch.from_numpy(w.block_table).cuda(),
                seq_lens=torch.from_numpy(w.seq_lens).cuda())


def run(w, parts=0, fn=None, dev=None):
    dev = dev or to_dev(w)
    fn = fn or mla.decode_e4m3
    say(f"{fn.__name__} B={w.B} Sq={w.Sq} H={w.H} L={w.seq_lens.tolist()[:4]} parts={parts} "
        f"kv_scale={w.kv_scale}")
    O, lse = fn(dev["q_nope"], dev["q_rope"], dev["kv_pool"], w.kv_scale, dev["block_table"],
                dev["seq_lens"], float(w.scale), causal=w.causal, num_partitions=parts)
    torch.cuda.synchronize()
    return O.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle(w):
    return mla_attention_folded(w.q_nope, w.q_rope, E4M3Pool(w.kv_pool, w.kv_scale),
                                w.block_table, w.seq_lens, w.scale, w.causal)


def check(O, lse, O_ref, lse_ref, what=""):
    assert np.isfinite(O).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    d = np.abs(O - O_ref)
    rms = math.sqrt(float((O_ref ** 2).mean()))
    dl = float(np.abs(lse - lse_ref).max())
    say(f"{what}: max|dO|={d.max():.2e} mean|dO|={d.mean():.2e} rms(O)={rms:.3f} max|dLSE|={dl:.2e}")
    assert d.max() <= MAX_ABS * rms and d.mean() <= MEAN_ABS * rms, what
    if rms <= 1.0:
        assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, what
    assert dl <= LSE_ABS, what


def total_pages(w):
    return int(((w.seq_lens + PAGE - 1) // PAGE).sum())


# ------------------------------------------------------------------------------------
def test_tiny_config():
    w = e4m3()
    O, lse = run(w)
    check(O, lse, *oracle(w), "tiny")


SMALL = [
    ("spec4-short", dict(seed=201, B=3, Sq=4, H=16, lens=("uniform", 700, 3000))),
    ("spec8-short", dict(seed=202, B=2, Sq=8, H=16, lens=("uniform", 900, 2500))),
    ("spec16-short", dict(seed=203, B=2, Sq=16, H=16, lens=("uniform", 1000, 2200))),
    ("h128-short", dict(seed=204, B=3, Sq=1, H=128, lens=("uniform", 300, 1500))),
    ("odd-M", dict(seed=205, B=2, Sq=3, H=5, lens=("uniform", 130, 700))),
    ("ragged-mtile", dict(seed=206, B=2, Sq=5, H=20, lens=("uniform", 200, 900))),
    ("tail-shorter-than-drafts", dict(seed=207, B=2, Sq=6, H=16, lens=("fixed", 64 * 9 + 2))),
    ("one-page", dict(seed=208, B=3, Sq=2, H=16, lens=("fixed", 40))),
    ("half-page-tail", dict(seed=209, B=2, Sq=4, H=16, lens=("fixed", 64 * 5 + 32))),
    ("peaked-q4", dict(seed=210, B=2, Sq=4, H=16, lens=("uniform", 500, 1500), q_sigma=4.0)),
    ("wide-codes", dict(seed=211, B=2, Sq=4, H=16, lens=("uniform", 400, 1200), kv_sigma=4.0)),
    ("scale-not-pow2", dict(seed=212, B=2, Sq=4, H=16, lens=("uniform", 400, 1200),
                            kv_scale=0.0173)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_workloads(name, kw):
    w = e4m3(**kw)
    O, lse = run(w)
    check(O, lse, *oracle(w), name)


def test_non_causal():
    w = e4m3(seed=213, B=2, Sq=4, H=16, lens=("uniform", 300, 900), causal=False)
    O, lse = run(w)
    check(O, lse, *oracle(w), "non-causal")


def test_forced_partition_counts():
    """1 (no split), 2, 7 and one page (two 32-row blocks) per partition."""
    w = e4m3(seed=214, B=3, Sq=4, H=16, lens=("uniform", 400, 1300))
    ref = oracle(w)
    dev = to_dev(w)
    for parts in (1, 2, 7, total_pages(w)):
        O, lse = run(w, parts=parts, dev=dev)
        check(O, lse, *ref, f"parts={parts}")


def test_more_partitions_than_pages():
    w = e4m3(seed=215, B=2, Sq=2, H=16, lens=("uniform", 64, 200))
    O, lse = run(w, parts=total_pages(w) + 5)
    check(O, lse, *oracle(w), "parts>pages")


COMBINE_CASES = [
    ("pieces-per-group-long", dict(seed=221, B=1, Sq=4, H=16, lens=("fixed", 64 * 130)), 100),
    ("pieces-per-group-empty", dict(seed=222, B=1, Sq=4, H=16, lens=("fixed", 200)), 20),
    ("pieces-per-wave-empty", dict(seed=224, B=3, Sq=2, H=16, lens=("fixed", 150)), 40),
]


@pytest.mark.parametrize("name,kw,parts", COMBINE_CASES, ids=[c[0] for c in COMBINE_CASES])
def test_combine_paths(name, kw, parts):
    w = e4m3(**kw)
    O, lse = run(w, parts=parts)
    check(O, lse, *oracle(w), name)


def test_split_and_combine_entry_points_equal_decode():
    w = e4m3(seed=225, B=2, Sq=4, H=16, lens=("uniform", 600, 1200))
    dev = to_dev(w)
    O1, l1 = run(w, parts=9, dev=dev)
    ws = mla.new_workspace(w.B, w.Sq, w.H, w.max_pages, 9)
    O2, l2 = mla.decode_splitkv_e4m3(dev["q_nope"], dev["q_rope"], dev["kv_pool"], w.kv_scale,
                                     dev["block_table"], dev["seq_lens"], float(w.scale), True,
                                     9, workspace=ws)
    mla.decode_combine(dev["seq_lens"], w.max_pages, w.Sq, w.H, O2, l2, ws, 9)
    torch.cuda.synchronize()
    assert np.array_equal(O1, O2.cpu().numpy()) and np.array_equal(l1, l2.cpu().numpy())


def test_single_pass_equals_two_passes():
    w = e4m3(seed=233, B=1, Sq=4, H=16, lens=("uniform", 1500, 2500))
    dev = to_dev(w)
    for parts in (40, 7):  # a workgroup per merged row, and a wave per row
        O1, l1 = run(w, parts=parts, dev=dev)
        O2, l2 = run(w, parts=parts, dev=dev, fn=mla.decode_single_pass_e4m3)
        assert np.array_equal(O1, O2) and np.array_equal(l1, l2)
        check(O2, l2, *oracle(w), f"single-pass parts={parts}")


def test_bound_decode_matches():
    w = e4m3(seed=226, B=2, Sq=4, H=16, lens=("uniform", 600, 1200))
    dev = to_dev(w)
    O1, l1 = run(w, parts=5, dev=dev)
    bd = mla.BoundDecode(dev["q_nope"], dev["q_rope"], dev["kv_pool"], dev["block_table"],
                         dev["seq_lens"], float(w.scale), True, 5, kv_scale=w.kv_scale)
    bd()
    torch.cuda.synchronize()
    assert np.array_equal(O1, bd.out.cpu().numpy()) and np.array_equal(l1, bd.lse.cpu().numpy())


def test_prefill_shape():
    w = e4m3(seed=227, B=1, Sq=96, H=16, lens=("fixed", 64 * 20 + 96))
    O, lse = run(w)
    check(O, lse, *oracle(w), "prefill-small")


def test_deterministic_repeats():
    w = e4m3(seed=228, B=2, Sq=4, H=16, lens=("uniform", 700, 1400))
    dev = to_dev(w)
    a = run(w, dev=dev)
    b = run(w, dev=dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_block_table_permutation_invariance():
    w = e4m3(seed=229, B=2, Sq=4, H=16, lens=("uniform", 500, 1200))
    O1, l1 = run(w, parts=1)
    perm = np.random.default_rng(6).permutation(w.num_pages)
    pool2 = np.full_like(w.kv_pool, E4M3_NAN)
    pool2[perm] = w.kv_pool
    w.kv_pool = pool2
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)],
                             -1).astype(np.int32)
    O2, l2 = run(w, parts=1)
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2)


def test_single_row_is_exact():
    """L = Sq = 1 with a power-of-two scale: O is that row's dequantized latent exactly."""
    w = e4m3(seed=230, B=3, Sq=1, H=16, lens=("fixed", 1))
    O, lse = run(w)
    for b in range(3):
        exact = e4m3_bits_to_f64(w.kv_pool[w.block_table[b, 0], 0, :512]) * w.kv_scale
        assert np.array_equal(O[b, 0], np.broadcast_to(exact, (16, 512)))
    check(O, lse, *oracle(w), "single-row")


def test_uniform_scores():
    """q = 0: O is the mean of the visible dequantized rows."""
    w = e4m3(seed=231, B=2, Sq=4, H=16, lens=("uniform", 200, 700))
    w.q_nope = np.zeros_like(w.q_nope)
    w.q_rope = np.zeros_like(w.q_rope)
    O, lse = run(w)
    O_ref, l_ref = oracle(w)
    assert np.abs(O - O_ref).max() < 1e-5 and np.abs(lse - l_ref).max() < 1e-5


def test_rescale_path():
    """The re-walk case on an E4M3 pool (which takes every block's maximum from its
    first walk on, so a jump past 32 log2 units over the first block's reference
    sends the piece straight to the walk from the true maxima).  The pool scale is
    1/8 so that the x8 keys of the later pages stay exact E4M3 values (no
    saturation): their codes are re-made with the oracle's quantizer."""
    from oracle import e4m3_quantize, gather_latent_rows
    w = e4m3(seed=119, B=2, Sq=4, H=16, lens=("fixed", 64 * 12 + 5), q_sigma=4.0,
             kv_scale=0.125)
    codes = w.kv_pool.copy()
    for b in range(w.B):
        for p in range(6, 13):
            page = w.block_table[b, p]
            vals = e4m3_bits_to_f64(codes[page]) * 8.0  # in code units: exact, below 448
            nan = np.isnan(vals)
            new = e4m3_quantize(np.where(nan, 0.0, vals))
            new[nan] = E4M3_NAN
            assert np.array_equal(e4m3_bits_to_f64(new)[~nan], vals[~nan])
            codes[page] = new
    w.kv_pool = codes
    pool = E4M3Pool(w.kv_pool, w.kv_scale)
    q = np.concatenate([w.q_nope.view(np.uint16), w.q_rope.view(np.uint16)], axis=-1)
    jump = -np.inf
    for b in range(w.B):
        rows = gather_latent_rows(pool, w.block_table, b, int(w.seq_lens[b]) - w.Sq + 1)
        qb = (q[b].reshape(-1, q.shape[-1]).astype(np.uint32) << 16).view(np.float32)
        s = float(w.scale) * (qb.astype(np.float64) @ rows.T)
        jump = max(jump, float((s[:, 32:].max(1) - s[:, :32].max(1)).max()) / math.log(2.0))
    say(f"e4m3 rescale: largest score jump over the first block {jump:.1f} (log2 units)")
    assert jump > 64.0
    O_ref, l_ref = oracle(w)
    for parts in (1, 3):
        O, lse = run(w, parts=parts)
        check(O, lse, O_ref, l_ref, f"e4m3 rescale parts={parts}")


def test_error_flags_for_bad_pages():
    w = e4m3(seed=232, B=2, Sq=2, H=16, lens=("fixed", 300))
    dev = to_dev(w)
    ws = mla.new_workspace(w.B, w.Sq, w.H, w.max_pages, 2)
    args = (dev["q_nope"], dev["q_rope"], dev["kv_pool"], w.kv_scale)
    mla.decode_e4m3(*args, dev["block_table"], dev["seq_lens"], float(w.scale), True, 2,
                    workspace=ws)
    assert mla.read_error_flags(ws) == 0
    bad_bt = dev["block_table"].clone()
    bad_bt[0, 1] = w.num_pages + 3
    mla.decode_e4m3(*args, bad_bt, dev["seq_lens"], float(w.scale), True, 2, workspace=ws)
    assert mla.read_error_flags(ws) & 2


# ------------------------------------------------------------------------------------
# Full-size workloads in the benchmark's launch configuration, sampled rows.
FULL = ["spec4", "spec16", "prefill"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    w = e4m3(name)
    say(f"{name}: generated, {w.kv_bytes() / 1e9:.2f} GB of E4M3 latent rows")
    O, lse = run(w)
    rng = np.random.default_rng(8)
    M = w.Sq * w.H
    pool = E4M3Pool(w.kv_pool, w.kv_scale)
    bs = sorted(set([0, w.B - 1] + rng.integers(0, w.B, size=2).tolist()))
    for b in bs:
        ms = sorted(set([0, M - 1, M // 2] + rng.integers(0, M, size=6).tolist()))
        o_ref, l_ref = mla_attention_rows(w.q_nope, w.q_rope, pool, w.block_table, w.seq_lens,
                                          w.scale, w.causal, b, ms)
        check(O[b].reshape(M, 512)[ms], lse[b].reshape(M)[ms], o_ref, l_ref, f"{name} b={b}")
    assert np.isfinite(O).all() and np.isfinite(lse).all()
