"""GPU parity of the NoPE-MLA entry points (512-wide rows, no RoPE part) against the
oracle's mla_attention_nope.  Same bar as every other parity test: |dLSE| <= 1e-3,
max |dO| <= 2e-2 * rms(O_ref), mean |dO| <= 2e-3 * rms(O_ref), absolute where
rms <= 1.  Unused pages and rows past each length hold bf16 NaN."""
import math
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import bf16_bits_to_f64, mla_attention_nope  # noqa: E402
import mla_latent_kv_16_amd as mla  # noqa: E402
from mla_latent_kv_16_amd.workloads import BF16_NAN, PAGE, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_ABS = 2e-2, 2e-3, 1e-3


def say(*a):
    print("[gpu-nope]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(mla.LIB_PATH):
        pytest.fail("libmla.so is not built")
    torch.cuda.init()


def nope(name="tiny", **kw):
    return make_workload(name, rope=False, **kw)


def to_dev(w):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return dict(q_nope=t(w.q_nope), kv_pool=t(w.kv_pool),
                block_table=torch.from_numpy(w.block_table).cuda(),
                seq_lens=torch.from_numpy(w.seq_lens).cuda())


def run(w, parts=0, dev=None):
    dev = dev or to_dev(w)
    say(f"nope B={w.B} Sq={w.Sq} H={w.H} L={w.seq_lens.tolist()[:4]} parts={parts}")
    O, lse = mla.decode_nope(dev["q_nope"], dev["kv_pool"], dev["block_table"], dev["seq_lens"],
                             float(w.scale), causal=w.causal, num_partitions=parts)
    torch.cuda.synchronize()
    return O.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle(w):
    return mla_attention_nope(w.q_nope, w.kv_pool, w.block_table, w.seq_lens, w.scale, w.causal)


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


SMALL = [
    ("tiny", dict()),
    ("spec4-short", dict(seed=1001, B=3, Sq=4, H=16, lens=("uniform", 700, 3000))),
    ("spec16-short", dict(seed=1002, B=2, Sq=16, H=16, lens=("uniform", 1000, 2200))),
    ("h128-short", dict(seed=1003, B=3, Sq=1, H=128, lens=("uniform", 300, 1500))),
    ("odd-M", dict(seed=1004, B=2, Sq=3, H=5, lens=("uniform", 130, 700))),
    ("tail-shorter-than-drafts", dict(seed=1005, B=2, Sq=6, H=16, lens=("fixed", 64 * 9 + 2))),
    ("one-page", dict(seed=1006, B=3, Sq=2, H=16, lens=("fixed", 40))),
    ("half-page-tail", dict(seed=1007, B=2, Sq=4, H=16, lens=("fixed", 64 * 5 + 32))),
    ("peaked-q4", dict(seed=1008, B=2, Sq=4, H=16, lens=("uniform", 500, 1500), q_sigma=4.0)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_workloads(name, kw):
    w = nope(**kw)
    O, lse = run(w)
    check(O, lse, *oracle(w), name)


def test_non_causal():
    w = nope(seed=1009, B=2, Sq=4, H=16, lens=("uniform", 300, 900), causal=False)
    O, lse = run(w)
    check(O, lse, *oracle(w), "non-causal")


def test_forced_partition_counts():
    w = nope(seed=1010, B=3, Sq=4, H=16, lens=("uniform", 400, 1300))
    ref = oracle(w)
    dev = to_dev(w)
    for parts in (1, 2, 7, total_pages(w), total_pages(w) + 5):
        O, lse = run(w, parts=parts, dev=dev)
        check(O, lse, *ref, f"parts={parts}")


@pytest.mark.parametrize("kw,parts", [
    (dict(seed=1011, B=1, Sq=4, H=16, lens=("fixed", 64 * 130)), 100),
    (dict(seed=1012, B=3, Sq=2, H=16, lens=("fixed", 150)), 40),
], ids=["pieces-per-group", "pieces-per-wave-empty"])
def test_combine_paths(kw, parts):
    w = nope(**kw)
    O, lse = run(w, parts=parts)
    check(O, lse, *oracle(w), f"combine parts={parts}")


def test_split_and_combine_entry_points_equal_decode():
    w = nope(seed=1013, B=2, Sq=4, H=16, lens=("uniform", 600, 1200))
    dev = to_dev(w)
    O1, l1 = run(w, parts=9, dev=dev)
    bd = mla.BoundDecode(dev["q_nope"], None, dev["kv_pool"], dev["block_table"],
                         dev["seq_lens"], float(w.scale), True, 9, nope=True)
    bd.splitkv()
    bd.combine()
    torch.cuda.synchronize()
    assert np.array_equal(O1, bd.out.cpu().numpy()) and np.array_equal(l1, bd.lse.cpu().numpy())


def test_block_table_permutation_invariance():
    w = nope(seed=1014, B=2, Sq=4, H=16, lens=("uniform", 500, 1200))
    O1, l1 = run(w, parts=1)
    perm = np.random.default_rng(7).permutation(w.num_pages)
    pool2 = np.full_like(w.kv_pool, BF16_NAN)
    pool2[perm] = w.kv_pool
    w.kv_pool = pool2
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)],
                             -1).astype(np.int32)
    O2, l2 = run(w, parts=1)
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2)


def test_single_row_is_exact():
    w = nope(seed=1015, B=3, Sq=1, H=16, lens=("fixed", 1))
    O, lse = run(w)
    for b in range(3):
        exact = bf16_bits_to_f64(w.kv_pool[w.block_table[b, 0], 0])
        assert np.array_equal(O[b, 0], np.broadcast_to(exact, (16, 512)))


def test_prefill_shape():
    w = nope(seed=1016, B=1, Sq=96, H=16, lens=("fixed", 64 * 20 + 96))
    O, lse = run(w)
    check(O, lse, *oracle(w), "prefill-small")


@pytest.mark.parametrize("name", ["spec4", "spec16", "prefill"])
def test_full_size_sampled(name):
    w = nope(name)
    O, lse = run(w)
    rng = np.random.default_rng(9)
    M = w.Sq * w.H
    for b in sorted(set([0, w.B - 1] + rng.integers(0, w.B, size=2).tolist())):
        ms = sorted(set([0, M - 1, M // 2] + rng.integers(0, M, size=6).tolist()))
        o_ref, l_ref = mla_attention_nope(w.q_nope, w.kv_pool, w.block_table, w.seq_lens, w.scale,
                                          w.causal, (b, ms))
        check(O[b].reshape(M, 512)[ms], lse[b].reshape(M)[ms], o_ref, l_ref, f"{name} b={b}")
    assert np.isfinite(O).all() and np.isfinite(lse).all()
