"""The no-allocation decode (mla_decode_noalloc) through the C ABI.

Its workspace is a static device array of the library, shared by every call on a
GPU and keeping the previous call's contents; these tests call it twice in a row,
the second time with a smaller input, and compare each result with mla_decode (the
entry point it is a variant of) at the same partition count, bit for bit, and with
the fp64 oracle to the usual bar.
"""
import ctypes
import math
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import mla_attention_folded  # noqa: E402
import mla_latent_kv_16_amd as mla  # noqa: E402
from mla_latent_kv_16_amd.workloads import make_workload  # noqa: E402

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


def say(*a):
    print("[gpu-noalloc]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(mla.LIB_PATH):
        pytest.fail("libmla.so is not built")
    torch.cuda.init()


def to_dev(w):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return dict(q_nope=t(w.q_nope), q_rope=t(w.q_rope), kv_pool=t(w.kv_pool),
                block_table=torch.from_numpy(w.block_table).cuda(),
                seq_lens=torch.from_numpy(w.seq_lens).cuda())


def p(t):
    return ctypes.c_void_p(t.data_ptr())


def noalloc(w, d, parts):
    """mla_decode_noalloc through ctypes; returns (status, O, lse)."""
    O = torch.full((w.B, w.Sq, w.H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((w.B, w.Sq, w.H), float("nan"), dtype=torch.float32, device="cuda")
    st = mla.lib().mla_decode_noalloc(
        p(d["q_nope"]), p(d["q_rope"]), p(d["kv_pool"]), w.num_pages, 64, p(d["block_table"]),
        w.max_pages, p(d["seq_lens"]), w.B, w.Sq, w.H, float(w.scale), 1, parts, p(O), p(lse),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return st, O, lse


def check_oracle(O, lse, w, what):
    O_ref, l_ref = mla_attention_folded(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                                        w.scale, True)
    O = O.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(O).all() and np.isfinite(lse).all(), what
    d = np.abs(O - O_ref)
    rms = math.sqrt(float((O_ref ** 2).mean()))
    dl = float(np.abs(lse - l_ref).max())
    say(f"{what}: max|dO|={d.max():.2e} mean|dO|={d.mean():.2e} rms={rms:.3f} max|dLSE|={dl:.2e}")
    assert d.max() <= 2e-2 * rms and d.mean() <= 2e-3 * rms and dl <= 1e-3, what
    if rms <= 1.0:
        assert d.max() <= 2e-2 and d.mean() <= 2e-3, what


def test_two_calls_in_a_row_match_mla_decode():
    """A larger call, then a smaller one on the same static workspace: each equals
    mla_decode at the same (automatic) partition count bit for bit."""
    big = make_workload("tiny", seed=150, B=4, Sq=4, H=16, lens=("uniform", 2000, 4000))
    small = make_workload("tiny", seed=151, B=2, Sq=2, H=16, lens=("uniform", 300, 900))
    for w, what in ((big, "first call (B=4, Sq=4)"), (small, "second call (B=2, Sq=2)")):
        d = to_dev(w)
        G = mla.auto_partitions(w.B, w.Sq, w.H, w.max_pages)
        assert G > 1 and mla.workspace_size(w.B, w.Sq, w.H, w.max_pages, G) <= SCRATCH_BYTES
        say(f"{what}: G={G}")
        st, O, lse = noalloc(w, d, 0)
        assert st == 0, mla.status_string(st)
        O_ref, l_ref = mla.decode(d["q_nope"], d["q_rope"], d["kv_pool"], d["block_table"],
                                  d["seq_lens"], float(w.scale), True, G)
        torch.cuda.synchronize()
        assert torch.equal(O, O_ref) and torch.equal(lse, l_ref), what
        check_oracle(O, lse, w, what)


def test_explicit_partitions_over_the_limit_are_rejected():
    """An explicit partition count whose partial results exceed the 64 MiB array is
    refused before anything is enqueued; the same count works through mla_decode."""
    w = make_workload("tiny", seed=152, B=64, Sq=1, H=128, lens=("uniform", 64, 200))
    d = to_dev(w)
    G = 400  # (64 + 400) slots x 2 M-tiles x 64 rows x 2,052 bytes = 122 MB
    assert mla.workspace_size(w.B, w.Sq, w.H, w.max_pages, G) > SCRATCH_BYTES
    st, O, _ = noalloc(w, d, G)
    assert st == -3  # MLA_ERR_WORKSPACE
    assert torch.isnan(O).all()  # nothing ran


def test_automatic_count_shrinks_to_fit():
    """When the automatic count's partials would not fit, the call takes the largest
    count that does; the result still matches the oracle, and the next, smaller call
    on the same array matches mla_decode bit for bit."""
    w = make_workload("tiny", seed=153, B=128, Sq=1, H=128, lens=("uniform", 64, 300))
    G_auto = mla.auto_partitions(w.B, w.Sq, w.H, w.max_pages)
    assert mla.workspace_size(w.B, w.Sq, w.H, w.max_pages, G_auto) > SCRATCH_BYTES
    d = to_dev(w)
    st, O, lse = noalloc(w, d, 0)
    assert st == 0, mla.status_string(st)
    check_oracle(O, lse, w, f"B=128 H=128 (automatic count {G_auto} shrunk to fit)")
    small = make_workload("tiny", seed=154, B=3, Sq=4, H=16, lens=("uniform", 500, 1500))
    ds = to_dev(small)
    st, O, lse = noalloc(small, ds, 0)
    assert st == 0
    G = mla.auto_partitions(small.B, small.Sq, small.H, small.max_pages)
    O_ref, l_ref = mla.decode(ds["q_nope"], ds["q_rope"], ds["kv_pool"], ds["block_table"],
                              ds["seq_lens"], float(small.scale), True, G)
    torch.cuda.synchronize()
    assert torch.equal(O, O_ref) and torch.equal(lse, l_ref)
