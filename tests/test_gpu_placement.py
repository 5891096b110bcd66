"""Where the split-KV workgroups run.

The GPU hands workgroups to its eight XCDs round-robin, and each XCD has its own L2
(TokenSpeed review page, "Optimizing Attention on MI300X" entry: round-robin
dispatch collapses the L2 hit rate unless the workgroups that share data sit on one
XCD).  With several KV partitions the split pass renumbers its workgroups so that the
M-tiles of one partition, and neighbouring partitions, run on one XCD; with one
partition it runs them in launch order, longest first.  These tests read the XCC id
register of every split-KV workgroup through mla_decode_splitkv_placement and check
that placement on the device, plus that recording it changes no result.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mla_latent_kv_16_amd as mla  # noqa: E402
from mla_latent_kv_16_amd.workloads import make_workload  # noqa: E402

pytestmark = pytest.mark.gpu

XCDS = 8


def say(*a):
    print("[gpu-placement]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def dev_inputs(w):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return (t(w.q_nope), t(w.q_rope), t(w.kv_pool), torch.from_numpy(w.block_table).cuda(),
            torch.from_numpy(w.seq_lens).cuda())


def placement(w, parts):
    args = dev_inputs(w)
    say(f"placement B={w.B} Sq={w.Sq} H={w.H} parts={parts}")
    O = torch.zeros((w.B, w.Sq, w.H, 512), dtype=torch.float32, device="cuda")
    lse = torch.zeros((w.B, w.Sq, w.H), dtype=torch.float32, device="cuda")
    ws = mla.new_workspace(w.B, w.Sq, w.H, w.block_table.shape[1], parts)
    _, _, trace = mla.decode_splitkv_placement(*args, float(w.scale), causal=True,
                                               num_partitions=parts, out=O, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return args, O, lse, ws, trace.cpu().numpy()


# (name, workload keywords, partitions): M-tiles per partition 4, 1 and 2; the last
# has a workgroup count that is not a multiple of 8
CASES = [
    ("spec16-shape", dict(seed=701, B=4, Sq=16, H=16, lens=("uniform", 3000, 6000)), 64),
    ("spec4-shape", dict(seed=702, B=4, Sq=4, H=16, lens=("fixed", 64 * 300 + 4)), 256),
    ("uneven", dict(seed=703, B=3, Sq=8, H=16, lens=("uniform", 1500, 2500)), 37),
]


@pytest.mark.parametrize("name,kw,parts", CASES, ids=[c[0] for c in CASES])
def test_split_workgroups_share_an_xcd_per_partition(name, kw, parts):
    w = make_workload("tiny", **kw)
    n_mt = (w.Sq * w.H + 63) // 64
    _, _, _, _, tr = placement(w, parts)
    n = parts * n_mt
    assert tr.shape == (n, 3)
    xcc, g, mt = tr[:, 0], tr[:, 1], tr[:, 2]
    # every (partition, M-tile) ran exactly once, on a real XCD
    assert sorted(zip(g.tolist(), mt.tolist())) == [(a, b) for a in range(parts)
                                                    for b in range(n_mt)]
    assert ((xcc >= 0) & (xcc < XCDS)).all(), np.unique(xcc)
    # the hardware dispatch the numbering relies on: launch-order workgroups dealt to
    # the XCDs round-robin, w on XCD (w + o) % 8, where the offset o carries over from
    # earlier launches; workgroups with equal w % 8 share an XCD either way
    o = int(xcc[0])
    assert (xcc == (np.arange(n) + o) % XCDS).all(), "workgroups are not dealt round-robin"
    per_xcd = np.bincount(xcc, minlength=XCDS)
    assert per_xcd.max() - per_xcd.min() <= 1, per_xcd
    # each XCD runs one contiguous run of partitions; the runs follow the rotation
    # (the XCD of launch-order residue class r = w % 8 holds the r-th run)
    spans = []
    for r in range(XCDS):
        gs = np.unique(g[xcc == (r + o) % XCDS])
        assert (np.diff(gs) == 1).all(), (x, gs)
        spans.append((gs.min(), gs.max()))
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert b0 in (a1, a1 + 1), spans
    # the M-tiles of a partition share its XCD unless the partition straddles two
    # XCDs' runs (only where the per-XCD workgroup count is not a multiple of n_mt)
    split = [p for p in range(parts) if len(np.unique(xcc[g == p])) > 1]
    if (n // XCDS) % n_mt == 0 and n % XCDS == 0:
        assert not split, split
    assert len(split) <= XCDS - 1
    say(f"{name}: {n} workgroups, per XCD {per_xcd.tolist()}, partitions on two XCDs: {split}")


def test_one_partition_runs_in_launch_order_heaviest_first():
    """One partition (as in a prefill chunk): all M-tiles read the same pages, so
    workgroup w takes M-tile n - 1 - w; the causally longer last M-tiles start first
    and are dealt over all eight XCDs rather than packed onto one."""
    w = make_workload("tiny", seed=705, B=1, Sq=96, H=16, lens=("fixed", 64 * 40 + 96))
    n_mt = (w.Sq * w.H + 63) // 64
    _, _, _, _, tr = placement(w, 1)
    assert (tr[:, 1] == 0).all()
    assert (tr[:, 2] == n_mt - 1 - np.arange(n_mt)).all()
    assert (tr[:, 0] == (np.arange(n_mt) + tr[0, 0]) % XCDS).all()
    # the eight longest M-tiles (the last ones, with the most causal rows) start first,
    # one on each XCD
    assert len(np.unique(tr[tr[:, 2] >= n_mt - XCDS, 0])) == XCDS


def test_placement_record_changes_no_result():
    w = make_workload("tiny", seed=704, B=2, Sq=8, H=16, lens=("uniform", 2000, 3000))
    parts = 24
    args, O, lse, ws, _ = placement(w, parts)
    O2 = torch.zeros_like(O)
    lse2 = torch.zeros_like(lse)
    ws2 = mla.new_workspace(w.B, w.Sq, w.H, w.block_table.shape[1], parts)
    mla.decode_splitkv(*args, float(w.scale), causal=True, num_partitions=parts, out=O2,
                       lse=lse2, workspace=ws2)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(lse, lse2)
    assert torch.equal(ws, ws2)


def test_timeline_is_ordered_and_changes_no_result():
    """The timeline record: every workgroup with pages stamps start <= page prefix <=
    first block <= walk over <= stores complete, on one clock, within the launch; the
    placement part matches the placement record; results are bitwise those of the
    plain split pass."""
    w = make_workload("tiny", seed=706, B=4, Sq=4, H=16, lens=("uniform", 2000, 5000))
    parts = 64
    args = dev_inputs(w)
    say(f"timeline B={w.B} Sq={w.Sq} H={w.H} parts={parts}")
    O = torch.zeros((w.B, w.Sq, w.H, 512), dtype=torch.float32, device="cuda")
    lse = torch.zeros((w.B, w.Sq, w.H), dtype=torch.float32, device="cuda")
    ws = mla.new_workspace(w.B, w.Sq, w.H, w.block_table.shape[1], parts)
    _, _, trace, ticks = mla.decode_splitkv_timeline(*args, float(w.scale), causal=True,
                                                     num_partitions=parts, out=O, lse=lse,
                                                     workspace=ws)
    torch.cuda.synchronize()
    tr, tk = trace.cpu().numpy(), ticks.cpu().numpy()
    n = parts  # one M-tile
    assert tr.shape == (n, 3) and tk.shape == (n, 5)
    assert sorted(tr[:, 1].tolist()) == list(range(parts))
    assert ((tr[:, 0] >= 0) & (tr[:, 0] < XCDS)).all()
    assert (tk > 0).all(), "every partition holds pages here, so every stamp is written"
    assert (np.diff(tk, axis=1) >= 0).all(), "stamps out of order"
    span_us = (tk[:, 4].max() - tk[:, 0].min()) / 100.0
    assert 0 < span_us < 1e6, span_us
    O2 = torch.zeros_like(O)
    lse2 = torch.zeros_like(lse)
    ws2 = mla.new_workspace(w.B, w.Sq, w.H, w.block_table.shape[1], parts)
    mla.decode_splitkv(*args, float(w.scale), causal=True, num_partitions=parts, out=O2,
                       lse=lse2, workspace=ws2)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(lse, lse2)
    say(f"timeline: {n} workgroups over {span_us:.1f} us")
