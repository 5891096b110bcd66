"""GPU parity of the draft-tree entry points (mla_decode_tree[_e4m3]) against the fp64
oracle's tree form, and against the causal decode for a chain.  Same bar as every
other parity test: |dLSE| <= 1e-3, max |dO| <= 2e-2 * rms(O_ref) and mean |dO| <=
2e-3 * rms(O_ref) (absolute where rms <= 1)."""
import math
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import E4M3Pool, mla_attention_tree, mla_attention_tree_rows  # noqa: E402
import mla_latent_kv_16_amd as mla  # noqa: E402
from mla_latent_kv_16_amd.workloads import make_tree_masks, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_ABS = 2e-2, 2e-3, 1e-3


def say(*a):
    print("[gpu-tree]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(mla.LIB_PATH):
        pytest.fail("libmla.so is not built")
    torch.cuda.init()


def to_dev(w, masks):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    pool = (torch.from_numpy(np.ascontiguousarray(w.kv_pool)).cuda() if w.kv_format == "e4m3"
            else t(w.kv_pool))
    return dict(q_nope=t(w.q_nope), q_rope=t(w.q_rope), kv_pool=pool,
                block_table=torch.from_numpy(w.block_table).cuda(),
                seq_lens=torch.from_numpy(w.seq_lens).cuda(),
                tree=torch.from_numpy(masks.view(np.int64)).cuda())


def run_tree(w, masks, parts=0, dev=None):
    dev = dev or to_dev(w, masks)
    say(f"tree {w.kv_format} B={w.B} Sq={w.Sq} H={w.H} L={w.seq_lens.tolist()[:4]} parts={parts}")
    kvs = w.kv_scale if w.kv_format == "e4m3" else None
    O, lse = mla.decode_tree(dev["q_nope"], dev["q_rope"], dev["kv_pool"], dev["block_table"],
                             dev["seq_lens"], dev["tree"], float(w.scale), num_partitions=parts,
                             kv_scale=kvs)
    torch.cuda.synchronize()
    return O.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def pool_of(w):
    return E4M3Pool(w.kv_pool, w.kv_scale) if w.kv_format == "e4m3" else w.kv_pool


def oracle(w, masks):
    return mla_attention_tree(w.q_nope, w.q_rope, pool_of(w), w.block_table, w.seq_lens, w.scale,
                              masks)


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


@pytest.mark.parametrize("Sq,H,parts", [(4, 16, 0), (16, 16, 7), (5, 20, 1)])
def test_chain_tree_is_the_causal_decode_bit_for_bit(Sq, H, parts):
    w = make_workload("tiny", seed=400 + Sq, B=3, Sq=Sq, H=H, lens=("uniform", 300, 1400))
    masks = make_tree_masks(w.B, w.Sq, "chain")
    dev = to_dev(w, masks)
    O1, l1 = run_tree(w, masks, parts, dev)
    O2, l2 = mla.decode(dev["q_nope"], dev["q_rope"], dev["kv_pool"], dev["block_table"],
                        dev["seq_lens"], float(w.scale), True, parts)
    torch.cuda.synchronize()
    assert np.array_equal(O1, O2.cpu().numpy()) and np.array_equal(l1, l2.cpu().numpy())


TREES = [
    # (name, workload kwargs, tree kind, partitions): draft rows straddling 32-row
    # blocks and pages, several M-tiles, odd head counts, split and unsplit
    ("random-spec8", dict(seed=410, B=3, Sq=8, H=16, lens=("uniform", 500, 1500)), "random", 0),
    ("random-spec16-split", dict(seed=411, B=2, Sq=16, H=16, lens=("uniform", 900, 2000)),
     "random", 9),
    ("star-spec4", dict(seed=412, B=3, Sq=4, H=16, lens=("uniform", 200, 800)), "star", 0),
    ("random-64-drafts", dict(seed=413, B=2, Sq=64, H=2, lens=("uniform", 300, 700)), "random", 3),
    ("random-odd", dict(seed=414, B=2, Sq=37, H=3, lens=("uniform", 100, 400)), "random", 0),
    ("drafts-cross-page", dict(seed=415, B=2, Sq=20, H=16, lens=("fixed", 64 * 7 + 10)), "random", 2),
    ("drafts-only", dict(seed=416, B=2, Sq=12, H=16, lens=("fixed", 12)), "random", 0),
    # three one-page partitions, the last holding the 64 drafts alone: under a star tree
    # drafts 32..63 see nothing in that piece's first block, so their exp2 reference is
    # set by its second block, while drafts 0..31 already have theirs
    ("star-drafts-own-partition", dict(seed=417, B=1, Sq=64, H=2, lens=("fixed", 64 * 3)),
     "star", 3),
]


@pytest.mark.parametrize("name,kw,kind,parts", TREES, ids=[t[0] for t in TREES])
def test_tree_matches_oracle(name, kw, kind, parts):
    w = make_workload("tiny", **kw)
    masks = make_tree_masks(w.B, w.Sq, kind, seed=kw["seed"])
    O, lse = run_tree(w, masks, parts)
    check(O, lse, *oracle(w, masks), name)


def test_tree_e4m3_matches_oracle():
    w = make_workload("tiny", seed=420, B=3, Sq=8, H=16, lens=("uniform", 500, 1500),
                      kv_format="e4m3")
    masks = make_tree_masks(w.B, w.Sq, "random", seed=420)
    O, lse = run_tree(w, masks, 5)
    check(O, lse, *oracle(w, masks), "e4m3 random tree")


def test_tree_full_size_spec16_sampled():
    """spec16's shape (B=16, Sq=16 drafts, H=16, 51K-205K contexts) with random trees,
    automatic partitions, rows sampled against the oracle."""
    w = make_workload("spec16")
    masks = make_tree_masks(w.B, w.Sq, "random", seed=16)
    O, lse = run_tree(w, masks)
    rng = np.random.default_rng(11)
    M = w.Sq * w.H
    for b in sorted(set([0, w.B - 1] + rng.integers(0, w.B, size=2).tolist())):
        ms = sorted(set([0, M - 1, M // 2] + rng.integers(0, M, size=6).tolist()))
        o_ref, l_ref = mla_attention_tree_rows(w.q_nope, w.q_rope, w.kv_pool, w.block_table,
                                               w.seq_lens, w.scale, masks, b, ms)
        check(O[b].reshape(M, 512)[ms], lse[b].reshape(M)[ms], o_ref, l_ref, f"spec16 tree b={b}")
