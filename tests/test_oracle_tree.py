"""Pins of the tree-masked oracle (tree-shaped drafts, atlas §16 Speculative decoding).

Each pin checks the oracle against something other than itself: the causal chain,
independent single-query decodes over explicitly re-paged rows, the loop form
against the folded form, and the stated reading (high bits ignored, own row always
visible).
"""
import numpy as np
import pytest

from oracle import (mla_attention_folded, mla_attention_loop, mla_attention_tree,
                    mla_attention_tree_loop, mla_attention_tree_rows, tree_visible)
from mla_latent_kv_16_amd.workloads import PAGE, make_tree_masks, make_workload


def small(seed, B=2, Sq=6, H=3, lens=("uniform", 70, 200)):
    return make_workload("tiny", seed=seed, B=B, Sq=Sq, H=H, lens=lens)


def test_chain_tree_is_the_causal_chain():
    w = small(301)
    masks = make_tree_masks(w.B, w.Sq, "chain")
    O, l = mla_attention_tree(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens, w.scale,
                              masks)
    O2, l2 = mla_attention_folded(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                                  w.scale, True)
    assert np.allclose(O, O2, atol=1e-12) and np.allclose(l, l2, atol=1e-12)


def _rows_bits(w, b, idx):
    """bf16 bit patterns of logical rows idx of request b, read through the block table."""
    idx = np.asarray(idx)
    return w.kv_pool[w.block_table[b, idx // PAGE], idx % PAGE]


def _single_decode(w, b, t, idx):
    """Draft t of request b as an independent Sq = 1 decode over exactly the rows idx,
    re-paged contiguously into a fresh pool."""
    rows = _rows_bits(w, b, idx)
    n = len(idx)
    pages = (n + PAGE - 1) // PAGE
    pool = np.zeros((pages, PAGE, rows.shape[1]), dtype=rows.dtype)
    pool.reshape(-1, rows.shape[1])[:n] = rows
    bt = np.arange(pages, dtype=np.int32)[None, :]
    return mla_attention_loop(w.q_nope[b:b + 1, t:t + 1], w.q_rope[b:b + 1, t:t + 1], pool, bt,
                              np.array([n], dtype=np.int32), w.scale, True)


@pytest.mark.parametrize("kind,seed", [("star", 302), ("random", 303), ("random", 304)])
def test_tree_equals_independent_decodes_over_visible_rows(kind, seed):
    w = small(seed, B=2, Sq=7, H=2)
    masks = make_tree_masks(w.B, w.Sq, kind, seed=seed)
    O, l = mla_attention_tree(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens, w.scale,
                              masks)
    for b in range(w.B):
        L = int(w.seq_lens[b])
        for t in range(w.Sq):
            # the ancestors of t by walking the mask bits directly
            idx = list(range(L - w.Sq)) + [L - w.Sq + u for u in range(t + 1)
                                             if (int(masks[b, t]) >> u) & 1]
            o1, l1 = _single_decode(w, b, t, idx)
            assert np.allclose(O[b, t], o1[0, 0], atol=1e-12), (b, t)
            assert np.allclose(l[b, t], l1[0, 0], atol=1e-12), (b, t)


def test_star_tree_sees_prefix_and_itself_only():
    L, Sq = 100, 5
    for t in range(Sq):
        v = tree_visible(L, Sq, t, 0)
        assert list(v) == list(range(L - Sq)) + [L - Sq + t]


def test_loop_and_folded_tree_forms_agree():
    w = small(305, B=3, Sq=9, H=2)
    masks = make_tree_masks(w.B, w.Sq, "random", seed=9)
    a = mla_attention_tree(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens, w.scale,
                           masks)
    b = mla_attention_tree_loop(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                                w.scale, masks)
    assert np.allclose(a[0], b[0], atol=1e-12) and np.allclose(a[1], b[1], atol=1e-12)


def test_bits_above_t_are_ignored_and_own_row_is_always_seen():
    w = small(306, B=2, Sq=6, H=2)
    masks = make_tree_masks(w.B, w.Sq, "random", seed=3)
    noisy = masks.copy()
    for t in range(w.Sq):
        above = np.uint64(((1 << 64) - 1) ^ ((1 << (t + 1)) - 1))
        noisy[:, t] = (masks[:, t] | above) & ~np.uint64(1 << t)  # no own bit, all high bits
    a = mla_attention_tree(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens, w.scale,
                           masks)
    b = mla_attention_tree(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens, w.scale,
                           noisy)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_tree_mask_generator_structure():
    m = make_tree_masks(3, 64, "random", seed=1)
    for b in range(3):
        for t in range(64):
            v = int(m[b, t])
            assert (v >> t) & 1 and v >> (t + 1) == 0  # own bit, nothing above
            for u in range(t):  # ancestor sets are closed: an ancestor's ancestors
                if (v >> u) & 1:
                    assert int(m[b, u]) & ~v == 0
    assert (make_tree_masks(1, 5, "chain") == np.array([[1, 3, 7, 15, 31]], dtype=np.uint64)).all()
    assert (make_tree_masks(1, 4, "star") == np.array([[1, 2, 4, 8]], dtype=np.uint64)).all()


def test_tree_rows_form_matches_folded_form():
    w = small(307, B=2, Sq=8, H=3)
    masks = make_tree_masks(w.B, w.Sq, "random", seed=5)
    O, l = mla_attention_tree(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens, w.scale,
                              masks)
    ms = [0, 5, 11, 23]
    o, ll = mla_attention_tree_rows(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                                    w.scale, masks, 1, ms)
    assert np.allclose(o, O[1].reshape(-1, 512)[ms], atol=1e-12)
    assert np.allclose(ll, l[1].reshape(-1)[ms], atol=1e-12)
