"""Pins of the NoPE-MLA oracle (512-wide rows, no RoPE part)."""
import numpy as np

from oracle import bf16_bits_to_f64, mla_attention_folded, mla_attention_loop, mla_attention_nope
from mla_latent_kv_16_amd.workloads import make_workload


def test_nope_is_mla_with_zero_rope_parts():
    """Padding every row with a zero 64-wide k_rope and the queries with a zero q_rope
    reduces the pinned 576-wide oracle to NoPE."""
    w = make_workload("tiny", seed=901, B=3, Sq=4, H=3, lens=("uniform", 70, 220), rope=False)
    assert w.kv_pool.shape[2] == 512 and w.q_rope.shape[3] == 0
    pool576 = np.concatenate([w.kv_pool, np.zeros(w.kv_pool.shape[:2] + (64,), np.uint16)], axis=2)
    qr = np.zeros(w.q_nope.shape[:3] + (64,), np.uint16)
    for causal in (True, False):
        a = mla_attention_nope(w.q_nope, w.kv_pool, w.block_table, w.seq_lens, w.scale, causal)
        b = mla_attention_loop(w.q_nope, qr, pool576, w.block_table, w.seq_lens, w.scale, causal)
        assert np.allclose(a[0], b[0], atol=1e-12) and np.allclose(a[1], b[1], atol=1e-12)


def test_nope_single_row_returns_that_row():
    w = make_workload("tiny", seed=902, B=2, Sq=1, H=4, lens=("fixed", 1), rope=False)
    O, l = mla_attention_nope(w.q_nope, w.kv_pool, w.block_table, w.seq_lens, w.scale)
    for b in range(w.B):
        row = bf16_bits_to_f64(w.kv_pool[w.block_table[b, 0], 0])
        assert np.array_equal(O[b, 0], np.broadcast_to(row, (4, 512)))


def test_nope_sampled_rows_match_full():
    w = make_workload("tiny", seed=903, B=2, Sq=3, H=5, lens=("uniform", 100, 300), rope=False)
    O, l = mla_attention_nope(w.q_nope, w.kv_pool, w.block_table, w.seq_lens, w.scale)
    ms = [0, 7, 14]
    o, ll = mla_attention_nope(w.q_nope, w.kv_pool, w.block_table, w.seq_lens, w.scale, True,
                               (1, ms))
    assert np.allclose(o, O[1].reshape(15, 512)[ms], atol=1e-12)
    assert np.allclose(ll, l[1].reshape(15)[ms], atol=1e-12)


def test_rope_workloads_unchanged_by_the_option():
    a = make_workload("tiny", seed=904)
    b = make_workload("tiny", seed=904, rope=True)
    assert np.array_equal(a.kv_pool, b.kv_pool) and np.array_equal(a.q_rope, b.q_rope)
