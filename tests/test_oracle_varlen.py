"""Pins of the per-request draft-count oracle (mla_attention_varlen)."""
import numpy as np

from oracle import mla_attention_loop, mla_attention_varlen
from mla_latent_kv_16_amd.workloads import make_workload


def test_varlen_equals_each_request_alone_with_its_own_draft_count():
    """Request b with q_lens[b] drafts is the same as the causal loop oracle on that
    request alone with Sq = q_lens[b] (its queries being the first q_lens[b] slots)."""
    w = make_workload("tiny", seed=501, B=4, Sq=6, H=3, lens=("uniform", 80, 200))
    q_lens = np.array([6, 1, 3, 4], dtype=np.int32)
    O, l = mla_attention_varlen(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens, w.scale,
                                q_lens)
    for b in range(w.B):
        n = int(q_lens[b])
        o1, l1 = mla_attention_loop(w.q_nope[b:b + 1, :n], w.q_rope[b:b + 1, :n], w.kv_pool,
                                    w.block_table[b:b + 1], w.seq_lens[b:b + 1], w.scale, True)
        assert np.allclose(O[b, :n], o1[0], atol=1e-12) and np.allclose(l[b, :n], l1[0], atol=1e-12)
        assert (O[b, n:] == 0).all() and np.isneginf(l[b, n:]).all()


def test_full_draft_counts_are_the_fixed_count_decode():
    from oracle import mla_attention_folded
    w = make_workload("tiny", seed=502, B=3, Sq=5, H=2, lens=("uniform", 60, 150))
    q_lens = np.full(w.B, w.Sq, dtype=np.int32)
    a = mla_attention_varlen(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens, w.scale,
                             q_lens)
    b = mla_attention_folded(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens, w.scale,
                             True)
    assert np.allclose(a[0], b[0], atol=1e-12) and np.allclose(a[1], b[1], atol=1e-12)


def test_one_draft_is_plain_decode_over_the_whole_context():
    """q_lens[b] = 1: the single query sees all L_b rows (Sq = 1 is full attention)."""
    w = make_workload("tiny", seed=503, B=2, Sq=4, H=2, lens=("uniform", 60, 150))
    q_lens = np.ones(w.B, dtype=np.int32)
    O, l = mla_attention_varlen(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens, w.scale,
                                q_lens)
    o1, l1 = mla_attention_loop(w.q_nope[:, :1], w.q_rope[:, :1], w.kv_pool, w.block_table,
                                w.seq_lens, w.scale, False)
    assert np.allclose(O[:, 0], o1[:, 0], atol=1e-12) and np.allclose(l[:, 0], l1[:, 0], atol=1e-12)
