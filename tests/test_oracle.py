"""Pins for the fp64 oracle: each test checks it against something other than itself.

None of these tests needs a GPU.  Together they are chosen so that a plausible
mistake in the oracle (a dropped RoPE term, a wrong sign, an off-by-one causal
mask, a transposed operand, a wrong page index, a base-2 LSE) fails one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (
    bf16_bits_to_f64,
    gather_latent_rows,
    lse_merge,
    mla_attention_folded,
    mla_attention_loop,
    mla_attention_pages,
    mla_attention_rows,
)
from mla_latent_kv_16_amd.workloads import (
    BF16_NAN, D_C, D_R, D_ROW, PAGE, WORKLOADS, f32_to_bf16_bits, make_workload)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small(seed=11, B=2, Sq=3, H=4, lens=("uniform", 70, 300), **kw):
    return make_workload("tiny", seed=seed, B=B, Sq=Sq, H=H, lens=lens, **kw)


def run_loop(w, causal=None, scale=None):
    return mla_attention_loop(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                              w.scale if scale is None else scale,
                              w.causal if causal is None else causal)


def run_folded(w, causal=None, **kw):
    return mla_attention_folded(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                                w.scale, w.causal if causal is None else causal, **kw)


# --------------------------------------------------------------------------------------
# bf16 widening: exact on known bit patterns (IEEE binary32 top halves).
def test_bf16_widening_known_values():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x3F00, 0x0000, 0x8000, 0x7F80, 0x0001],
                    dtype=np.uint16)
    v = bf16_bits_to_f64(bits)
    assert v[:7].tolist() == [1.0, -1.0, 2.0, 0.5, 0.0, -0.0, math.inf]
    assert v[7] == 2.0 ** -133  # smallest bf16 subnormal
    assert np.isnan(bf16_bits_to_f64(np.array([BF16_NAN], dtype=np.uint16)))[0]


# --------------------------------------------------------------------------------------
# Hand-derived closed form (tests/golden/closed_form_pow2.json).
def _golden_inputs(fx):
    B, Sq, H = fx["B"], fx["Sq"], fx["H"]
    pool = np.full((fx["pool_pages"], PAGE, D_ROW), BF16_NAN, dtype=np.uint16)
    bt = np.array(fx["block_table"], dtype=np.int32)
    for j, row in enumerate(fx["rows"]):
        vals = np.zeros(D_ROW, dtype=np.float32)
        for k, v in row["c"].items():
            vals[int(k)] = v
        for k, v in row["r"].items():
            vals[D_C + int(k)] = v
        pool[bt[0, j // PAGE], j % PAGE] = f32_to_bf16_bits(vals)
    qn = np.zeros((B, Sq, H, D_C), dtype=np.float32)
    qr = np.zeros((B, Sq, H, D_R), dtype=np.float32)
    for q in fx["queries"]:
        for k, v in q["q_nope"].items():
            qn[0, q["t"], q["h"], int(k)] = v
        for k, v in q["q_rope"].items():
            qr[0, q["t"], q["h"], int(k)] = v
    assert fx["scale"] == "ln2"
    return (f32_to_bf16_bits(qn), f32_to_bf16_bits(qr), pool, bt,
            np.array(fx["seq_lens"], dtype=np.int32), math.log(2.0))


def _expect(e):
    O = np.zeros(D_C)
    for k, (num, den) in e["O"].items():
        O[int(k)] = num / den
    num, den = e["lse_ln_of"]
    return O, math.log(num / den)


@pytest.mark.parametrize("form", ["loop", "folded"])
def test_golden_closed_form(form):
    with open(os.path.join(GOLDEN, "closed_form_pow2.json")) as f:
        fx = json.load(f)
    qn, qr, pool, bt, lens, scale = _golden_inputs(fx)
    fn = mla_attention_loop if form == "loop" else mla_attention_folded
    O, LSE = fn(qn, qr, pool, bt, lens, scale, True)
    for e in fx["expected_causal"]:
        o_ref, lse_ref = _expect(e)
        np.testing.assert_allclose(O[0, e["t"], e["h"]], o_ref, atol=1e-14, rtol=0)
        assert abs(LSE[0, e["t"], e["h"]] - lse_ref) < 1e-14
    O, LSE = fn(qn, qr, pool, bt, lens, scale, False)
    o_ref, lse_ref = _expect(fx["expected_noncausal_t0h0"])
    np.testing.assert_allclose(O[0, 0, 0], o_ref, atol=1e-14, rtol=0)
    assert abs(LSE[0, 0, 0] - lse_ref) < 1e-14


# --------------------------------------------------------------------------------------
# Brute force: materialise per-head keys and values with W_UK / W_UV and run plain
# multi-head attention; the absorbed oracle must agree (review page, Attack 1:
# "absorb + project").
@pytest.mark.parametrize("seed,B,Sq,H", [(3, 1, 1, 2), (4, 2, 3, 4), (5, 1, 4, 3)])
def test_bruteforce_unabsorbed(seed, B, Sq, H):
    D_NOPE_HEAD, D_V_HEAD = 128, 128
    w = small(seed=seed, B=B, Sq=Sq, H=H, lens=("uniform", 40, 300))
    rng = np.random.default_rng(1000 + seed)
    W_UK = rng.standard_normal((H, D_NOPE_HEAD, D_C)) / math.sqrt(D_C)
    W_UV = rng.standard_normal((H, D_V_HEAD, D_C)) / math.sqrt(D_C)
    q_u = rng.standard_normal((B, Sq, H, D_NOPE_HEAD))
    q_r = bf16_bits_to_f64(w.q_rope)
    # absorbed query in fp64: q_nope = W_UK[h]^T q_u
    q_abs = np.einsum("hkc,bthk->bthc", W_UK, q_u)
    scale = 192.0 ** -0.5
    O, LSE = mla_attention_loop(q_abs, q_r, w.kv_pool, w.block_table, w.seq_lens, scale, True)

    for b in range(B):
        L = int(w.seq_lens[b])
        # brute force reads rows through its own page walk
        c = np.zeros((L, D_C))
        r = np.zeros((L, D_R))
        for j in range(L):
            page = int(w.block_table[b, j // PAGE])
            row = bf16_bits_to_f64(w.kv_pool[page, j % PAGE])
            c[j], r[j] = row[:D_C], row[D_C:]
        for h in range(H):
            k_nope = c @ W_UK[h].T          # [L, 128] per-head keys
            v = c @ W_UV[h].T               # [L, 128] per-head values
            keys = np.concatenate([k_nope, r], axis=1)
            for t in range(Sq):
                n = L - Sq + t + 1
                q = np.concatenate([q_u[b, t, h], q_r[b, t, h]])
                logits = scale * (keys[:n] @ q)
                wts = np.exp(logits - logits.max())
                lse_u = logits.max() + math.log(wts.sum())
                o_u = (wts / wts.sum()) @ v[:n]
                assert abs(LSE[b, t, h] - lse_u) <= 1e-10 * max(1.0, abs(lse_u))
                np.testing.assert_allclose(W_UV[h] @ O[b, t, h], o_u, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------------------
# Fold identity: the folded product with the mask taken from m // H equals the per
# (t, h) loop (launch news, decode-kernel paragraph: the fold is a layout choice).
@pytest.mark.parametrize("causal", [True, False])
def test_fold_identity(causal):
    w = small(seed=21, B=3, Sq=4, H=5, lens=("uniform", 5, 260))
    O1, L1 = run_loop(w, causal=causal)
    O2, L2 = run_folded(w, causal=causal, row_chunk=7)
    np.testing.assert_allclose(O2, O1, atol=1e-12, rtol=0)
    np.testing.assert_allclose(L2, L1, atol=1e-12, rtol=0)


def test_sampled_rows_match_full():
    w = small(seed=22, B=2, Sq=3, H=4)
    O, LSE = run_folded(w)
    for b in range(2):
        ms = [0, 5, 11]
        o, l = mla_attention_rows(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                                  w.scale, True, b, ms)
        np.testing.assert_allclose(o, O[b].reshape(-1, D_C)[ms], atol=1e-13, rtol=0)
        np.testing.assert_allclose(l, LSE[b].reshape(-1)[ms], atol=1e-13, rtol=0)


# --------------------------------------------------------------------------------------
# Normalisation: a c_kv column that is the same constant in every row shifts every
# score by the same amount, so the softmax weights (which sum to one) reproduce that
# constant exactly in O, and LSE moves by exactly scale * q[col] * constant.
def test_constant_column_normalisation():
    w = small(seed=31, B=2, Sq=2, H=3)
    base_O, base_L = run_loop(w)
    col, const = 7, 0.75
    pool = w.kv_pool.copy()
    for b in range(w.B):
        L = int(w.seq_lens[b])
        for j in range(L):
            pool[w.block_table[b, j // PAGE], j % PAGE, col] = f32_to_bf16_bits(
                np.array([const], np.float32))[0]
    base_pool = w.kv_pool.copy()
    for b in range(w.B):
        for j in range(int(w.seq_lens[b])):
            base_pool[w.block_table[b, j // PAGE], j % PAGE, col] = 0
    O0, L0 = mla_attention_loop(w.q_nope, w.q_rope, base_pool, w.block_table, w.seq_lens,
                                w.scale, True)
    O1, L1 = mla_attention_loop(w.q_nope, w.q_rope, pool, w.block_table, w.seq_lens,
                                w.scale, True)
    np.testing.assert_allclose(O1[..., col], const, atol=1e-13, rtol=0)
    other = [c for c in range(D_C) if c != col]
    np.testing.assert_allclose(O1[..., other], O0[..., other], atol=1e-13, rtol=0)
    shift = float(w.scale) * bf16_bits_to_f64(w.q_nope[..., col]) * const
    np.testing.assert_allclose(L1 - L0, shift, atol=1e-12, rtol=0)
    assert np.isfinite(base_O).all() and np.isfinite(base_L).all()


# --------------------------------------------------------------------------------------
# Single visible row: the output is that row's c_kv exactly and LSE is its score.
def test_single_row_context():
    w = make_workload("tiny", seed=41, B=3, Sq=1, H=4, lens=("fixed", 1))
    O, LSE = run_loop(w)
    for b in range(3):
        row = bf16_bits_to_f64(w.kv_pool[w.block_table[b, 0], 0])
        for h in range(4):
            assert np.array_equal(O[b, 0, h], row[:D_C])
            q = np.concatenate([bf16_bits_to_f64(w.q_nope[b, 0, h]),
                                bf16_bits_to_f64(w.q_rope[b, 0, h])])
            assert abs(LSE[b, 0, h] - float(w.scale) * float(q @ row)) < 1e-12


# Uniform logits (q = 0): O is the plain mean of the visible c_kv rows, LSE = ln n_vis.
def test_uniform_logits():
    w = small(seed=42, B=2, Sq=4, H=2, lens=("uniform", 64, 200))
    qn = np.zeros_like(w.q_nope)
    qr = np.zeros_like(w.q_rope)
    O, LSE = mla_attention_loop(qn, qr, w.kv_pool, w.block_table, w.seq_lens, w.scale, True)
    for b in range(2):
        L = int(w.seq_lens[b])
        for t in range(4):
            n = L - 4 + t + 1
            rows = np.stack([bf16_bits_to_f64(w.kv_pool[w.block_table[b, j // PAGE], j % PAGE])
                             for j in range(n)])
            for h in range(2):
                np.testing.assert_allclose(O[b, t, h], rows[:, :D_C].mean(axis=0), atol=1e-13, rtol=0)
                assert abs(LSE[b, t, h] - math.log(n)) < 1e-13


# --------------------------------------------------------------------------------------
# Causal mask: an Sq-token verify equals Sq separate one-token decodes, draft t with
# seq_len L - Sq + t + 1 (atlas §16: drafts verified in parallel, visible causally).
def test_causal_equals_sequential_decodes():
    w = small(seed=51, B=2, Sq=5, H=3, lens=("uniform", 66, 250))
    O, LSE = run_loop(w)
    for t in range(5):
        lens = w.seq_lens - 5 + t + 1
        o1, l1 = mla_attention_loop(w.q_nope[:, t:t + 1], w.q_rope[:, t:t + 1], w.kv_pool,
                                    w.block_table, lens.astype(np.int32), w.scale, True)
        np.testing.assert_allclose(O[:, t], o1[:, 0], atol=1e-12, rtol=0)
        np.testing.assert_allclose(LSE[:, t], l1[:, 0], atol=1e-12, rtol=0)


def test_sq1_causal_is_full_attention():
    w = small(seed=52, B=2, Sq=1, H=3)
    O1, L1 = run_loop(w, causal=True)
    O2, L2 = run_loop(w, causal=False)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


# --------------------------------------------------------------------------------------
# Paging: moving pages to other physical slots (and updating the block table) does
# not change the result (atlas §07: logical blocks on scattered physical pages).
def test_block_table_permutation_invariance():
    w = small(seed=61, B=3, Sq=2, H=3, lens=("uniform", 100, 400))
    O1, L1 = run_loop(w)
    rng = np.random.default_rng(7)
    perm = rng.permutation(w.num_pages)      # new slot of old page p is perm[p]
    pool2 = np.full_like(w.kv_pool, BF16_NAN)
    pool2[perm] = w.kv_pool
    bt2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    O2, L2 = mla_attention_loop(w.q_nope, w.q_rope, pool2, bt2, w.seq_lens, w.scale, True)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


# Contiguous pages: the result equals dense attention from torch's
# scaled_dot_product_attention (CPU, fp64, math path), one shared K/V head broadcast
# to every query head, value width 512, boolean bottom-right causal mask.
@pytest.mark.parametrize("causal", [True, False])
def test_dense_sdpa_special_case(causal):
    Sq, H, L = 3, 4, 190
    w = make_workload("tiny", seed=71, B=1, Sq=Sq, H=H, lens=("fixed", L), poison=True)
    O, _ = run_loop(w, causal=causal)
    rows = gather_latent_rows(w.kv_pool, w.block_table, 0, L)
    q = np.concatenate([bf16_bits_to_f64(w.q_nope[0]), bf16_bits_to_f64(w.q_rope[0])], -1)
    qt = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)            # [1, H, Sq, 576]
    kt = torch.from_numpy(rows).expand(1, H, L, D_ROW)
    vt = torch.from_numpy(rows[:, :D_C]).expand(1, H, L, D_C)
    if causal:
        t = torch.arange(Sq)[:, None]
        j = torch.arange(L)[None, :]
        mask = j <= (L - Sq + t)
    else:
        mask = None
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, scale=float(w.scale))
    np.testing.assert_allclose(O[0], ref[0].permute(1, 0, 2).numpy(), atol=1e-10, rtol=1e-10)


# --------------------------------------------------------------------------------------
# Split + combine: for every contiguous partition of a request's pages, merging the
# per-range partials by log-sum-exp gives the unsplit result (§7.1 of "Faster kernels,
# slower engine": partial results materialised, then reduced in a second pass).
def test_split_merge_all_partitions():
    L = 7 * PAGE + 13     # 8 pages, ragged tail
    w = make_workload("tiny", seed=81, B=1, Sq=3, H=2, lens=("fixed", L))
    O, LSE = run_loop(w)
    n_pages = 8
    count = 0
    for mask in range(1 << (n_pages - 1)):
        cuts = [0] + [i + 1 for i in range(n_pages - 1) if mask >> i & 1] + [n_pages]
        parts = [mla_attention_pages(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                                     w.scale, True, 0, lo, hi)
                 for lo, hi in zip(cuts[:-1], cuts[1:])]
        Om, Lm = lse_merge(parts)
        np.testing.assert_allclose(Om, O[0], atol=1e-12, rtol=0)
        np.testing.assert_allclose(Lm, LSE[0], atol=1e-12, rtol=0)
        count += 1
    assert count == 128


def test_merge_with_empty_part():
    """A split whose rows are all masked for some draft has LSE -inf and no weight."""
    L = 2 * PAGE + 1      # last page holds one row, visible only to the last draft
    w = make_workload("tiny", seed=82, B=1, Sq=4, H=2, lens=("fixed", L))
    O, LSE = run_loop(w)
    p_last = mla_attention_pages(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                                 w.scale, True, 0, 2, 3)
    assert np.isneginf(p_last[1][:3]).all() and np.isfinite(p_last[1][3]).all()
    p_head = mla_attention_pages(w.q_nope, w.q_rope, w.kv_pool, w.block_table, w.seq_lens,
                                 w.scale, True, 0, 0, 2)
    Om, Lm = lse_merge([p_head, p_last])
    np.testing.assert_allclose(Om, O[0], atol=1e-12, rtol=0)
    np.testing.assert_allclose(Lm, LSE[0], atol=1e-12, rtol=0)


# --------------------------------------------------------------------------------------
# Large-L statistics: with N(0,1) latent rows the scores of a query are Gaussian with
# variance sigma^2 = scale^2 |q|^2, so LSE ~ ln n + sigma^2 / 2 and the exponentially
# tilted mean of c_kv is scale * q_nope.  Sanity only (tolerance ~ several / sqrt(ESS)).
def test_large_context_statistics():
    L = 32768
    w = make_workload("tiny", seed=91, B=1, Sq=1, H=2, lens=("fixed", L))
    O, LSE = run_folded(w)
    for h in range(2):
        qn = bf16_bits_to_f64(w.q_nope[0, 0, h])
        qr = bf16_bits_to_f64(w.q_rope[0, 0, h])
        sc = float(w.scale)
        var = sc * sc * (qn @ qn + qr @ qr)
        ess = L * math.exp(-var)
        assert abs(LSE[0, 0, h] - (math.log(L) + var / 2)) < 6 * math.sqrt(math.exp(var) / L)
        assert np.abs(O[0, 0, h] - sc * qn).max() < 6 / math.sqrt(ess)


# --------------------------------------------------------------------------------------
# Generator sanity (the oracle consumes these inputs; poison must sit where promised).
def test_workload_layout_and_poison():
    w = make_workload("tiny")
    assert w.q_nope.shape == (1, 1, 16, 512) and w.kv_pool.shape == (8, 64, 576)
    assert sorted(w.block_table[0].tolist()) == sorted(set(w.block_table[0].tolist()))
    used = set(w.block_table[0].tolist())
    for p in range(8):
        if p not in used:
            assert (w.kv_pool[p] == BF16_NAN).all()
        else:
            assert not (w.kv_pool[p] == BF16_NAN).any()
    w2 = make_workload("tiny", seed=3, B=2, Sq=2, H=2, lens=("fixed", 70))
    for b in range(2):
        assert (w2.kv_pool[w2.block_table[b, 1], 6:] == BF16_NAN).all()
        assert not (w2.kv_pool[w2.block_table[b, 1], :6] == BF16_NAN).any()
    assert WORKLOADS["spec4"].lens == ("fixed", 65540)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5], dtype=np.float32)
    v = bf16_bits_to_f64(f32_to_bf16_bits(x))
    assert v.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5]
