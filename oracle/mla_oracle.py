"""Plain fp64 CPU oracle for absorbed MLA over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this file: only
``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` use it.  It shares no code with the HIP library (no kernels, no
headers, no helpers, no constants generated for both); the two meet only through
the seeded inputs that ``mla_latent_kv_16_amd.workloads`` draws.

What it computes, and where the pages say so
--------------------------------------------
The pages print no MLA equation.  What they do fix:

* All heads share one cached low-rank latent per token, and the RoPE part of the
  key is decoupled from it ("LLM inference systems atlas", §06 State
  architectures and §22 DeepSeek V2 -> V3).  The latent is 512 wide (TokenSpeed
  review page, DeepSeek-V3 entry).
* The kernel runs attention in the "absorb + project" form: the up-projection of
  the keys is folded into the query beforehand and the value up-projection is
  applied to the output afterwards (TokenSpeed review page, Attack 1).  So scores
  are q · [c_kv ; k_rope] and the values are c_kv itself.
* Logical blocks of a request map to scattered physical pages through a block
  table ("LLM inference systems atlas", §07 PagedAttention).
* Speculative decoding scores all draft positions of a request in parallel
  (atlas §16 Speculative decoding); the drafts form a chain, so draft t sees the
  cached prefix and drafts 0..t.  A prefill chunk on top of a cached prefix sees
  the prefix and, causally, itself (atlas §11 Chunked prefill).
* The decode kernel folds the draft axis into the head axis to fill the matrix
  tile (TokenSpeed launch news, decode-kernel paragraph; review page, Attack 1):
  folded row m = t * H + h.  The fold changes the layout, not the result.
* Split-KV decode materialises per-split partial results and reduces them in a
  second pass ("Faster kernels, slower engine", §7.1 Gluon MLA decode); the
  reduction is the log-sum-exp merge in ``lse_merge``.

Readings where the pages are silent (each listed in the design notes):
  seq_lens[b] counts every visible row including the Sq new rows, already in the
  pool; draft t sees rows j <= L_b - Sq + t (bottom-right causal); Sq = 1 is full
  attention; the softmax scale multiplies the whole 576-wide dot product; LSE is
  the natural log of the sum of exp(scaled scores) over visible rows.

Definition (for b < B, t < Sq, h < H):
  K_b[j]   = pool[block_table[b, j // 64], j % 64, :576]           j < L_b
  n_vis    = L_b - Sq + t + 1  if causal else L_b
  s_j      = scale * (q_nope[b,t,h] . K_b[j][:512] + q_rope[b,t,h] . K_b[j][512:])
  LSE      = log(sum_{j < n_vis} exp(s_j))
  O[b,t,h] = sum_{j < n_vis} exp(s_j - LSE) * K_b[j][:512]

Tree-shaped drafts (tree_visible, mla_attention_tree[_loop]) replace the causal
chain among the drafts by each draft's ancestor set; their pins live in
tests/test_oracle_tree.py.

Parity pins for every function here live in tests/test_oracle.py (brute-force
unabsorbed MLA, fold identity, normalisation, single-row and uniform closed
forms, causal = sequential decodes, paging invariance, dense SDPA special case,
split/merge associativity, large-L statistics, hand-derived golden fixtures).
"""
from __future__ import annotations

import numpy as np

PAGE_ROWS = 64
NOPE = 512
ROPE = 64
ROW = NOPE + ROPE


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly.

    A bf16 value is the top half of an IEEE binary32; shifting it into the high
    16 bits of a uint32 gives that binary32, which float64 represents exactly.
    """
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode OCP FP8 E4M3 (E4M3FN) bit patterns (uint8) to float64 exactly.

    Sign bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0 holds
    the subnormals m/8 * 2^-6; the all-ones exponent with all-ones mantissa is NaN
    and there is no infinity, so the largest finite value is 1.75 * 2^8 = 448.
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((e == 0xF) & ((b & 0x7) == 0x7), np.nan, out)


class E4M3Pool:
    """A latent pool stored as E4M3 codes with one per-tensor scale, read as float64.

    Indexing returns the dequantized rows (code value * scale, exact in float64), so
    the gather below reads it like any float pool.
    """

    def __init__(self, codes: np.ndarray, scale: float):
        self.codes = np.asarray(codes, dtype=np.uint8)
        self.scale = float(scale)
        self.shape = self.codes.shape

    def __getitem__(self, idx):
        return e4m3_bits_to_f64(self.codes[idx]) * self.scale


def _f64(x) -> np.ndarray:
    """bf16 bit patterns (uint16) are widened exactly; any float array is taken as is.

    Float inputs let the pins feed values that are not bf16 (e.g. a query with the
    key up-projection absorbed in fp64).
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)


def visible_rows(L: int, Sq: int, t: int, causal: bool) -> int:
    """Number of rows query t of a request sees (prefix + drafts 0..t when causal)."""
    return int(L - Sq + t + 1) if causal else int(L)


def gather_latent_rows(pool: np.ndarray, block_table: np.ndarray, b: int, n: int) -> np.ndarray:
    """Logical rows 0..n-1 of request b, fetched page by page through the block table.

    Returns float64 [n, 576].  Only the pages that hold rows < n are touched.
    """
    j = np.arange(n)
    phys = block_table[b, j // PAGE_ROWS]
    if n and (phys < 0).any():
        raise ValueError("block table has no page for a visible row")
    return _f64(pool[phys, j % PAGE_ROWS, :])


def _query_rows(q_nope, q_rope, b, t, h):
    qn = _f64(q_nope[b, t, h])
    qr = _f64(q_rope[b, t, h])
    return qn, qr


def mla_attention_loop(q_nope, q_rope, pool, block_table, seq_lens, scale, causal=True):
    """Unfolded form: an explicit loop over (request, draft, head).

    Inputs are the bf16 bit arrays of the workload; returns fp64 (O [B,Sq,H,512],
    LSE [B,Sq,H]).  Meant for small inputs.
    """
    B, Sq, H = q_nope.shape[:3]
    scale = float(scale)
    O = np.zeros((B, Sq, H, NOPE))
    LSE = np.zeros((B, Sq, H))
    for b in range(B):
        L = int(seq_lens[b])
        rows = gather_latent_rows(pool, block_table, b, L)
        for t in range(Sq):
            n = visible_rows(L, Sq, t, causal)
            kv = rows[:n]
            for h in range(H):
                qn, qr = _query_rows(q_nope, q_rope, b, t, h)
                s = scale * (kv[:, :NOPE] @ qn + kv[:, NOPE:] @ qr)
                mx = s.max()
                lse = mx + np.log(np.exp(s - mx).sum())
                O[b, t, h] = np.exp(s - lse) @ kv[:, :NOPE]
                LSE[b, t, h] = lse
    return O, LSE


def _folded_rows(q_nope, q_rope, b):
    """Queries of request b with the draft axis folded into the head axis: [Sq*H, 576]."""
    Sq, H = q_nope.shape[1:3]
    qn = _f64(q_nope[b]).reshape(Sq * H, NOPE)
    qr = _f64(q_rope[b]).reshape(Sq * H, ROPE)
    return np.concatenate([qn, qr], axis=1)


def _attend_folded(Q, rows, m_idx, H, Sq, L, scale, causal):
    """Softmax attention of folded query rows Q (row m_idx[i] = t*H + h) over rows[:L]."""
    S = (Q @ rows.T) * scale                        # [n_rows, L]
    t = m_idx // H
    n_vis = (L - Sq + t + 1) if causal else np.full_like(t, L)
    j = np.arange(rows.shape[0])
    S = np.where(j[None, :] < n_vis[:, None], S, -np.inf)
    mx = S.max(axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(np.exp(S - mx).sum(axis=1))
    P = np.exp(S - lse[:, None])
    return P @ rows[:, :NOPE], lse


def mla_attention_folded(q_nope, q_rope, pool, block_table, seq_lens, scale, causal=True,
                         row_chunk=2048):
    """Folded form: per request one [Sq*H, 576] x [576, L] product, masked by t = m // H.

    Rows are processed in chunks of ``row_chunk`` folded rows so that prefill-sized
    inputs fit in memory; chunking rows changes nothing since rows are independent.
    """
    B, Sq, H = q_nope.shape[:3]
    M = Sq * H
    O = np.zeros((B, M, NOPE))
    LSE = np.zeros((B, M))
    for b in range(B):
        L = int(seq_lens[b])
        rows = gather_latent_rows(pool, block_table, b, L)
        Q = _folded_rows(q_nope, q_rope, b)
        for m0 in range(0, M, row_chunk):
            m1 = min(M, m0 + row_chunk)
            O[b, m0:m1], LSE[b, m0:m1] = _attend_folded(
                Q[m0:m1], rows, np.arange(m0, m1), H, Sq, L, float(scale), causal)
    return O.reshape(B, Sq, H, NOPE), LSE.reshape(B, Sq, H)


def mla_attention_rows(q_nope, q_rope, pool, block_table, seq_lens, scale, causal, b, m_list):
    """Folded rows ``m_list`` (m = t*H + h) of request b only: (O [n,512], LSE [n]).

    Used to check outputs sampled from full-size workloads.
    """
    Sq, H = q_nope.shape[1:3]
    L = int(seq_lens[b])
    rows = gather_latent_rows(pool, block_table, b, L)
    m_idx = np.asarray(m_list, dtype=np.int64)
    Q = _folded_rows(q_nope, q_rope, b)[m_idx]
    return _attend_folded(Q, rows, m_idx, H, Sq, L, float(scale), causal)


def mla_attention_pages(q_nope, q_rope, pool, block_table, seq_lens, scale, causal, b,
                        page_lo, page_hi):
    """Attention of request b restricted to its logical pages [page_lo, page_hi).

    This is one split's partial result: (O_s [Sq,H,512], LSE_s [Sq,H]).  A query that
    sees no row of the range gets LSE_s = -inf and O_s = 0.
    """
    Sq, H = q_nope.shape[1:3]
    L = int(seq_lens[b])
    rows = gather_latent_rows(pool, block_table, b, L)
    O = np.zeros((Sq, H, NOPE))
    LSE = np.full((Sq, H), -np.inf)
    lo = page_lo * PAGE_ROWS
    for t in range(Sq):
        hi = min(page_hi * PAGE_ROWS, visible_rows(L, Sq, t, causal))
        if hi <= lo:
            continue
        kv = rows[lo:hi]
        for h in range(H):
            qn, qr = _query_rows(q_nope, q_rope, b, t, h)
            s = float(scale) * (kv[:, :NOPE] @ qn + kv[:, NOPE:] @ qr)
            mx = s.max()
            lse = mx + np.log(np.exp(s - mx).sum())
            O[t, h] = np.exp(s - lse) @ kv[:, :NOPE]
            LSE[t, h] = lse
    return O, LSE


def tree_visible(L: int, Sq: int, t: int, mask_word: int) -> np.ndarray:
    """Rows draft t sees under a draft tree: the cached prefix rows 0 .. L-Sq-1, then
    the draft rows L-Sq+t' for every t' <= t whose bit t' is set in mask_word, and
    always its own row L-Sq+t.

    Drafts of a tree are verified in parallel, each against its own branch (atlas
    §16 Speculative decoding; the atlas node on tree-shaped drafts).  Reading: drafts
    are numbered so that every ancestor precedes its descendants, bit t' of a
    draft's mask word marks ancestor t', bits above t are ignored, and a draft always
    sees itself.
    """
    prefix = np.arange(L - Sq)
    own = [L - Sq + u for u in range(t + 1) if u == t or (int(mask_word) >> u) & 1]
    return np.concatenate([prefix, np.asarray(own, dtype=np.int64)])


def mla_attention_tree_loop(q_nope, q_rope, pool, block_table, seq_lens, scale, tree_mask):
    """Tree-masked attention, explicit loop over (request, draft, head): each query
    attends to exactly the rows tree_visible() lists.  tree_mask: uint64 [B, Sq].
    Returns fp64 (O [B,Sq,H,512], LSE [B,Sq,H]).  Meant for small inputs."""
    B, Sq, H = q_nope.shape[:3]
    scale = float(scale)
    O = np.zeros((B, Sq, H, NOPE))
    LSE = np.zeros((B, Sq, H))
    for b in range(B):
        L = int(seq_lens[b])
        rows = gather_latent_rows(pool, block_table, b, L)
        for t in range(Sq):
            kv = rows[tree_visible(L, Sq, t, int(tree_mask[b, t]))]
            for h in range(H):
                qn, qr = _query_rows(q_nope, q_rope, b, t, h)
                s = scale * (kv[:, :NOPE] @ qn + kv[:, NOPE:] @ qr)
                mx = s.max()
                lse = mx + np.log(np.exp(s - mx).sum())
                O[b, t, h] = np.exp(s - lse) @ kv[:, :NOPE]
                LSE[b, t, h] = lse
    return O, LSE


def mla_attention_tree(q_nope, q_rope, pool, block_table, seq_lens, scale, tree_mask):
    """Tree-masked attention in the folded form: per request one [Sq*H, 576] x [576, L]
    product with each folded row m = t*H + h masked to tree_visible(L, Sq, t, ...)."""
    B, Sq, H = q_nope.shape[:3]
    M = Sq * H
    O = np.zeros((B, M, NOPE))
    LSE = np.zeros((B, M))
    for b in range(B):
        L = int(seq_lens[b])
        rows = gather_latent_rows(pool, block_table, b, L)
        Q = _folded_rows(q_nope, q_rope, b)
        vis = np.zeros((Sq, L), dtype=bool)
        for t in range(Sq):
            vis[t, tree_visible(L, Sq, t, int(tree_mask[b, t]))] = True
        S = (Q @ rows.T) * float(scale)
        S = np.where(np.repeat(vis, H, axis=0), S, -np.inf)
        mx = S.max(axis=1, keepdims=True)
        LSE[b] = mx[:, 0] + np.log(np.exp(S - mx).sum(axis=1))
        O[b] = np.exp(S - LSE[b][:, None]) @ rows[:, :NOPE]
    return O.reshape(B, Sq, H, NOPE), LSE.reshape(B, Sq, H)


def mla_attention_tree_rows(q_nope, q_rope, pool, block_table, seq_lens, scale, tree_mask, b,
                            m_list):
    """Folded rows ``m_list`` (m = t*H + h) of request b under a draft tree:
    (O [n,512], LSE [n]), each row attending to tree_visible() of its draft."""
    Sq, H = q_nope.shape[1:3]
    L = int(seq_lens[b])
    rows = gather_latent_rows(pool, block_table, b, L)
    Q = _folded_rows(q_nope, q_rope, b)
    O = np.zeros((len(m_list), NOPE))
    LSE = np.zeros(len(m_list))
    for k, m in enumerate(m_list):
        kv = rows[tree_visible(L, Sq, int(m) // H, int(tree_mask[b, int(m) // H]))]
        s = (kv @ Q[int(m)]) * float(scale)
        mx = s.max()
        LSE[k] = mx + np.log(np.exp(s - mx).sum())
        O[k] = np.exp(s - LSE[k]) @ kv[:, :NOPE]
    return O, LSE


def mla_attention_varlen(q_nope, q_rope, pool, block_table, seq_lens, scale, q_lens):
    """Per-request draft counts: request b verifies q_lens[b] <= Sq drafts, which
    are its last q_lens[b] rows; draft t < q_lens[b] sees rows j <= L_b - q_lens[b] + t.
    Query slots t >= q_lens[b] are padding and see nothing: O = 0, LSE = -inf.

    Speculative decoding verifies a varying number of candidates per request (atlas
    §16 Speculative decoding: longer drafts are not always faster); the reading is
    that a batch pads its queries to the largest count.  Returns fp64
    (O [B,Sq,H,512], LSE [B,Sq,H])."""
    B, Sq, H = q_nope.shape[:3]
    O = np.zeros((B, Sq, H, NOPE))
    LSE = np.full((B, Sq, H), -np.inf)
    for b in range(B):
        n = int(q_lens[b])
        if n < 1:
            continue
        o, l = mla_attention_folded(q_nope[b:b + 1, :n], q_rope[b:b + 1, :n], pool,
                                    block_table[b:b + 1], seq_lens[b:b + 1], scale, True)
        O[b, :n], LSE[b, :n] = o[0], l[0]
    return O, LSE


def e4m3_quantize(x) -> np.ndarray:
    """float32 values -> E4M3 codes: the nearest E4M3 value, ties to the code with an
    even mantissa, magnitudes past the largest finite value (448) saturated to it.

    Written as a search over the 127 finite non-negative codes (decoded by
    e4m3_bits_to_f64), not by bit manipulation.  Sign is kept, so -0.0 gives 0x80.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    codes = np.arange(127, dtype=np.uint8)           # 0x00 .. 0x7E (0x7F is NaN)
    vals = e4m3_bits_to_f64(codes)                    # increasing, 0 .. 448
    a = np.minimum(np.abs(x), vals[-1])
    d = np.abs(a[..., None] - vals)                   # distance to every code
    best = d.min(axis=-1, keepdims=True)
    tie = d == best                                   # one or two nearest codes
    even = tie & (codes % 2 == 0)
    pick = np.where(even.any(axis=-1), even.argmax(axis=-1), tie.argmax(axis=-1))
    return (codes[pick] | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)).astype(np.uint8)


def kv_append(pool, block_table, seq_lens, kv_new):
    """The pool after writing each request's new latent rows: kv_new[b, t] (t < Sq)
    becomes logical row L_b - Sq + t of request b, i.e. the rows the decode then
    reads as its drafts ("absorb + project" brackets the attention; the new tokens'
    latents are cached before they are attended to).  Returns a new array."""
    out = np.array(pool, copy=True)
    B, Sq = kv_new.shape[:2]
    for b in range(B):
        L = int(seq_lens[b])
        for t in range(Sq):
            j = L - Sq + t
            out[block_table[b, j // PAGE_ROWS], j % PAGE_ROWS] = kv_new[b, t]
    return out


def mla_attention_nope(q_nope, pool, block_table, seq_lens, scale, causal=True, b_m=None):
    """NoPE-MLA: the cached row is the 512-wide latent alone (no decoupled RoPE key;
    "Faster kernels, slower engine", "Two stacks, one inverted flag": Kimi-K3's MLA
    layers are NoPE-MLA).  Scores are scale * q_nope . c_kv and the values are c_kv.
    pool [P, 64, 512].  Returns fp64 (O [B,Sq,H,512], LSE [B,Sq,H]); with
    b_m = (b, m_list), only those folded rows of request b: (O [n,512], LSE [n])."""
    B, Sq, H = q_nope.shape[:3]
    M = Sq * H

    def one(b, m_idx):
        L = int(seq_lens[b])
        rows = gather_latent_rows(pool, block_table, b, L)          # [L, 512]
        Q = _f64(q_nope[b]).reshape(M, NOPE)[m_idx]
        S = (Q @ rows.T) * float(scale)
        t = m_idx // H
        n_vis = (L - Sq + t + 1) if causal else np.full_like(t, L)
        S = np.where(np.arange(L)[None, :] < n_vis[:, None], S, -np.inf)
        mx = S.max(axis=1, keepdims=True)
        lse = mx[:, 0] + np.log(np.exp(S - mx).sum(axis=1))
        return np.exp(S - lse[:, None]) @ rows, lse

    if b_m is not None:
        return one(b_m[0], np.asarray(b_m[1], dtype=np.int64))
    O = np.zeros((B, M, NOPE))
    LSE = np.zeros((B, M))
    for b in range(B):
        O[b], LSE[b] = one(b, np.arange(M))
    return O.reshape(B, Sq, H, NOPE), LSE.reshape(B, Sq, H)


def absorb_q(q_heads, w_uk_t):
    """The query with the key up-projection absorbed (TokenSpeed review page, Attack 1:
    "absorb" before the latent attention): q_lat[b,t,h,c] = sum_k q_heads[b,t,h,k] *
    W_UK[h][k][c], with w_uk_t[h, c, k] = W_UK[h][k][c].  q_heads [B,Sq,H,128]
    (bf16 bits or floats), w_uk_t [H,512,128].  Returns fp64 [B,Sq,H,512]."""
    return np.einsum("bthk,hck->bthc", _f64(q_heads), _f64(w_uk_t))


def project_o(O, w_uv):
    """The value up-projection applied to the latent output (the "project" after the
    attention): out[b,t,h,v] = sum_c O[b,t,h,c] * W_UV[h][v][c].  O [B,Sq,H,512]
    (floats), w_uv [H,128,512] (bf16 bits or floats).  Returns fp64 [B,Sq,H,128]."""
    return np.einsum("bthc,hvc->bthv", np.asarray(O, dtype=np.float64), _f64(w_uv))


def lse_merge(parts):
    """Merge split partials [(O_s, LSE_s), ...] into (O, LSE).

    LSE = log(sum_s exp(LSE_s)) (max-shifted) and O = sum_s exp(LSE_s - LSE) * O_s.
    Parts whose LSE_s is -inf (no visible row) carry zero weight.
    """
    lses = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])
    outs = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])
    mx = lses.max(axis=0)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    tot = np.exp(lses - safe).sum(axis=0)
    lse = np.where(np.isfinite(mx), safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    w = np.where(np.isfinite(lses), np.exp(lses - np.where(np.isfinite(lse), lse, 0.0)), 0.0)
    return (w[..., None] * outs).sum(axis=0), lse
