// The split-KV attention pass with two waves per SIMD (eight waves per workgroup),
// for bf16 latent pools.
//
// A workgroup covers the same work as splitkv_kernel: one (KV partition, M-tile of
// 64 folded query rows) pair, walking the partition's pages as 32-row blocks staged
// in LDS with direct global->LDS copies.  The work inside it is cut finer so that each
// wave fits in 256 registers and two waves share every SIMD: wave w = 4 p + c owns
// query rows 32 p .. 32 p + 31 of the M-tile, scores a QUARTER c of the 576-wide
// contraction (S^T = K Q^T partials on v_mfma_f32_32x32x16_bf16, its 144 query
// columns resident in registers) and accumulates O for the QUARTER c of the 512
// output columns.  The four partial S^T tiles of a query half are summed through LDS:
// wave c owns kv rows 8 c .. 8 c + 7 of each 32-row block (its S^T registers
// 4 c .. 4 c + 3), adds the other three waves' partials of those rows, runs the
// softmax on them and publishes its bf16 P; every wave then reads the whole P of its
// query half as the A operand of O += P V.
//
// With one wave per SIMD the LDS operand reads of the single-wave-per-SIMD kernel
// are latency-bound (a wave waits on each read before its MFMA); a second wave on
// the SIMD issues its MFMAs while the first one waits, so the matrix cores stay busy.
// The price is more LDS traffic per flop (each K and V operand read feeds one MFMA,
// and the partial scores cross LDS), which gfx950's LDS sustains at two waves per
// SIMD.  The LDS holds a three-slot ring of 36 KB blocks, the partial scores (32 KB)
// and the P tiles (4 KB): one block is in flight while one is scored, which suits the
// compute-bound shapes (prefix prefill, many drafts), whose KV comes from L2.
//
// Prior art for the fold and the split-KV structure: TokenSpeed launch news,
// decode-kernel paragraph (drafts folded into heads); "Faster kernels, slower
// engine", §7.1 Gluon MLA decode (split-KV with materialised partials).
#include "mla_device.h"
#include "mla_internal.h"

#include <math.h>

namespace mla {
namespace w8 {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKSteps = kRow / 16 / 4;       // 9 MFMA k-steps: a quarter of the 576-wide row
constexpr int kColTiles = kNope / 32 / 4;    // 4 output column tiles of 32: a quarter of 512
constexpr int kRing = 3;                     // ring slots of one 32-row block (36,864 bytes)
constexpr int kCopiesHi = 5;                 // 16-byte-per-lane copies: waves 0..3 take 5,
constexpr int kCopiesLo = 4;                 // waves 4..7 take 4 (36 per block)
constexpr float kLazyRescale = 32.0f;
constexpr float kLazyWeight = 4294967296.0f;  // 2^kLazyRescale
constexpr float kLn2 = 0.69314718055994531f;

// Row (0..31) of register i of a 32x32 MFMA accumulator held by `lane`.
__device__ __forceinline__ int acc_row(int lane, int i) {
  return 4 * (lane >> 5) + 8 * (i >> 2) + (i & 3);
}

// LDS layout: ring | partial scores xs[wave][group][lane] (f32x4) | P tiles.
constexpr int kRingBytes = kRing * kStageBytes;       // 110,592
constexpr int kXsBytes = kWaves * 4 * 64 * 16;         // 32,768
constexpr int kPBytes = 2 * 2 * 64 * 16;               // 4,096: [p][ks][lane] 16 bytes
constexpr int kLdsBytes = kRingBytes + kXsBytes + kPBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

struct State {
  f32x16 acc[kColTiles];  // O: column 128 c + 32 ct + lane % 32, rows acc_row(lane, i)
  float m_ref;            // exp2 reference (log2 domain) of query row lane % 32
  float m_seen;           // max scaled score of that row over the blocks whose max was taken
  float p_hi;             // largest per-block sum of this lane's weights (blocks without max)
  float l_run;            // this lane's share of the row's exp2 sum
  float l_bf;             // the same over the bf16-rounded weights
};

// ---- staging ------------------------------------------------------------------------
// A block's 2,304 sixteen-byte LDS chunks are 36 copies of 64 lanes; copy g covers LDS
// chunks 64 g .. 64 g + 63.  Wave w issues copies w, w + 8, w + 16, w + 24 and, for
// w < 4, 32 + w.  LDS chunk q is row q / 72, position q % 72, and receives the pool
// chunk (q % 72) ^ swz(row) of that row (the swizzled layout of a staged page).  Rows
// at or past `valid` re-read row valid - 1 (finite data, masked in the scores).
__device__ __forceinline__ int copy_index(int wave, int i) { return i < 4 ? wave + 8 * i : 32 + wave; }

__device__ __forceinline__ uint32_t copy_src(int g, int lane, int valid) {
  const uint32_t q = 64 * g + lane;
  const uint32_t rr = q / kChunks;
  const uint32_t pos = q - rr * kChunks;
  const uint32_t rs = min(rr, (uint32_t)(valid - 1));
  return rs * kRowBytes + ((pos ^ swz(rr)) << 4);
}

struct Offsets {
  uint32_t off[kCopiesHi];
};

__device__ __forceinline__ Offsets offsets() {
  Offsets so;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kCopiesHi; ++i) so.off[i] = copy_src(copy_index(wave, i), lane, kKvBlock);
  return so;
}

// This wave's copies of the block at `src` (wave-uniform) into `slot`.
__device__ __forceinline__ void stage(const uint8_t* src, uint8_t* slot, int valid,
                                      const Offsets& so) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t base = lds_addr(slot);
  const int n = wave < 4 ? kCopiesHi : kCopiesLo;
  if (valid == kKvBlock) {
#pragma unroll
    for (int i = 0; i < kCopiesHi; ++i)
      if (i < n) dma16(src, so.off[i], base + 1024 * copy_index(wave, i));
  } else {
#pragma unroll
    for (int i = 0; i < kCopiesHi; ++i)
      if (i < n) {
        const int g = copy_index(wave, i);
        dma16(src, copy_src(g, lane, valid), base + 1024 * g);
      }
  }
}

// ---- LDS read bases -----------------------------------------------------------------
// K (A operand of S^T): lane reads kv row lane % 32 at k = 144 c + 16 kk + 8 h, chunk
// C = 18 c + 2 kk + h; with kk = 4 a + j the per-lane part depends on j only and a adds
// 128 bytes.  V (B operand of P V, read transposed): in 16-lane group G, lane 4 r4 + c4
// addresses kv row 8 second + 4 h + r4 (+ 16 ks) at columns 128 c + 32 ct + 16 (G % 2)
// + 4 c4; with ct = 2 a + b the per-lane part depends on b and a adds 128 bytes.
struct Bases {
  int k[4];
  int v[2][2];
};

__device__ __forceinline__ Bases bases(int c) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  Bases rb;
  const int r = lane & 31, sw = swz(r);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int C = 18 * c + 2 * j + h;
    rb.k[j] = r * kRowBytes + (((C & ~7) | ((C & 7) ^ sw)) << 4);
  }
  const int G = lane >> 4, n = lane & 15, r4 = n >> 2, c4 = n & 3;
#pragma unroll
  for (int second = 0; second < 2; ++second) {
    const int row = 8 * second + 4 * h + r4;
    const int sw2 = swz(row);
#pragma unroll
    for (int b = 0; b < 2; ++b)
      rb.v[second][b] = row * kRowBytes + 256 * c +
                        (((4 * b + 2 * (G & 1) + (c4 >> 1)) ^ sw2) << 4) + 8 * (c4 & 1);
  }
  return rb;
}

__device__ __forceinline__ bf16x8 k_read(const uint8_t* blk, const Bases& rb, int kk) {
  return lds_read_b128(blk + rb.k[kk & 3], (kk >> 2) * 128);
}

__device__ __forceinline__ bf16x8 v_read(const uint8_t* blk, const Bases& rb, int ks, int ct) {
  const int off = (ct >> 1) * 128 + ks * 16 * kRowBytes;
  const bf16x4 lo = lds_read_tr(blk + rb.v[0][ct & 1], off);
  const bf16x4 hi = lds_read_tr(blk + rb.v[1][ct & 1], off);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// This wave's partial S^T of one staged block (its quarter of the contraction).
__device__ __forceinline__ f32x16 qk_partial(const uint8_t* blk, const Bases& rb,
                                             const bf16x8* qreg) {
  bf16x8 kb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kb[u] = k_read(blk, rb, u);
  f32x16 s = {};
#pragma unroll
  for (int kk = 0; kk < kKSteps; ++kk) {
    const bf16x8 a = kb[kk % 4];
    if (kk + 4 < kKSteps) kb[kk % 4] = k_read(blk, rb, kk + 4);
    s = mfma32(a, qreg[kk], s);
    __builtin_amdgcn_sched_barrier(0);
  }
  return s;
}

// Publishes this wave's partial S^T: register group j (kv rows 8 j + 4 h + 0..3) goes
// to xs[wave][j]; the owner reads its own group back with the others'.
__device__ __forceinline__ void store_partial(f32x4* xs, const f32x16& s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    xs[(wave * 4 + j) * 64 + lane] = f32x4{s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]};
}

// ---- one iteration ---------------------------------------------------------------------
// Scores block i (its partial S^T from every wave of the query half is in xs) and, when
// HAS_NEXT, computes this wave's partial S^T of block i + 1 on the MFMA pipe in
// between, issuing the copies of a later block alongside.  `full`: block i takes the
// row max (every wave then sums all 32 kv rows of its query rows).  `lim`: rows of
// block i this lane's query row sees.  C is this wave's quarter (wave % 4).
template <bool HAS_NEXT, int C>
__device__ __forceinline__ void step(const uint8_t* blk, const uint8_t* blk_next, const Bases& rb,
                                     const bf16x8* qreg, f32x4* xs, uint8_t* pbuf, State& st,
                                     int lim, float scale_log2, bool full, const uint8_t* job_src,
                                     uint8_t* job_slot, const Offsets& so) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = wave >> 2, h = lane >> 5;
  const f32x4* xq = xs + (4 * p) * 4 * 64 + lane;  // xs[4 p + q][j][lane] = xq[(4 q + j) 64]
  // the query half's four partials of this wave's kv rows (group C)
  f32x4 part[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) part[q] = xq[(4 * q + C) * 64];
  bf16x8 kb[4];
  if constexpr (HAS_NEXT) {
#pragma unroll
    for (int u = 0; u < 4; ++u) kb[u] = k_read(blk_next, rb, u);
  }
  __builtin_amdgcn_sched_barrier(0);

  f32x16 n0 = {};
  f32x4 x = {};  // this wave's scores: kv rows 8 C + 4 h + 0..3 of query row lane % 32
  float m_use = 0.0f, psum = 0.0f;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int n_copies = wv < 4 ? kCopiesHi : kCopiesLo;
  const uint32_t job_base = job_slot ? lds_addr(job_slot) : 0u;

#pragma unroll
  for (int kk = 0; kk < kKSteps; ++kk) {
    if constexpr (HAS_NEXT) {
      const bf16x8 a = kb[kk % 4];
      if (kk + 4 < kKSteps) kb[kk % 4] = k_read(blk_next, rb, kk + 4);
      n0 = mfma32(a, qreg[kk], n0);
    }
    // copies of a later block, one per two MFMAs (wave-uniform)
    if ((kk & 1) == 0 && job_src && (kk >> 1) < n_copies)
      dma16(job_src, so.off[kk >> 1], job_base + 1024 * copy_index(wv, kk >> 1));
    if (kk == 0) {
      // summed in wave order, so every wave forms bitwise the same scores
      x = ((part[0] + part[1]) + part[2]) + part[3];
    } else if (kk == 1) {
      if (full) {
        // the row max over all 32 kv rows of the block (scaling by a positive factor
        // commutes with it); the other groups' partials are read and summed one group
        // at a time, in the same wave order
        float mloc = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 sj;
          if (j == C) {
            sj = x;
          } else {
            f32x4 pj[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) pj[q] = xq[(4 * q + j) * 64];
            sj = ((pj[0] + pj[1]) + pj[2]) + pj[3];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            mloc = fmaxf(mloc, 8 * j + 4 * h + e < lim ? sj[e] : -INFINITY);
        }
        mloc = pair32_max(mloc) * scale_log2;
        st.m_seen = fmaxf(st.m_seen, mloc);
        if (st.m_ref == -INFINITY) st.m_ref = mloc;  // a row's first visible block sets it
      }
    } else if (kk == 2) {
      m_use = st.m_ref == -INFINITY ? 0.0f : st.m_ref;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = __builtin_amdgcn_exp2f(fmaf(x[e], scale_log2, -m_use));
        x[e] = 8 * C + 4 * h + e < lim ? t : 0.0f;  // select: a masked row may overflow
        psum += x[e];
      }
    } else if (kk == 3) {
      st.l_run += psum;
      if (!full) st.p_hi = fmaxf(st.p_hi, psum);  // every weight is <= its sum
      // this wave's P: kv rows 8 C + 4 h + 0..3 of the block, the half (C % 2) of k-step
      // C / 2 of the A operand of O = P V; a row dominated by one key returns that key's
      // c_kv up to fp32 rounding because O is divided by the sum of the rounded weights
      const bf16x4 pb = {static_cast<__bf16>(x[0]), static_cast<__bf16>(x[1]),
                         static_cast<__bf16>(x[2]), static_cast<__bf16>(x[3])};
      *reinterpret_cast<bf16x4*>(pbuf + ((2 * p + (C >> 1)) * 64 + lane) * 16 + 8 * (C & 1)) = pb;
      const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
      float pbf = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[0], pb[1]}, ones, 0.0f, false);
      pbf = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[2], pb[3]}, ones, pbf, false);
      st.l_bf += pbf;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // the first V operands of block i (this wave's own reads of a block landed before
  // the previous iteration's barrier) are requested before the barrier that publishes P
  bf16x8 vb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) vb[u] = v_read(blk, rb, 0, u);
  // every wave's P of block i is in LDS; every wave is done with block i's partials
  __syncthreads();
  bf16x8 pa[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    pa[ks] = *reinterpret_cast<const bf16x8*>(pbuf + ((2 * p + ks) * 64 + lane) * 16);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < 2 * kColTiles; ++t) {
    const int ks = t >> 2, ct = t & 3;
    const bf16x8 v = vb[t & 3];
    if (t + 4 < 2 * kColTiles) vb[t & 3] = v_read(blk, rb, 1, t & 3);
    st.acc[ct] = mfma32(pa[ks], v, st.acc[ct]);
    if constexpr (HAS_NEXT) {
      if (t == 3) store_partial(xs, n0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Physical pages of 64 consecutive logical pages of one request, one per lane.
struct PageIds {
  int id;
  int first;
};

__device__ __forceinline__ void load_page_ids(const SplitArgs& a, PageIds& pi, int b, int first,
                                              int end) {
  const int idx = first + (int)(threadIdx.x & 63);
  int phys = 0;
  if (idx < end) {
    phys = a.block_table[(size_t)b * a.max_pages + idx];
    if (phys < 0 || (int64_t)phys >= a.num_pages) {
      atomicOr(a.flags, kFlagBadPageId);
      phys = 0;
    }
  }
  pi.id = phys;
  pi.first = first;
}

__device__ __forceinline__ const uint8_t* block_source(const SplitArgs& a, PageIds& pi, int b,
                                                       int lo, int hi, int L, int i, int& valid) {
  const int pg = lo + (i >> 1), half = i & 1;
  if (pg - pi.first >= 64 || pg < pi.first) load_page_ids(a, pi, b, pg, hi);
  const uint32_t phys = __builtin_amdgcn_readlane(pi.id, pg - pi.first);
  valid = min(kKvBlock, L - pg * kPage - half * kKvBlock);
  return reinterpret_cast<const uint8_t*>(a.kv_pool) +
         ((size_t)phys * kPageBytes + (size_t)half * kStageBytes);
}

__device__ __forceinline__ uint8_t* ring_slot(uint8_t* ring, int i) {
  uint32_t off = (uint32_t)(i % kRing) * kStageBytes;
  asm volatile("" : "+s"(off));
  return ring + off;
}

// Normalises and writes this wave's 32 rows x 128 columns (final O / LSE when the piece
// is the whole request, else a partial slot).  l_tot, l_bf: full row sums for row lane % 32.
__device__ __forceinline__ void write_rows(const SplitArgs& a, const State& st, float l_tot,
                                           float l_bf, int b, int m_slice, int row_in_tile,
                                           int c, bool whole, int slot) {
  const int lane = threadIdx.x & 63;
  const int M = a.M;
  const bool seen = l_tot > 0.0f;
  const float inv = (seen && l_bf > 0.0f) ? a.kv_scale / l_bf : 0.0f;
  const float lse2 = seen ? st.m_ref + __builtin_amdgcn_logf(l_tot) : -INFINITY;
  float* base = whole ? a.O + ((size_t)b * M + m_slice) * kNope
                      : a.part_o + ((size_t)slot * a.slot_rows + row_in_tile) * kNope;
  const int col = 128 * c + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = acc_row(lane, i);
    const float inv_i = __shfl(inv, r, 64);
    if (m_slice + r < M) {
      float* rowp = base + (size_t)r * kNope + col;
#pragma unroll
      for (int ct = 0; ct < kColTiles; ++ct)
        __builtin_nontemporal_store(st.acc[ct][i] * inv_i, rowp + 32 * ct);
    }
  }
  if (c == 0 && lane < 32 && m_slice + lane < M) {
    if (whole)
      a.lse[(size_t)b * M + m_slice + lane] = lse2 * kLn2;
    else
      a.part_lse[(size_t)slot * a.slot_rows + row_in_tile + lane] = lse2;
  }
}

// One piece: logical pages [lo, hi) of request b against M-tile mt; C = wave % 4.
template <int C>
__device__ __forceinline__ void run_piece(const SplitArgs& a, uint8_t* lds, int b, int L, int mt,
                                          int lo, int hi, bool whole, int slot) {
  uint8_t* ring = lds;
  f32x4* xs = reinterpret_cast<f32x4*>(lds + kRingBytes);
  uint8_t* pbuf = lds + kRingBytes + kXsBytes;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = wave >> 2, c = C;
  const int M = a.M;
  int sq = a.Sq;
  if (a.q_lens) {
    const int want = __builtin_amdgcn_readfirstlane(a.q_lens[b]);
    sq = min(max(want, 1), min(a.Sq, max(L, 1)));
  }
  const int m_slice = mt * kMTile + p * kRowsPerWave;
  const int m_q = m_slice + (lane & 31);
  const bool q_ok = m_q < sq * a.H;
  const int t = q_ok ? m_q / a.H : 0;
  const int n_vis = !q_ok ? 0 : (a.causal ? L - sq + t + 1 : L);
  const int m_last = min(sq * a.H, (mt + 1) * kMTile) - 1;
  const int n_vis_max = m_last < mt * kMTile ? 0 : (a.causal ? L - sq + m_last / a.H + 1 : L);
  const int nb = max(0, min(2 * (hi - lo), (n_vis_max + kKvBlock - 1) / kKvBlock - 2 * lo));

  // Q^T as the B operand of S^T: lane holds query row m_q, k = 144 c + 16 kk + 8 h
  bf16x8 qreg[kKSteps];
  {
    const int h = lane >> 5;
    const size_t qrow = (size_t)b * M + (q_ok ? m_q : 0);
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
      const int k0 = 144 * c + 16 * kk + 8 * h;
      bf16x8 v;
      if (k0 < kNope)
        v = *reinterpret_cast<const bf16x8*>(a.q_nope + qrow * kNope + k0);
      else
        v = *reinterpret_cast<const bf16x8*>(a.q_rope + qrow * kRope + (k0 - kNope));
      qreg[kk] = q_ok ? v : bf16x8{};
    }
  }

  State st;
  st.m_seen = -INFINITY;
  const Bases rb = bases(c);
  const Offsets so = offsets();
  PageIds pi;
  load_page_ids(a, pi, b, lo, hi);
  wait_vmem_all();
  auto lim_of = [&](int i) { return n_vis - (lo + (i >> 1)) * kPage - (i & 1) * kKvBlock; };

  for (int pass = 0; pass < 3; ++pass) {
#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) st.acc[ct] = f32x16{};
    st.m_ref = pass < 2 ? -INFINITY : st.m_seen;
    st.l_run = 0.0f;
    st.l_bf = 0.0f;
    st.p_hi = 0.0f;
    // the row max: at the first block of the first walk (where every row that sees any
    // of the piece sees its first row) and in every block of the later walks
    auto full_of = [&](int i) { return pass > 0 || i == 0; };
    wait_vmem_all();
    // prologue: blocks 0 and 1 in flight, block 0 scored into partials
    const uint8_t* src_next = nullptr;  // block i + 2 (copied during iteration i)
    int valid_next = kKvBlock;
    {
      int valid;
      if (nb > 0) {
        const uint8_t* s0 = block_source(a, pi, b, lo, hi, L, 0, valid);
        stage(s0, ring_slot(ring, 0), valid, so);
      }
      if (nb > 1) {
        const uint8_t* s1 = block_source(a, pi, b, lo, hi, L, 1, valid);
        stage(s1, ring_slot(ring, 1), valid, so);
      }
      if (nb > 2) src_next = block_source(a, pi, b, lo, hi, L, 2, valid_next);
    }
    // block 0 has landed (block 1's copies may still be in flight)
    if (nb > 1) {
      if (wave < 4)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCopiesHi) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCopiesLo) : "memory");
    } else {
      wait_vmem_all();
    }
    __syncthreads();
    if (nb > 0) store_partial(xs, qk_partial(ring_slot(ring, 0), rb, qreg));
    int i = 0;
    for (; i + 1 < nb; ++i) {
      wait_vmem_all();  // block i + 1 has landed in this wave's share
      // block i + 1 is in LDS; block i's partials are published; every wave is done
      // with block i - 1, whose slot receives block i + 2
      __syncthreads();
      const uint8_t* job = nullptr;
      if (src_next) {
        if (valid_next == kKvBlock)
          job = src_next;
        else  // a request's partial last block: copied here with clamped rows
          stage(src_next, ring_slot(ring, i + 2), valid_next, so);
      }
      step<true, C>(ring_slot(ring, i), ring_slot(ring, i + 1), rb, qreg, xs, pbuf, st,
                    lim_of(i), a.scale_log2, full_of(i), job, ring_slot(ring, i + 2), so);
      src_next = nullptr;
      if (i + 3 < nb) src_next = block_source(a, pi, b, lo, hi, L, i + 3, valid_next);
    }
    if (i < nb) {
      __syncthreads();
      step<false, C>(ring_slot(ring, i), nullptr, rb, qreg, xs, pbuf, st, lim_of(i),
                     a.scale_log2, full_of(i), nullptr, nullptr, so);
    }
    const bool broke = (st.m_ref != -INFINITY && st.m_seen > st.m_ref + kLazyRescale) ||
                       st.p_hi > kLazyWeight;
    int* redo_flag = reinterpret_cast<int*>(pbuf);
    __syncthreads();  // every wave is done with the ring, the partials and the P tiles
    if (threadIdx.x == 0) *redo_flag = 0;
    __syncthreads();
    if (__builtin_amdgcn_ballot_w64(broke) && lane == 0) *redo_flag = 1;
    __syncthreads();
    const bool redo = *redo_flag != 0;
    __syncthreads();
    if (!redo) break;
  }

  // row sums: each wave summed the weights of its kv rows; the four waves of a query
  // half add theirs in wave order, then the two lane halves
  f32x2* sums = reinterpret_cast<f32x2*>(lds + kRingBytes);
  sums[wave * 64 + lane] = f32x2{st.l_run, st.l_bf};
  __syncthreads();
  f32x2 tot = sums[(4 * p) * 64 + lane];
#pragma unroll
  for (int q = 1; q < 4; ++q) tot += sums[(4 * p + q) * 64 + lane];
  write_rows(a, st, pair32_sum(tot[0]), pair32_sum(tot[1]), b, m_slice, p * kRowsPerWave, c,
             whole, slot);
  __syncthreads();  // the sums have been read before the next piece reuses the LDS
}

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
splitkv8_kernel(SplitArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  static_assert((2 * kMaxBatch + 1) * sizeof(int) <= kXsBytes,
                "the page prefix and lengths are built in the partial-score buffer");
  const int lam = a.G > 1 ? xcd_logical_id(blockIdx.x, a.n_split)
                          : a.n_split - 1 - (int)blockIdx.x;
  const int g = lam / a.n_mt;
  const int mt = lam - g * a.n_mt;

  int* prefix = reinterpret_cast<int*>(lds + kRingBytes);
  int* lens = prefix + kMaxBatch + 1;
  build_page_prefix(a.seq_lens, a.B, a.len_min, a.max_pages, prefix, a.flags, true, lens);
  if (a.q_lens && threadIdx.x < 64) {
    for (int j = threadIdx.x; j < a.B; j += 64) {
      const int q = a.q_lens[j];
      if (q < 1 || q > min(a.Sq, lens[j])) atomicOr(a.flags, kFlagBadSeqLen);
    }
  }
  const int64_t T = prefix[a.B];
  const int64_t p0 = part_begin(T, a.G, g);
  const int64_t p1 = part_begin(T, a.G, g + 1);
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid + 1] > p0) hi = mid; else lo = mid + 1;
  }
  int pb0 = prefix[lo];
  const int L_first = lens[lo];
  __syncthreads();
  if (p0 >= p1) return;

  for (int b = lo; b < a.B && pb0 < p1; ++b) {
    const int Lb = b == lo ? L_first : clamp_len(a.seq_lens[b], a.len_min, a.max_pages, a.flags,
                                                  false);
    const int pb1 = pb0 + (Lb + kPage - 1) / kPage;
    if (pb1 > pb0) {
      const int plo = (int)((p0 > pb0 ? p0 : pb0) - pb0);
      const int phi = (int)((p1 < pb1 ? p1 : pb1) - pb0);
      const bool whole = plo == 0 && phi == pb1 - pb0;
      const int bb = __builtin_amdgcn_readfirstlane(b);
      const int LL = __builtin_amdgcn_readfirstlane(Lb);
      const int lo_p = __builtin_amdgcn_readfirstlane(plo);
      const int hi_p = __builtin_amdgcn_readfirstlane(phi);
      const int slot = (b + g) * a.n_mt + mt;
      switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 3) {  // wave-uniform
        case 0: run_piece<0>(a, lds, bb, LL, mt, lo_p, hi_p, whole, slot); break;
        case 1: run_piece<1>(a, lds, bb, LL, mt, lo_p, hi_p, whole, slot); break;
        case 2: run_piece<2>(a, lds, bb, LL, mt, lo_p, hi_p, whole, slot); break;
        default: run_piece<3>(a, lds, bb, LL, mt, lo_p, hi_p, whole, slot); break;
      }
    }
    pb0 = pb1;
  }
}

}  // namespace w8

hipError_t launch_splitkv8(const SplitArgs& a, hipStream_t stream) {
  const int64_t n_split = (int64_t)a.G * a.n_mt;
  if (n_split != a.n_split || n_split <= 0 || n_split > 0x7fffffff || a.arrive || a.kv_e4m3 ||
      a.kv_nope || a.tree_mask)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(w8::splitkv8_kernel, dim3((unsigned)n_split), dim3(w8::kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace mla
