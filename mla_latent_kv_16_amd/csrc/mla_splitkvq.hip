// The split-KV attention pass with the work of a workgroup cut in quarters, for bf16
// latent pools.
//
// A workgroup covers the same work as splitkv_kernel: one (KV partition, M-tile of
// 64 folded query rows) pair, walking the partition's pages as 32-row blocks staged
// in LDS with direct global->LDS copies.  Its four waves split it differently: wave c
// holds ALL 64 query rows of the M-tile (two 32-row query tiles), scores a QUARTER c
// of the 576-wide contraction (S^T = K Q^T partials on v_mfma_f32_32x32x16_bf16, its
// 144 query columns of both tiles resident in registers) and accumulates O for the
// QUARTER c of the 512 output columns.  Each K operand read from LDS therefore feeds
// two MFMAs (one per query tile) and each V column is read by one wave only, so a
// block costs about 116 KB of LDS reads per workgroup, against 152 KB when wave pairs
// split the contraction in halves.
//
// The four partial S^T tiles are summed through LDS: wave c owns kv rows 8 c .. 8 c + 7
// of each 32-row block (its S^T registers 4 c .. 4 c + 3), adds the other three waves'
// partials of those rows, runs the softmax on them for both query tiles and publishes
// its bf16 P; every wave then reads the whole P as the A operand of O += P V.  Each
// query row's weights are spread over the four waves, so the row sums are added
// through LDS once per piece.  The LDS holds a three-slot ring of 36 KB blocks, the
// partial scores (32 KB) and the P tiles (4 KB): one block is in flight while one is
// scored, which suits the compute-bound shapes (prefix prefill, many drafts), whose KV
// comes from L2.
//
// Prior art for the fold and the split-KV structure: TokenSpeed launch news,
// decode-kernel paragraph (drafts folded into heads); "Faster kernels, slower
// engine", §7.1 Gluon MLA decode (split-KV with materialised partials).
#include "mla_device.h"
#include "mla_internal.h"

#include <math.h>

namespace mla {
namespace wq {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQTiles = 2;                   // 32-row query tiles per wave: the whole M-tile
constexpr int kKSteps = kRow / 16 / 4;       // 9 MFMA k-steps: a quarter of the 576-wide row
constexpr int kColTiles = kNope / 32 / 4;    // 4 output column tiles of 32: a quarter of 512
constexpr int kRing = 3;                     // ring slots of one 32-row block (36,864 bytes)
constexpr int kCopies = 9;                   // 16-byte-per-lane copies per wave (36 per block)
constexpr float kLazyRescale = 32.0f;
constexpr float kLazyWeight = 4294967296.0f;  // 2^kLazyRescale
constexpr float kLn2 = 0.69314718055994531f;
static_assert(kQTiles * 32 == kMTile, "a wave holds the whole M-tile");
static_assert(kKSteps >= 2 * 4, "the softmax of both query tiles takes S^T slots 0..7");

// Row (0..31) of register i of a 32x32 MFMA accumulator held by `lane`.
__device__ __forceinline__ int acc_row(int lane, int i) {
  return 4 * (lane >> 5) + 8 * (i >> 2) + (i & 3);
}

// LDS layout: ring | partial scores xs[wave][tile][group][lane] (f32x4) | P tiles.
constexpr int kRingBytes = kRing * kStageBytes;                // 110,592
constexpr int kXsBytes = kWaves * kQTiles * 4 * 64 * 16;        // 32,768
constexpr int kPBytes = kQTiles * 2 * 64 * 16;                  // 4,096: [tile][ks][lane]
constexpr int kLdsBytes = kRingBytes + kXsBytes + kPBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

__device__ __forceinline__ int xs_index(int wave, int p, int j, int lane) {
  return ((wave * kQTiles + p) * 4 + j) * 64 + lane;
}

struct State {
  f32x16 acc[kQTiles][kColTiles];  // O: column 128 c + 32 ct + lane % 32, rows acc_row
  float m_ref[kQTiles];            // exp2 reference (log2 domain) of query row lane % 32
  float m_seen[kQTiles];           // max scaled score of that row over blocks with a max
  float p_hi[kQTiles];             // largest per-block sum of this lane's weights
  float l_run[kQTiles];            // this lane's share of the row's exp2 sum
  float l_bf[kQTiles];             // the same over the bf16-rounded weights
};

// ---- staging ------------------------------------------------------------------------
// A block's 2,304 sixteen-byte LDS chunks are 36 copies of 64 lanes; copy g covers LDS
// chunks 64 g .. 64 g + 63, and wave w issues copies w, w + 4, .., w + 32.  LDS chunk q
// is row q / 72, position q % 72, and receives the pool chunk (q % 72) ^ swz(row) of
// that row (the swizzled layout of a staged page).  Rows at or past `valid` re-read
// row valid - 1 (finite data, masked in the scores).
__device__ __forceinline__ int copy_index(int wave, int i) { return wave + kWaves * i; }

__device__ __forceinline__ uint32_t copy_src(int g, int lane, int valid) {
  const uint32_t q = 64 * g + lane;
  const uint32_t rr = q / kChunks;
  const uint32_t pos = q - rr * kChunks;
  const uint32_t rs = min(rr, (uint32_t)(valid - 1));
  return rs * kRowBytes + ((pos ^ swz(rr)) << 4);
}

struct Offsets {
  uint32_t off[kCopies];
};

__device__ __forceinline__ Offsets offsets() {
  Offsets so;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kCopies; ++i) so.off[i] = copy_src(copy_index(wave, i), lane, kKvBlock);
  return so;
}

// This wave's copies of the block at `src` (wave-uniform) into `slot`.
__device__ __forceinline__ void stage(const uint8_t* src, uint8_t* slot, int valid,
                                      const Offsets& so) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t base = lds_addr(slot);
  if (valid == kKvBlock) {
#pragma unroll
    for (int i = 0; i < kCopies; ++i) dma16(src, so.off[i], base + 1024 * copy_index(wave, i));
  } else {
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
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
// + 4 c4; with ct = 2 a + b the per-lane part depends on b and a adds 128 bytes.  The
// element order of a V operand (element 4 second + r4 is kv row 8 second + 4 h + r4)
// is the order in which the waves publish P, so the contraction pairs each weight with
// its own kv row.
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

// This wave's partial S^T of one staged block (its quarter of the contraction) for both
// query tiles: each K operand feeds the two tiles' MFMAs.
__device__ __forceinline__ void qk_partial(const uint8_t* blk, const Bases& rb,
                                           const bf16x8 (&qreg)[kQTiles][kKSteps],
                                           f32x16 (&s)[kQTiles]) {
  bf16x8 kb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kb[u] = k_read(blk, rb, u);
#pragma unroll
  for (int p = 0; p < kQTiles; ++p) s[p] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < kKSteps; ++kk) {
    const bf16x8 a = kb[kk % 4];
    if (kk + 4 < kKSteps) kb[kk % 4] = k_read(blk, rb, kk + 4);
#pragma unroll
    for (int p = 0; p < kQTiles; ++p) s[p] = mfma32(a, qreg[p][kk], s[p]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Publishes this wave's partial S^T: register group j (kv rows 8 j + 4 h + 0..3) of
// query tile p goes to xs[wave][p][j]; the owner reads its own group back with the
// others'.
__device__ __forceinline__ void store_partial(f32x4* xs, const f32x16 (&s)[kQTiles]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int p = 0; p < kQTiles; ++p)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xs[xs_index(wave, p, j, lane)] =
          f32x4{s[p][4 * j], s[p][4 * j + 1], s[p][4 * j + 2], s[p][4 * j + 3]};
}

// ---- one iteration ---------------------------------------------------------------------
// Scores block i (every wave's partial S^T of it is in xs) and, when HAS_NEXT, computes
// this wave's partial S^T of block i + 1 on the MFMA pipe in between, issuing the
// copies of a later block alongside (one per k-step).  `full`: block i takes the row
// max (each wave then sums all 32 kv rows of its query rows).  `lim[p]`: rows of block
// i this lane's query row of tile p sees.  C is this wave's quarter (wave-uniform).
template <bool HAS_NEXT>
__device__ __forceinline__ void step(int C, const uint8_t* blk, const uint8_t* blk_next,
                                     const Bases& rb,
                                     const bf16x8 (&qreg)[kQTiles][kKSteps], f32x4* xs,
                                     uint8_t* pbuf, State& st, const int (&lim)[kQTiles],
                                     float scale_log2, bool full, const uint8_t* job_src,
                                     uint8_t* job_slot, const Offsets& so) {
  const int lane = threadIdx.x & 63, h = lane >> 5;
  // the four partials of this wave's kv rows (group C), both query tiles
  f32x4 part[kQTiles][4];
#pragma unroll
  for (int p = 0; p < kQTiles; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) part[p][q] = xs[xs_index(q, p, C, lane)];
  bf16x8 kb[4];
  if constexpr (HAS_NEXT) {
#pragma unroll
    for (int u = 0; u < 4; ++u) kb[u] = k_read(blk_next, rb, u);
  }
  __builtin_amdgcn_sched_barrier(0);

  f32x16 nx[kQTiles] = {};
  f32x4 x[kQTiles] = {};  // this wave's scores: kv rows 8 C + 4 h + 0..3 of row lane % 32
  float psum[kQTiles] = {0.0f, 0.0f};
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t job_base = job_slot ? lds_addr(job_slot) : 0u;

#pragma unroll
  for (int kk = 0; kk < kKSteps; ++kk) {
    if constexpr (HAS_NEXT) {
      const bf16x8 a = kb[kk % 4];
      if (kk + 4 < kKSteps) kb[kk % 4] = k_read(blk_next, rb, kk + 4);
#pragma unroll
      for (int p = 0; p < kQTiles; ++p) nx[p] = mfma32(a, qreg[p][kk], nx[p]);
    }
    // copies of a later block, one per k-step (wave-uniform)
    if (job_src) dma16(job_src, so.off[kk], job_base + 1024 * copy_index(wv, kk));
    const int p = kk & 1;
    if (kk < 2) {
      // summed in wave order, so every wave forms bitwise the same scores
      x[p] = ((part[p][0] + part[p][1]) + part[p][2]) + part[p][3];
    } else if (kk < 4) {
      if (full) {
        // the row max over all 32 kv rows of the block (scaling by a positive factor
        // commutes with it); the other groups' partials are read and summed one group
        // at a time, in the same wave order
        float mloc = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 sj;
          if (j == C) {
            sj = x[p];
          } else {
            f32x4 pj[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) pj[q] = xs[xs_index(q, p, j, lane)];
            sj = ((pj[0] + pj[1]) + pj[2]) + pj[3];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            mloc = fmaxf(mloc, 8 * j + 4 * h + e < lim[p] ? sj[e] : -INFINITY);
        }
        mloc = pair32_max(mloc) * scale_log2;
        st.m_seen[p] = fmaxf(st.m_seen[p], mloc);
        if (st.m_ref[p] == -INFINITY) st.m_ref[p] = mloc;  // a row's first visible block
      }
    } else if (kk < 6) {
      const float m_use = st.m_ref[p] == -INFINITY ? 0.0f : st.m_ref[p];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = __builtin_amdgcn_exp2f(fmaf(x[p][e], scale_log2, -m_use));
        x[p][e] = 8 * C + 4 * h + e < lim[p] ? t : 0.0f;  // select: a masked row may overflow
        psum[p] += x[p][e];
      }
    } else if (kk < 8) {
      st.l_run[p] += psum[p];
      if (!full) st.p_hi[p] = fmaxf(st.p_hi[p], psum[p]);  // every weight is <= its sum
      // this wave's P: kv rows 8 C + 4 h + 0..3 of the block, the half (C % 2) of k-step
      // C / 2 of the A operand of O = P V; a row dominated by one key returns that
      // key's c_kv up to fp32 rounding because O is divided by the sum of the rounded
      // weights
      const bf16x4 pb = {static_cast<__bf16>(x[p][0]), static_cast<__bf16>(x[p][1]),
                         static_cast<__bf16>(x[p][2]), static_cast<__bf16>(x[p][3])};
      *reinterpret_cast<bf16x4*>(pbuf + ((2 * p + (C >> 1)) * 64 + lane) * 16 + 8 * (C & 1)) =
          pb;
      const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
      float pbf = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[0], pb[1]}, ones, 0.0f, false);
      pbf = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[2], pb[3]}, ones, pbf, false);
      st.l_bf[p] += pbf;
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
  bf16x8 pa[kQTiles][2];
#pragma unroll
  for (int p = 0; p < kQTiles; ++p)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      pa[p][ks] = *reinterpret_cast<const bf16x8*>(pbuf + ((2 * p + ks) * 64 + lane) * 16);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < 2 * kColTiles; ++t) {
    const int ks = t >> 2, ct = t & 3;
    const bf16x8 v = vb[t & 3];
    if (t + 4 < 2 * kColTiles) vb[t & 3] = v_read(blk, rb, 1, t & 3);
#pragma unroll
    for (int p = 0; p < kQTiles; ++p) st.acc[p][ct] = mfma32(pa[p][ks], v, st.acc[p][ct]);
    if constexpr (HAS_NEXT) {
      if (t == 3) store_partial(xs, nx);
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

// Normalises and writes query tile p's 32 rows x this wave's 128 columns (final O / LSE
// when the piece is the whole request, else a partial slot).  l_tot, l_bf: full row sums
// for row lane % 32 of the tile.
__device__ __forceinline__ void write_rows(const SplitArgs& a, const State& st, int p,
                                           float l_tot, float l_bf, int b, int m_slice,
                                           int row_in_tile, int c, bool whole, int slot) {
  const int lane = threadIdx.x & 63;
  const int M = a.M;
  const bool seen = l_tot > 0.0f;
  const float inv = (seen && l_bf > 0.0f) ? a.kv_scale / l_bf : 0.0f;
  const float lse2 = seen ? st.m_ref[p] + __builtin_amdgcn_logf(l_tot) : -INFINITY;
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
        __builtin_nontemporal_store(st.acc[p][ct][i] * inv_i, rowp + 32 * ct);
    }
  }
  if (c == 0 && lane < 32 && m_slice + lane < M) {
    if (whole)
      a.lse[(size_t)b * M + m_slice + lane] = lse2 * kLn2;
    else
      a.part_lse[(size_t)slot * a.slot_rows + row_in_tile + lane] = lse2;
  }
}

// One piece: logical pages [lo, hi) of request b against M-tile mt.
__device__ __forceinline__ void run_piece(const SplitArgs& a, uint8_t* lds, int b, int L, int mt,
                                          int lo, int hi, bool whole, int slot) {
  const int C = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // this wave's quarter
  uint8_t* ring = lds;
  f32x4* xs = reinterpret_cast<f32x4*>(lds + kRingBytes);
  uint8_t* pbuf = lds + kRingBytes + kXsBytes;
  const int lane = threadIdx.x & 63;
  const int M = a.M;
  int sq = a.Sq;
  if (a.q_lens) {
    const int want = __builtin_amdgcn_readfirstlane(a.q_lens[b]);
    sq = min(max(want, 1), min(a.Sq, max(L, 1)));
  }
  int n_vis[kQTiles];
  bool q_ok[kQTiles];
  // Q^T as the B operand of S^T: lane holds query row m_q of tile p, k = 144 c + 16 kk + 8 h
  bf16x8 qreg[kQTiles][kKSteps];
#pragma unroll
  for (int p = 0; p < kQTiles; ++p) {
    const int m_q = mt * kMTile + 32 * p + (lane & 31);
    q_ok[p] = m_q < sq * a.H;
    const int t = q_ok[p] ? m_q / a.H : 0;
    n_vis[p] = !q_ok[p] ? 0 : (a.causal ? L - sq + t + 1 : L);
    const int h = lane >> 5;
    const size_t qrow = (size_t)b * M + (q_ok[p] ? m_q : 0);
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
      const int k0 = 144 * C + 16 * kk + 8 * h;
      bf16x8 v;
      if (k0 < kNope)
        v = *reinterpret_cast<const bf16x8*>(a.q_nope + qrow * kNope + k0);
      else
        v = *reinterpret_cast<const bf16x8*>(a.q_rope + qrow * kRope + (k0 - kNope));
      qreg[p][kk] = q_ok[p] ? v : bf16x8{};
    }
  }
  const int m_last = min(sq * a.H, (mt + 1) * kMTile) - 1;
  const int n_vis_max = m_last < mt * kMTile ? 0 : (a.causal ? L - sq + m_last / a.H + 1 : L);
  const int nb = max(0, min(2 * (hi - lo), (n_vis_max + kKvBlock - 1) / kKvBlock - 2 * lo));

  State st;
#pragma unroll
  for (int p = 0; p < kQTiles; ++p) st.m_seen[p] = -INFINITY;
  const Bases rb = bases(C);
  const Offsets so = offsets();
  PageIds pi;
  load_page_ids(a, pi, b, lo, hi);
  wait_vmem_all();
  auto lims = [&](int i, int (&lim)[kQTiles]) {
#pragma unroll
    for (int p = 0; p < kQTiles; ++p)
      lim[p] = n_vis[p] - (lo + (i >> 1)) * kPage - (i & 1) * kKvBlock;
  };

  for (int pass = 0; pass < 3; ++pass) {
#pragma unroll
    for (int p = 0; p < kQTiles; ++p) {
#pragma unroll
      for (int ct = 0; ct < kColTiles; ++ct) st.acc[p][ct] = f32x16{};
      st.m_ref[p] = pass < 2 ? -INFINITY : st.m_seen[p];
      st.l_run[p] = 0.0f;
      st.l_bf[p] = 0.0f;
      st.p_hi[p] = 0.0f;
    }
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
    if (nb > 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCopies) : "memory");
    else
      wait_vmem_all();
    __syncthreads();
    if (nb > 0) {
      f32x16 s0[kQTiles];
      qk_partial(ring_slot(ring, 0), rb, qreg, s0);
      store_partial(xs, s0);
    }
    int i = 0;
    int lim[kQTiles];
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
      lims(i, lim);
      step<true>(C, ring_slot(ring, i), ring_slot(ring, i + 1), rb, qreg, xs, pbuf, st, lim,
                    a.scale_log2, full_of(i), job, ring_slot(ring, i + 2), so);
      src_next = nullptr;
      if (i + 3 < nb) src_next = block_source(a, pi, b, lo, hi, L, i + 3, valid_next);
    }
    if (i < nb) {
      __syncthreads();
      lims(i, lim);
      step<false>(C, ring_slot(ring, i), nullptr, rb, qreg, xs, pbuf, st, lim, a.scale_log2,
                     full_of(i), nullptr, nullptr, so);
    }
    bool broke = false;
#pragma unroll
    for (int p = 0; p < kQTiles; ++p)
      broke = broke || (st.m_ref[p] != -INFINITY && st.m_seen[p] > st.m_ref[p] + kLazyRescale) ||
              st.p_hi[p] > kLazyWeight;
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

  // row sums: each wave summed the weights of its kv rows; the four waves add theirs in
  // wave order, then the two lane halves
  f32x2* sums = reinterpret_cast<f32x2*>(lds + kRingBytes);
#pragma unroll
  for (int p = 0; p < kQTiles; ++p)
    sums[(C * kQTiles + p) * 64 + lane] = f32x2{st.l_run[p], st.l_bf[p]};
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kQTiles; ++p) {
    f32x2 tot = sums[p * 64 + lane];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) tot += sums[(q * kQTiles + p) * 64 + lane];
    write_rows(a, st, p, pair32_sum(tot[0]), pair32_sum(tot[1]), b, mt * kMTile + 32 * p,
               32 * p, C, whole, slot);
  }
  __syncthreads();  // the sums have been read before the next piece reuses the LDS
}

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
splitkvq_kernel(SplitArgs a) {
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
      run_piece(a, lds, bb, LL, mt, lo_p, hi_p, whole, slot);
    }
    pb0 = pb1;
  }
}

}  // namespace wq

hipError_t launch_splitkvq(const SplitArgs& a, hipStream_t stream) {
  const int64_t n_split = (int64_t)a.G * a.n_mt;
  if (n_split != a.n_split || n_split <= 0 || n_split > 0x7fffffff || a.arrive || a.kv_e4m3 ||
      a.kv_nope || a.tree_mask)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(wq::splitkvq_kernel, dim3((unsigned)n_split), dim3(wq::kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace mla
