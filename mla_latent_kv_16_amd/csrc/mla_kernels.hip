// gfx950 kernels of the paged latent-KV MLA library.
//
//  splitkv_kernel<NW>  one workgroup = (KV partition g, M-tile mt) with NW waves.
//                      It walks the pages of its partition (possibly across
//                      request boundaries), staging each 64-row page into LDS
//                      with direct global->LDS copies; every wave scores its 16
//                      folded query rows against the staged rows (S^T = K Q^T on
//                      bf16 MFMA), runs the online softmax and accumulates
//                      O += P V.  A request the partition covers whole gets its
//                      final O/LSE; otherwise the piece writes a normalised
//                      partial and its log-sum-exp.
//  combine_kernel      merges the partials of split requests by log-sum-exp.
//
// Split-KV with materialised partials and a reduction pass is the decode design
// the "Faster kernels, slower engine" page describes for MI355X (§7.1 Gluon MLA
// decode).  Folding the draft axis into the head axis so that Sq x H rows fill the
// matrix tile is TokenSpeed's decode-kernel idea (launch news, decode-kernel
// paragraph; review page, Attack 1: H_eff = num_heads x q_seqlen).  On gfx950 the
// folded rows form the N axis of S^T = K Q^T: the staged page is the MFMA A
// operand read straight from LDS, Q stays in registers for the whole walk, and
// the S^T accumulator layout is already the A operand layout of P V.
#include "mla_device.h"
#include "mla_internal.h"

#include <math.h>

namespace mla {

// Skip the O rescale until a row's running max has grown by more than this many
// powers of two.  Until then p = exp2(s - m_ref) stays below 2^32, far inside the
// range of bf16 P and of the fp32 sums (at most 2^32 * 2^21 rows); the final
// normalisation uses the same m_ref, so the result does not depend on when (or
// whether) rescales happen.  Normally only a row's first visible block sets m_ref;
// the rescale is left for adversarial score ranges and runs outside the hot loop.
constexpr float kLazyRescale = 32.0f;

struct WaveState {
  f32x4 acc[kDBlocks];  // O: rows 4 * (lane / 16) + i, columns 16 * db + lane % 16
  float m_ref;          // running max (log2 domain) of this lane's query row
  float l_run;          // this lane's share of that row's exp2 sum (gives the LSE)
  float l_bf;           // the same sum over the bf16-rounded P that enters P V
  float m_pending;      // max that triggered a rescale request
};

// Query row (0..15 within the wave) of element i of an O accumulator.
__device__ __forceinline__ int acc_row(int lane, int i) { return 4 * (lane >> 4) + i; }

__device__ __forceinline__ float row_max(float x) { return pair32_max(xor16_max(x)); }
__device__ __forceinline__ float row_sum(float x) { return pair32_sum(xor16_sum(x)); }

// ---- staging a page into LDS ----------------------------------------------------
// The page is 8 groups of 8 rows; group j is 576 sixteen-byte chunks, i.e. 9 copies
// of 64 lanes x 16 bytes.  Wave w copies groups w, w + NW, ...  LDS chunk position
// q of a group receives the global chunk the swizzled layout wants there.  The
// swizzle of row 8 j + rr depends on j only through j % 2, and every group a wave
// copies has the same parity, so the 9 per-lane source offsets (relative to the
// group's first row) are fixed per wave.
struct StageOffsets {
  int off[9];
};

__device__ __forceinline__ StageOffsets stage_offsets() {
  StageOffsets so;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const int q = i * 64 + lane;
    const int rr = q / kChunks;
    const int pos = q - rr * kChunks;
    so.off[i] = rr * kRowBytes + ((pos ^ swz(8 * wave + rr)) << 4);
  }
  return so;
}

// Stage logical page `pg` of request b into `stage`.  Rows at or past `valid` re-read
// the page's last valid row (finite data whose scores are masked), so nothing past
// L_b is touched.
template <int NW>
__device__ __forceinline__ void stage_page(const SplitArgs& a, const StageOffsets& so,
                                           uint8_t* stage, int b, int pg, int L) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int phys = a.block_table[(size_t)b * a.max_pages + pg];
  if (phys < 0 || (int64_t)phys >= a.num_pages) {
    if (threadIdx.x == 0) atomicOr(a.flags, kFlagBadPageId);
    phys = 0;
  }
  phys = __builtin_amdgcn_readfirstlane(phys);
  const int valid = min(kPage, L - pg * kPage);
  const uint8_t* page = reinterpret_cast<const uint8_t*>(a.kv_pool) + (size_t)phys * kPageBytes;
  const uint32_t lds0 = lds_addr(stage);
  if (valid == kPage) {
#pragma unroll
    for (int j = 0; j < 8 / NW; ++j) {
      const int row0 = 8 * (wave + NW * j);
      const uint8_t* src = page + row0 * kRowBytes;
      const uint32_t dst = lds0 + row0 * kRowBytes;
#pragma unroll
      for (int i = 0; i < 9; ++i) dma16(src, so.off[i], dst + i * 1024);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8 / NW; ++j) {
      const int row0 = 8 * (wave + NW * j);
      const uint32_t dst = lds0 + row0 * kRowBytes;
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        const int q = i * 64 + lane;
        const int rr = q / kChunks;
        const int pos = q - rr * kChunks;
        const int r = row0 + rr;
        const int rs = min(r, valid - 1);
        dma16(page, rs * kRowBytes + ((pos ^ swz(r)) << 4), dst + i * 1024);
      }
    }
  }
}

// ---- per-lane LDS read bases ---------------------------------------------------
// Every LDS address of the walk is (per-lane base) + (compile-time offset): the xor
// swizzle touches only the low three chunk bits, so for each k-step or column
// block the per-lane part takes one of a few values and the rest is an immediate.
struct ReadBases {
  int a[2];   // S^T A operand (kv rows), MFMA k-step kk with kk % 2 == index
  int tr[4];  // V operand (transposed), column block db with db % 4 == index
};

__device__ __forceinline__ ReadBases read_bases() {
  const int lane = threadIdx.x & 63;
  ReadBases rb;
  // A operand of S^T = K Q^T: lane reads kv row lane % 16, k slice 8 * (lane / 16)
  const int row = lane & 15, c0 = lane >> 4, sw = swz(row);
#pragma unroll
  for (int k = 0; k < 2; ++k) rb.a[k] = row * kRowBytes + (((4 * k + c0) ^ sw) << 4);
  // B operand of O += P V: lanes 4 r + c of each 16-lane group address kv row
  // 4 * group + r (and that + 16) at columns 16 * db + 4 c
  const int ra0 = 4 * (lane >> 4) + ((lane & 15) >> 2);
  const int cw = (lane & 3) >> 1;
  const int swa = swz(ra0);  // rows ra0 + 16 share it
#pragma unroll
  for (int p = 0; p < 4; ++p)
    rb.tr[p] = ra0 * kRowBytes + (((2 * p + cw) ^ swa) << 4) + (lane & 1) * 8;
  return rb;
}

// One block of 32 kv rows, starting at byte `blk` of LDS, against this wave's query
// rows: S^T = K Q^T, mask, online softmax, O += P V.  Returns false, with O and the
// sums untouched, when a row with a finite running max needs a rescale; the caller
// applies it and runs the block again.
//
// LDS operand reads run a fixed distance ahead of the MFMAs that consume them and
// sched_barrier pins that order, so the compiler neither serialises each read with
// its MFMA nor hoists every read (and its registers) to the top.
__device__ __forceinline__ bool attend_block(const uint8_t* blk, const ReadBases& rb,
                                             const bf16x8* qreg, WaveState& ws, int lim,
                                             float scale_log2) {
  const int lane = threadIdx.x & 63;
  constexpr int NQK = 2 * kQSteps;  // 36 MFMAs: 2 sub-blocks of 16 kv rows x 18 k-steps
  constexpr int DQ = 4;             // A-operand reads in flight
  constexpr int DV = 2;             // V-operand read pairs in flight

  auto qk_off = [&](int step) {  // step = 2 kk + jj
    const int kk = step >> 1, jj = step & 1;
    return rb.a[kk & 1] + jj * 16 * kRowBytes + (kk >> 1) * 128;
  };
  auto pv_off = [&](int db, int which) {  // which: 0 = rows ra, 1 = rows ra + 16
    return rb.tr[db & 3] + (db >> 2) * 128 + which * 16 * kRowBytes;
  };

  // ---- S^T = K Q^T; lane holds kv rows 16 jj + 4 (lane / 16) + i of column lane % 16
  f32x4 s[2] = {f32x4{}, f32x4{}};
  bf16x8 abuf[DQ];
#pragma unroll
  for (int u = 0; u < DQ; ++u) abuf[u] = lds_read_b128(blk, qk_off(u));
#pragma unroll
  for (int step = 0; step < NQK; ++step) {
    s[step & 1] = mfma(abuf[step % DQ], qreg[step >> 1], s[step & 1]);
    if (step + DQ < NQK) abuf[step % DQ] = lds_read_b128(blk, qk_off(step + DQ));
    __builtin_amdgcn_sched_barrier(0);
  }

  // first V operands go out before the softmax, which does not need them
  bf16x4 vb0[DV], vb1[DV];
#pragma unroll
  for (int u = 0; u < DV; ++u) {
    vb0[u] = lds_read_tr(blk, pv_off(u, 0));
    vb1[u] = lds_read_tr(blk, pv_off(u, 1));
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- scale into the log2 domain, causal / length mask
  float x[8];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[jj * 4 + i] = s[jj][i] * scale_log2;
  if (__builtin_amdgcn_ballot_w64(lim < kBlockRows)) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (jj * 16 + 4 * (lane >> 4) + i >= lim) x[jj * 4 + i] = -INFINITY;
  }

  // ---- online softmax
  float mloc = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  mloc = row_max(mloc);
  const float m_new = fmaxf(ws.m_ref, mloc);
  if (__builtin_amdgcn_ballot_w64(m_new > ws.m_ref + kLazyRescale)) {
    // rows still at -inf have O = 0 and l = 0 and just adopt the new max
    if (__builtin_amdgcn_ballot_w64(ws.m_ref != -INFINITY && m_new > ws.m_ref + kLazyRescale)) {
      ws.m_pending = m_new;
      return false;
    }
    ws.m_ref = m_new;
  }
  const float m_use = (ws.m_ref == -INFINITY) ? 0.0f : ws.m_ref;
  float psum = 0.0f;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    x[v] = __builtin_amdgcn_exp2f(x[v] - m_use);
    psum += x[v];
  }
  ws.l_run += psum;

  // P as the A operand of O += P V: lane holds query row lane % 16 and, as its 8 k
  // values, kv rows 4 (lane / 16) + 0..3 and 16 + 4 (lane / 16) + 0..3.  The V
  // operand is read in that same kv-row order.  O is later divided by the sum of
  // the rounded weights it was built from, so a row dominated by one key returns
  // that key's c_kv up to fp32 rounding rather than up to bf16 rounding.
  const bf16x8 pop = pack_bf16(x);
  float pbf = 0.0f;
#pragma unroll
  for (int v = 0; v < 8; ++v) pbf += static_cast<float>(pop[v]);
  ws.l_bf += pbf;
  __builtin_amdgcn_sched_barrier(0);

  // ---- O += P V, V = c_kv columns of the same staged rows, read transposed
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db) {
    const int u = db % DV;
    const bf16x8 bv = {vb0[u][0], vb0[u][1], vb0[u][2], vb0[u][3],
                       vb1[u][0], vb1[u][1], vb1[u][2], vb1[u][3]};
    ws.acc[db] = mfma(pop, bv, ws.acc[db]);
    if (db + DV < kDBlocks) {
      vb0[u] = lds_read_tr(blk, pv_off(db + DV, 0));
      vb1[u] = lds_read_tr(blk, pv_off(db + DV, 1));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  return true;
}

// Rare path: scale O rows and sums by exp2(m_ref - m_pending) for rows whose finite
// max grew past the lazy threshold, and adopt the new max.
__device__ __forceinline__ void apply_rescale(WaveState& ws) {
  const int lane = threadIdx.x & 63;
  const bool grow = ws.m_pending > ws.m_ref;
  const float alpha =
      (grow && ws.m_ref != -INFINITY) ? __builtin_amdgcn_exp2f(ws.m_ref - ws.m_pending) : 1.0f;
  if (grow) ws.m_ref = ws.m_pending;
  ws.l_run *= alpha;
  ws.l_bf *= alpha;
  float al[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, acc_row(lane, i), 64);
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.acc[db][i] *= al[i];
}

template <int NW>
__device__ __forceinline__ void run_piece(const SplitArgs& a, uint8_t* kv_lds, int b, int mt,
                                          int lo, int hi, bool whole, int slot) {
  constexpr int MT = kRowsPerWave * NW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int M = a.M;
  const int m_wave = mt * MT + wave * kRowsPerWave;
  const int m_q = m_wave + (lane & 15);  // the query row this lane scores
  const bool q_ok = m_q < M;
  const int L = clamp_len(a.seq_lens[b], a.Sq, a.max_pages, a.flags, false);
  const int t = q_ok ? m_q / a.H : 0;
  const int n_vis = a.causal ? L - a.Sq + t + 1 : L;

  // Q^T as the B operand of S^T = K Q^T: lane holds query row m_q,
  // k = 32 kk + 8 (lane / 16) + 0..7
  bf16x8 qreg[kQSteps];
  {
    const int kq = 8 * (lane >> 4);
    const size_t qrow = (size_t)b * M + (q_ok ? m_q : 0);
#pragma unroll
    for (int kk = 0; kk < kQSteps; ++kk) {
      const int k0 = kk * 32 + kq;
      bf16x8 v;
      if (k0 < kNope)
        v = *reinterpret_cast<const bf16x8*>(a.q_nope + qrow * kNope + k0);
      else
        v = *reinterpret_cast<const bf16x8*>(a.q_rope + qrow * kRope + (k0 - kNope));
      qreg[kk] = q_ok ? v : bf16x8{};
    }
  }

  WaveState ws;
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db) ws.acc[db] = f32x4{};
  ws.m_ref = -INFINITY;
  ws.l_run = 0.0f;
  ws.l_bf = 0.0f;
  ws.m_pending = -INFINITY;

  const StageOffsets so = stage_offsets();
  const ReadBases rb = read_bases();
  stage_page<NW>(a, so, kv_lds, b, lo, L);
  // Blocks of 32 kv rows, two per staged page.  The inner loop is the hot path; it
  // leaves only when a rescale is due, which is applied before resuming at the same
  // block (whose page is already staged and published).
  int blk = 2 * lo;
  int resumed = -1;
  for (;;) {
    for (; blk < 2 * hi; ++blk) {
      const int pg = blk >> 1, kb = blk & 1;
      uint8_t* stage = kv_lds + ((pg - lo) & 1) * kPageBytes;
      if (kb == 0 && blk != resumed) {
        wait_vmem_all();  // this wave's copies of page pg have landed
        __syncthreads();  // ... and everyone's; the other buffer is no longer read
        if (pg + 1 < hi)
          stage_page<NW>(a, so, kv_lds + (((pg + 1 - lo) & 1) * kPageBytes), b, pg + 1, L);
      }
      const int lim = n_vis - pg * kPage - kb * kBlockRows;
      if (!attend_block(stage + kb * kBlockRows * kRowBytes, rb, qreg, ws, lim, a.scale_log2))
        break;
    }
    if (blk >= 2 * hi) break;
    apply_rescale(ws);
    resumed = blk;
  }
  __syncthreads();  // both buffers free before the next piece stages into them

  // ---- epilogue: normalise; final result or partial for the combine pass
  const float l_tot = row_sum(ws.l_run);
  const float l_bf = row_sum(ws.l_bf);
  const bool seen = l_tot > 0.0f;
  const float inv = (seen && l_bf > 0.0f) ? 1.0f / l_bf : 0.0f;
  const float lse2 = seen ? ws.m_ref + __builtin_amdgcn_logf(l_tot) : -INFINITY;
  float inv_i[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) inv_i[i] = __shfl(inv, acc_row(lane, i), 64);

  float* obase = whole ? a.O + ((size_t)b * M + m_wave) * kNope
                       : a.part_o + ((size_t)slot * a.slot_rows + (m_wave - mt * MT)) * kNope;
  const int dcol = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = acc_row(lane, i);
    if (m_wave + r < M) {
      float* orow = obase + (size_t)r * kNope + dcol;
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) orow[db * 16] = ws.acc[db][i] * inv_i[i];
    }
  }
  if (lane < 16 && q_ok) {
    if (whole)
      a.lse[(size_t)b * M + m_q] = lse2 * 0.69314718055994531f;
    else
      a.part_lse[(size_t)slot * a.slot_rows + (m_q - mt * MT)] = lse2;
  }
}

template <int NW>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
splitkv_kernel(SplitArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[2 * kPageBytes];
  __shared__ int prefix[kMaxBatch + 1];

  const int lam = xcd_logical_id(blockIdx.x, gridDim.x);
  const int g = lam / a.n_mt;
  const int mt = lam - g * a.n_mt;

  build_page_prefix(a.seq_lens, a.B, a.Sq, a.max_pages, prefix, a.flags, true);
  const int64_t T = prefix[a.B];
  const int64_t p0 = part_begin(T, a.G, g);
  const int64_t p1 = part_begin(T, a.G, g + 1);
  if (p0 >= p1) return;

  // first request whose pages reach past p0
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid + 1] > p0) hi = mid; else lo = mid + 1;
  }
  for (int b = lo; b < a.B && prefix[b] < p1; ++b) {
    const int pb0 = prefix[b], pb1 = prefix[b + 1];
    if (pb1 <= pb0) continue;
    const int plo = (int)((p0 > pb0 ? p0 : pb0) - pb0);
    const int phi = (int)((p1 < pb1 ? p1 : pb1) - pb0);
    const bool whole = plo == 0 && phi == pb1 - pb0;
    run_piece<NW>(a, kv_lds, __builtin_amdgcn_readfirstlane(b), mt,
                  __builtin_amdgcn_readfirstlane(plo), __builtin_amdgcn_readfirstlane(phi), whole,
                  (b + g) * a.n_mt + mt);
  }
}

// One wave per folded query row of a split request: LSE-weighted sum of partials.
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(CombineArgs a) {
  __shared__ int prefix[kMaxBatch + 1];
  build_page_prefix(a.seq_lens, a.B, a.Sq, a.max_pages, prefix, a.flags, false);
  const int64_t T = prefix[a.B];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t gr = (int64_t)blockIdx.x * (kCombineThreads / 64) + wave;
  if (gr >= (int64_t)a.B * a.M) return;
  const int b = (int)(gr / a.M), m = (int)(gr - (int64_t)b * a.M);
  const int pb0 = prefix[b], pb1 = prefix[b + 1];
  if (pb1 <= pb0) return;
  const int g0 = part_of(T, a.G, pb0);
  const int g1 = part_of(T, a.G, pb1 - 1);
  if (g0 == g1) return;  // one partition held the whole request: already final
  const int mt = m / a.MT, ml = m - mt * a.MT;
  const int n = g1 - g0 + 1;
  // Partitions g0..g1 hold the request's pieces.  With more partitions than pages
  // some partitions are empty; they wrote nothing and carry no weight.
  auto lse_of = [&](int s) {
    const int g = g0 + s;
    if (part_begin(T, a.G, g) >= part_begin(T, a.G, g + 1)) return -INFINITY;
    const size_t slot = (size_t)(b + g) * a.n_mt + mt;
    return a.part_lse[slot * a.slot_rows + ml];
  };
  float mx = -INFINITY;
  for (int s = lane; s < n; s += 64) mx = fmaxf(mx, lse_of(s));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
  float tot = 0.0f;
  if (mx != -INFINITY)
    for (int s = lane; s < n; s += 64) tot += exp2f(lse_of(s) - mx);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) tot += __shfl_xor(tot, d, 64);
  const bool seen = tot > 0.0f;
  const float lse2 = seen ? mx + log2f(tot) : -INFINITY;

  f32x4 o0 = {}, o1 = {};
  const int d0 = lane * 8;
  constexpr int U = 8;
  int s = 0;
  for (; s + U <= n; s += U) {
    f32x4 v0[U], v1[U];
    float w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t slot = (size_t)(b + g0 + s + u) * a.n_mt + mt;
      const float* src = a.part_o + (slot * a.slot_rows + ml) * kNope + d0;
      v0[u] = *reinterpret_cast<const f32x4*>(src);
      v1[u] = *reinterpret_cast<const f32x4*>(src + 4);
      const float l = lse_of(s + u);
      w[u] = (seen && l != -INFINITY) ? exp2f(l - lse2) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (w[u] != 0.0f) {  // a zero-weight slot may hold stale data, even NaN
        o0 += w[u] * v0[u];
        o1 += w[u] * v1[u];
      }
    }
  }
  for (; s < n; ++s) {
    const float l = lse_of(s);
    const float w = (seen && l != -INFINITY) ? exp2f(l - lse2) : 0.0f;
    if (w != 0.0f) {
      const size_t slot = (size_t)(b + g0 + s) * a.n_mt + mt;
      const float* src = a.part_o + (slot * a.slot_rows + ml) * kNope + d0;
      o0 += w * *reinterpret_cast<const f32x4*>(src);
      o1 += w * *reinterpret_cast<const f32x4*>(src + 4);
    }
  }
  float* dst = a.O + ((size_t)b * a.M + m) * kNope + d0;
  *reinterpret_cast<f32x4*>(dst) = o0;
  *reinterpret_cast<f32x4*>(dst + 4) = o1;
  if (lane == 0) a.lse[(size_t)b * a.M + m] = lse2 * 0.69314718055994531f;
}

hipError_t launch_splitkv(const SplitArgs& a, int waves, hipStream_t stream) {
  const int64_t nwg = (int64_t)a.G * a.n_mt;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidValue;
  if (waves == 8)
    hipLaunchKernelGGL(splitkv_kernel<8>, dim3((unsigned)nwg), dim3(64 * 8), 0, stream, a);
  else if (waves == 4)
    hipLaunchKernelGGL(splitkv_kernel<4>, dim3((unsigned)nwg), dim3(64 * 4), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.M;
  const int64_t per = kCombineThreads / 64;
  const int64_t nwg = (rows + per - 1) / per;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)nwg), dim3(kCombineThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
