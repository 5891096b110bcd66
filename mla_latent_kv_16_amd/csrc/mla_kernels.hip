// gfx950 kernels of the paged latent-KV MLA library.
//
//  splitkv_kernel      one workgroup = (KV partition g, M-tile of 64 folded query
//                      rows), four waves.  It walks the pages of its partition
//                      (possibly across request boundaries) as 32-row blocks,
//                      staged into an LDS ring with direct global->LDS copies two
//                      blocks ahead.  A pair of waves owns 32 query rows: each
//                      wave scores half of the 576-wide contraction (S^T = K Q^T
//                      on v_mfma_f32_32x32x16_bf16, its half of Q resident in
//                      registers), the pair swaps halves through LDS, both run the
//                      online softmax on the full scores, and each accumulates
//                      O += P V for its 256 of the 512 output columns.  A request
//                      the partition covers whole gets its final O/LSE; otherwise
//                      the piece writes a normalised partial and its log-sum-exp.
//  combine_kernel      merges the partials of split requests by log-sum-exp.
//
// Split-KV with materialised partials and a reduction pass is the decode design
// the "Faster kernels, slower engine" page describes for MI355X (§7.1 Gluon MLA
// decode).  Folding the draft axis into the head axis so that Sq x H rows fill the
// matrix tile is TokenSpeed's decode-kernel idea (launch news, decode-kernel
// paragraph; review page, Attack 1: H_eff = num_heads x q_seqlen).  On gfx950 the
// folded rows form the N axis of S^T = K Q^T, so the staged page is the MFMA A
// operand read straight from LDS, a query row's 64 scores of a page sit in two
// lanes (row reductions are one permlane32 swap), and the S^T accumulator is
// already the A-operand layout of O = P V.
#include "mla_device.h"
#include "mla_internal.h"

#include <math.h>

namespace mla {

// A row's exp2 reference m_ref is the max of its first visible block and then stays
// fixed while the piece is walked, so p = exp2(s - m_ref) needs no running rescale
// of O inside the loop as long as later scores stay below m_ref + kLazyRescale
// (p < 2^32, far inside the range of bf16 P and of the fp32 sums).  Only blocks
// where some row still lacks a reference take the row max; elsewhere each wave
// bounds its weights by their per-block sum.  If any weight may have broken the
// bound, the piece is walked again taking every block's max (which, with the
// first block's reference again, usually breaks the same way but finds the true
// maxima), and if need be a third time with m_ref set to those maxima, where no
// score can exceed it.  The final normalisation uses the same m_ref as the sums, so
// the result does not depend on which reference was used.
constexpr float kLazyRescale = 32.0f;
constexpr float kLazyWeight = 4294967296.0f;  // 2^kLazyRescale
constexpr float kLn2 = 0.69314718055994531f;

struct WaveState {
  f32x16 acc[kColTilesPerWave];  // O: column 256 c + 32 ct + lane % 32, rows acc_row(lane, i)
  float m_ref;                   // exp2 reference (log2 domain) of query row lane % 32
  float m_seen;                  // max score of that row over the blocks whose max was taken
  float p_hi;                    // largest per-block sum of this lane's weights (a bound on
                                 // each weight, for blocks whose max was not taken)
  float l_run;                   // this lane's share of that row's exp2 sum (gives the LSE)
  float l_bf;                    // the same sum over the bf16-rounded P that enters P V
};

// Row (0..31) of register i of a 32x32 MFMA accumulator held by `lane`; the same map
// gives the kv row of an S^T register and the query row of an O register.
__device__ __forceinline__ int acc_row(int lane, int i) {
  return 4 * (lane >> 5) + 8 * (i >> 2) + (i & 3);
}

// ---- staging a block into LDS ----------------------------------------------------
// A block is 32 rows (half a page) = 4 groups of 8 rows; wave w copies group w:
// 576 sixteen-byte chunks, i.e. 9 direct global->LDS copies of 64 lanes x 16 bytes.
// LDS chunk position q of the group receives the global chunk the swizzled layout
// wants there; the swizzle of a row depends only on its index mod 16, so the half
// of the page does not matter.  Rows at or past `valid` re-read the block's last
// valid row (finite data whose scores are masked), so nothing past the request's
// length is touched.
struct StageOffsets {
  uint32_t off[kStageCopiesPerWave];  // per-lane source offset of copy i (rows 8 w .. 8 w + 7)
};

__device__ __forceinline__ StageOffsets stage_offsets() {
  StageOffsets so;
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kStageCopiesPerWave; ++i) {
    const uint32_t q = i * 64 + lane;
    const uint32_t rr = q / kChunks;
    const uint32_t pos = q - rr * kChunks;
    const uint32_t r = 8 * wave + rr;
    so.off[i] = r * kRowBytes + ((pos ^ swz(r)) << 4);
  }
  return so;
}

// Copies this wave's share of the block whose first row is at `src` (wave-uniform)
// into ring slot `slot`.
__device__ __forceinline__ void stage_block(const uint8_t* src, uint8_t* slot, int valid,
                                            const StageOffsets& so) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t dst = lds_addr(slot) + 8 * wave * kRowBytes;
  if (8 * (int)wave + 8 <= valid) {
#pragma unroll
    for (int i = 0; i < kStageCopiesPerWave; ++i) dma16(src, so.off[i], dst + i * 1024);
  } else {  // the request's last block: rows past its length re-read row valid - 1
#pragma unroll
    for (int i = 0; i < kStageCopiesPerWave; ++i) {
      const uint32_t q = i * 64 + lane;
      const uint32_t rr = q / kChunks;
      const uint32_t pos = q - rr * kChunks;
      const uint32_t r = 8 * wave + rr;
      const uint32_t rs = min(r, (uint32_t)(valid - 1));
      dma16(src, rs * kRowBytes + ((pos ^ swz(r)) << 4), dst + i * 1024);
    }
  }
}

// E4M3 blocks: wave w copies LDS chunk positions q = 320 w .. 320 w + 319 of its slot
// (five copies of 64 lanes x 16 bytes); positions past the block's 1,152 chunks are
// the slot's padding and re-read an in-block chunk.  LDS chunk q holds row q / 36,
// chunk (q % 36) ^ swz8(row) of the block.
struct StageOffsets8 {
  uint32_t off[kStageCopies8];
};

__device__ __forceinline__ uint32_t stage_src8(uint32_t q, int valid) {
  if (q >= (uint32_t)kBlockChunks8) q -= kBlockChunks8;  // padding
  const uint32_t r = q / kChunks8;
  const uint32_t pos = q - r * kChunks8;
  const uint32_t rs = min(r, (uint32_t)(valid - 1));  // rows past the length re-read the last
  return rs * kRowBytes8 + ((pos ^ swz8(r)) << 4);
}

__device__ __forceinline__ StageOffsets8 stage_offsets8() {
  StageOffsets8 so;
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < kStageCopies8; ++k)
    so.off[k] = stage_src8((kStageCopies8 * wave + k) * 64 + lane, kKvBlock);
  return so;
}

__device__ __forceinline__ uint32_t stage_dst8(const uint8_t* slot) {
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  return lds_addr(slot) + kStageCopies8 * 1024 * wave;
}

__device__ __forceinline__ void stage_block8(const uint8_t* src, uint8_t* slot, int valid,
                                             const StageOffsets8& so) {
  const uint32_t dst = stage_dst8(slot);
  if (valid == kKvBlock) {
#pragma unroll
    for (int k = 0; k < kStageCopies8; ++k) dma16(src, so.off[k], dst + k * 1024);
  } else {  // the request's last block
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < kStageCopies8; ++k)
      dma16(src, stage_src8((kStageCopies8 * wave + k) * 64 + lane, valid), dst + k * 1024);
  }
}

// E4M3 read bases.  K (A operand of S^T): the k order inside each pair of k-steps is
// permuted so that one sixteen-byte read feeds two MFMAs: for the wave's read t
// (0..8) lane half h holds k = 32 (9 c + t) + 16 h + 0..15, bytes 0..7 for k-step 2 t
// and 8..15 for k-step 2 t + 1 (the queries are loaded in the same order).  That is
// chunk 18 c + 2 t + h of row lane % 32.  V (B operand of P V): transposed 8-bit
// reads, where byte j of lane n of a 16-lane group comes from lane 2 j + n / 8 of the
// group.  Byte j must hold the kv row that P's element j stands for (16 ks + 4 h +
// j % 4 + 8 (j / 4), the S^T accumulator order), so lane 16 g + m addresses row
// 16 ks + 4 (g / 2) + 8 (m / 8) + (m / 2) % 4 at columns 256 c + 32 ct + 16 (g % 2) +
// 8 (m % 2).
struct ReadBases8 {
  int k[2];  // read t: k[t % 2] + 64 (t / 2)
  int v[2];  // column tile ct, k-step ks: v[ct % 2] + 64 (ct / 2) + 16 * 576 ks
};

__device__ __forceinline__ ReadBases8 read_bases8(int c) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  ReadBases8 rb;
  const int r = lane & 31, f = swz8(r);
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int C = 18 * c + 2 * v + h;
    rb.k[v] = r * kRowBytes8 + (((C & ~3) | ((C & 3) ^ f)) << 4);
  }
  const int g = lane >> 4, m = lane & 15;
  const int rv = 4 * (g >> 1) + 8 * (m >> 3) + ((m >> 1) & 3);
  const int fv = swz8(rv);  // bits 2 and 3 of the row do not depend on ks
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int C = 16 * c + 2 * par + (g & 1);
    rb.v[par] = rv * kRowBytes8 + (((C & ~3) | ((C & 3) ^ fv)) << 4) + 8 * (m & 1);
  }
  return rb;
}

// ---- per-lane LDS read bases ---------------------------------------------------
// Every LDS address of the walk is (per-lane base) + (compile-time offset): the xor
// swizzle touches only the low three chunk bits, so for each k-step or column tile
// the per-lane part takes one of a few values and the rest is an immediate.
struct ReadBases {
  int k[4];     // S^T A operand: kv row lane % 32, local k-step kk with kk % 4 == index
  int v[2][2];  // O B operand (V read transposed): [second 4-row group][column tile % 2]
};

// c: this wave's half of the 576-wide contraction (k-steps 18 c .. 18 c + 17) and
// of the 512 output columns (256 c .. 256 c + 255).
__device__ __forceinline__ ReadBases read_bases(int c) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  ReadBases rb;
  // A operand of S^T = K Q^T: lane reads kv row lane % 32 at k = 16 (18 c + kk) + 8 h,
  // i.e. chunk 36 c + 2 kk + h = 8 (kk / 4) + C with C = 36 c + 2 (kk % 4) + h
  const int r = lane & 31, sw = swz(r);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int C = 36 * c + 2 * j + h;
    rb.k[j] = r * kRowBytes + (((C & ~7) | ((C & 7) ^ sw)) << 4);
  }
  // B operand of O = P V: in 16-lane group G, lane 4 r4 + c4 addresses kv row
  // 16 ks + 8 second + 4 h + r4 at columns 256 c + 32 ct + 16 (G % 2) + 4 c4
  const int G = lane >> 4, n = lane & 15, r4 = n >> 2, c4 = n & 3;
#pragma unroll
  for (int second = 0; second < 2; ++second) {
    const int row = 8 * second + 4 * h + r4;
    const int sw2 = swz(row);
#pragma unroll
    for (int par = 0; par < 2; ++par)
      rb.v[second][par] = row * kRowBytes + 512 * c +
                          (((4 * par + 2 * (G & 1) + (c4 >> 1)) ^ sw2) << 4) + 8 * (c4 & 1);
  }
  return rb;
}

// NoPE blocks: wave w copies rows 8 w .. 8 w + 7 of the block (eight copies, one row
// each); lane l of copy i fetches chunk l ^ swzn(row) of that row into LDS position l.
struct StageOffsetsN {
  uint32_t off[kNopeCopies];
};

__device__ __forceinline__ StageOffsetsN stage_offsets_nope() {
  StageOffsetsN so;
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kNopeCopies; ++i) {
    const uint32_t r = 8 * wave + i;
    so.off[i] = r * kNopeRowBytes + ((lane ^ swzn(r)) << 4);
  }
  return so;
}

__device__ __forceinline__ uint32_t stage_dst_nope(const uint8_t* slot) {
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  return lds_addr(slot) + 8 * wave * kNopeRowBytes;
}

__device__ __forceinline__ void stage_block_nope(const uint8_t* src, uint8_t* slot, int valid,
                                                 const StageOffsetsN& so) {
  const uint32_t dst = stage_dst_nope(slot);
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (8 * (int)wave + 8 <= valid) {
#pragma unroll
    for (int i = 0; i < kNopeCopies; ++i) dma16(src, so.off[i], dst + i * 1024);
  } else {  // the request's last block: rows past its length re-read row valid - 1
    const uint32_t lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kNopeCopies; ++i) {
      const uint32_t r = 8 * wave + i;
      const uint32_t rs = min(r, (uint32_t)(valid - 1));
      dma16(src, rs * kNopeRowBytes + ((lane ^ swzn(r)) << 4), dst + i * 1024);
    }
  }
}

// NoPE read bases.  K (A operand of S^T): lane reads row lane % 32 at chunk
// 32 c + 2 kk + h; the xor covers four chunk bits, so the per-lane part takes one
// of eight values (kk % 8) and kk / 8 adds 256 bytes.  V (B operand of P V, read
// transposed): lane 4 r4 + c4 of 16-lane group G addresses row 8 second + 4 h + r4
// at chunk 32 c + 4 ct + 2 (G % 2) + c4 / 2, byte 8 (c4 % 2); the per-lane part
// depends on ct % 4 and ct / 4 adds 256 bytes.
struct ReadBasesN {
  int k[8];
  int v[2][4];
};

__device__ __forceinline__ ReadBasesN read_bases_nope(int c) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  ReadBasesN rb;
  const int r = lane & 31, sw = swzn(r);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int C = 32 * c + 2 * j + h;
    rb.k[j] = r * kNopeRowBytes + (((C & ~15) | ((C & 15) ^ sw)) << 4);
  }
  const int G = lane >> 4, n = lane & 15, r4 = n >> 2, c4 = n & 3;
#pragma unroll
  for (int second = 0; second < 2; ++second) {
    const int row = 8 * second + 4 * h + r4;
    const int sw2 = swzn(row);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int C = 32 * c + 4 * (q & 1) + 8 * (q >> 1) + 2 * (G & 1) + (c4 >> 1);
      rb.v[second][q] = row * kNopeRowBytes + (((C & ~15) | ((C & 15) ^ sw2)) << 4) + 8 * (c4 & 1);
    }
  }
  return rb;
}

// ---- the latent formats ----------------------------------------------------------
// Everything that depends on how a pool row is stored: bf16 (1,152-byte rows, 36 KB
// blocks, a four-slot ring), E4M3 with a per-tensor scale (576-byte rows, 18 KB
// blocks in 20 KB slots, a six-slot ring) or NoPE bf16 (the 512-wide latent alone:
// 1,024-byte rows, 32 KB blocks, a four-slot ring, 16 k-steps per wave).  The
// scores and P V run on bf16 MFMAs in every case: E4M3 operands are widened exactly
// in registers after the LDS read.
struct Bf16Kv {
  static constexpr int kQSteps = kQStepsPerWave;  // MFMA k-steps per wave
  static constexpr bool kLazyMax = true;          // row max only where a reference is due
  static constexpr bool kRopeQ = true;            // queries have a q_rope part
  static constexpr int kStagesN = kStages;        // ring slots
  static constexpr int kSlot = kStageBytes;       // bytes per slot
  static constexpr int kCopies = kStageCopiesPerWave;
  static constexpr int kPageB = kPageBytes;
  static constexpr int kHalfB = kStageBytes;      // a 32-row block of a page
  using Offsets = StageOffsets;
  using Bases = ReadBases;
  static __device__ __forceinline__ Offsets offsets() { return stage_offsets(); }
  static __device__ __forceinline__ Bases bases(int c) { return read_bases(c); }
  static __device__ __forceinline__ void stage(const uint8_t* src, uint8_t* slot, int valid,
                                               const Offsets& so) {
    stage_block(src, slot, valid, so);
  }
  static __device__ __forceinline__ uint32_t dst(const uint8_t* slot) {
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    return lds_addr(slot) + 8 * wave * kRowBytes;
  }
  // query element k of S^T k-step kk for lane half h (natural order)
  static __device__ __forceinline__ int q_k(int c, int kk, int h) {
    return (kQStepsPerWave * c + kk) * 16 + 8 * h;
  }
};

struct E4m3Kv {
  static constexpr int kQSteps = kQStepsPerWave;
  static constexpr bool kLazyMax = false;  // measured slower with the widening VALU
  static constexpr bool kRopeQ = true;
  static constexpr int kStagesN = kStages8;
  static constexpr int kSlot = kSlotBytes8;
  static constexpr int kCopies = kStageCopies8;
  static constexpr int kPageB = kPageBytes8;
  static constexpr int kHalfB = kBlockBytes8;
  using Offsets = StageOffsets8;
  using Bases = ReadBases8;
  static __device__ __forceinline__ Offsets offsets() { return stage_offsets8(); }
  static __device__ __forceinline__ Bases bases(int c) { return read_bases8(c); }
  static __device__ __forceinline__ void stage(const uint8_t* src, uint8_t* slot, int valid,
                                               const Offsets& so) {
    stage_block8(src, slot, valid, so);
  }
  static __device__ __forceinline__ uint32_t dst(const uint8_t* slot) { return stage_dst8(slot); }
  // k order permuted inside each pair of k-steps (see read_bases8)
  static __device__ __forceinline__ int q_k(int c, int kk, int h) {
    return 32 * (kKSteps8 * c + (kk >> 1)) + 16 * h + 8 * (kk & 1);
  }
};

struct NopeKv {
  static constexpr int kQSteps = kNopeQSteps;
  static constexpr bool kLazyMax = true;
  static constexpr bool kRopeQ = false;
  static constexpr int kStagesN = kStages;
  static constexpr int kSlot = kNopeBlockBytes;
  static constexpr int kCopies = kNopeCopies;
  static constexpr int kPageB = kNopePageBytes;
  static constexpr int kHalfB = kNopeBlockBytes;
  using Offsets = StageOffsetsN;
  using Bases = ReadBasesN;
  static __device__ __forceinline__ Offsets offsets() { return stage_offsets_nope(); }
  static __device__ __forceinline__ Bases bases(int c) { return read_bases_nope(c); }
  static __device__ __forceinline__ void stage(const uint8_t* src, uint8_t* slot, int valid,
                                               const Offsets& so) {
    stage_block_nope(src, slot, valid, so);
  }
  static __device__ __forceinline__ uint32_t dst(const uint8_t* slot) {
    return stage_dst_nope(slot);
  }
  static __device__ __forceinline__ int q_k(int c, int kk, int h) {
    return (kNopeQSteps * c + kk) * 16 + 8 * h;
  }
};

// A-operand (K) stream of S^T for one block: operands for k-steps 0..kQSteps-1 in order,
// with LDS reads running ahead of the MFMAs.
template <class Kv> struct KStream;

template <> struct KStream<Bf16Kv> {
  static constexpr int DQ = 4;  // reads in flight
  const uint8_t* blk;
  const ReadBases* rb;
  bf16x8 buf[DQ];
  __device__ __forceinline__ bf16x8 rd(int kk) const {
    return lds_read_b128(blk + rb->k[kk & 3], (kk >> 2) * 128);
  }
  __device__ __forceinline__ void start() {
#pragma unroll
    for (int u = 0; u < DQ; ++u) buf[u] = rd(u);
  }
  __device__ __forceinline__ bf16x8 next(int kk) {
    const bf16x8 a = buf[kk % DQ];
    if (kk + DQ < kQStepsPerWave) buf[kk % DQ] = rd(kk + DQ);
    return a;
  }
};

template <> struct KStream<E4m3Kv> {
  const uint8_t* blk;
  const ReadBases8* rb;
  u32x4 raw[2];  // sixteen-byte reads t and t + 1 (each feeds two k-steps)
  bf16x8 hi;     // the second k-step of the current read
  __device__ __forceinline__ u32x4 rd(int t) const {
    return lds_read_u128(blk + rb->k[t & 1], (t >> 1) * 64);
  }
  __device__ __forceinline__ void start() {
    raw[0] = rd(0);
    raw[1] = rd(1);
  }
  __device__ __forceinline__ bf16x8 next(int kk) {
    if (kk & 1) return hi;
    const int t = kk >> 1;
    const u32x4 w = raw[t & 1];
    if (t + 2 < kKSteps8) raw[t & 1] = rd(t + 2);
    hi = e4m3x8_to_bf16(w[2], w[3]);
    return e4m3x8_to_bf16(w[0], w[1]);
  }
};

// B-operand (V) stream of O = P V for one block: operands for MFMA t, which takes
// k-step ks = (t / 8) ^ F (16 kv rows) and column tile ct = t % 8 of the wave's 256
// columns.  F = 1 runs the block's second k-step first.
template <class Kv, int F> struct VStream;

template <int F> struct VStream<Bf16Kv, F> {
  static constexpr int DV = 4;  // read pairs in flight
  const uint8_t* blk;
  const ReadBases* rb;
  bf16x4 b0[DV], b1[DV];
  __device__ __forceinline__ bf16x4 rd(int t, int sd) const {
    const int ks = (t >> 3) ^ F, ct = t & 7;
    return lds_read_tr(blk + rb->v[sd][ct & 1], (ct >> 1) * 128 + ks * 16 * kRowBytes);
  }
  __device__ __forceinline__ void start() {
#pragma unroll
    for (int u = 0; u < DV; ++u) {
      b0[u] = rd(u, 0);
      b1[u] = rd(u, 1);
    }
  }
  __device__ __forceinline__ bf16x8 next(int t) {
    const int u = t % DV;
    const bf16x8 v = {b0[u][0], b0[u][1], b0[u][2], b0[u][3],
                      b1[u][0], b1[u][1], b1[u][2], b1[u][3]};
    if (t + DV < 2 * kColTilesPerWave) {
      b0[u] = rd(t + DV, 0);
      b1[u] = rd(t + DV, 1);
    }
    return v;
  }
};

template <int F> struct VStream<E4m3Kv, F> {
  static constexpr int DV = 4;  // reads in flight
  const uint8_t* blk;
  const ReadBases8* rb;
  i32x2 raw[DV];
  __device__ __forceinline__ i32x2 rd(int t) const {
    const int ks = (t >> 3) ^ F, ct = t & 7;
    return lds_read_tr8(blk + rb->v[ct & 1], (ct >> 1) * 64 + ks * 16 * kRowBytes8);
  }
  __device__ __forceinline__ void start() {
#pragma unroll
    for (int u = 0; u < DV; ++u) raw[u] = rd(u);
  }
  __device__ __forceinline__ bf16x8 next(int t) {
    const int u = t % DV;
    const i32x2 w = raw[u];
    if (t + DV < 2 * kColTilesPerWave) raw[u] = rd(t + DV);
    return e4m3x8_to_bf16((uint32_t)w[0], (uint32_t)w[1]);
  }
};

template <> struct KStream<NopeKv> {
  static constexpr int DQ = 4;  // reads in flight
  const uint8_t* blk;
  const ReadBasesN* rb;
  bf16x8 buf[DQ];
  __device__ __forceinline__ bf16x8 rd(int kk) const {
    return lds_read_b128(blk + rb->k[kk & 7], (kk >> 3) * 256);
  }
  __device__ __forceinline__ void start() {
#pragma unroll
    for (int u = 0; u < DQ; ++u) buf[u] = rd(u);
  }
  __device__ __forceinline__ bf16x8 next(int kk) {
    const bf16x8 a = buf[kk % DQ];
    if (kk + DQ < kNopeQSteps) buf[kk % DQ] = rd(kk + DQ);
    return a;
  }
};

template <int F> struct VStream<NopeKv, F> {
  static constexpr int DV = 4;  // read pairs in flight
  const uint8_t* blk;
  const ReadBasesN* rb;
  bf16x4 b0[DV], b1[DV];
  __device__ __forceinline__ bf16x4 rd(int t, int sd) const {
    const int ks = (t >> 3) ^ F, ct = t & 7;
    return lds_read_tr(blk + rb->v[sd][ct & 3], (ct >> 2) * 256 + ks * 16 * kNopeRowBytes);
  }
  __device__ __forceinline__ void start() {
#pragma unroll
    for (int u = 0; u < DV; ++u) {
      b0[u] = rd(u, 0);
      b1[u] = rd(u, 1);
    }
  }
  __device__ __forceinline__ bf16x8 next(int t) {
    const int u = t % DV;
    const bf16x8 v = {b0[u][0], b0[u][1], b0[u][2], b0[u][3],
                      b1[u][0], b1[u][1], b1[u][2], b1[u][3]};
    if (t + DV < 2 * kColTilesPerWave) {
      b0[u] = rd(t + DV, 0);
      b1[u] = rd(t + DV, 1);
    }
    return v;
  }
};

// ---- block copies issued from inside the pipeline step -------------------------
// The vector memory path takes a wave's copies of a block only at its own pace
// (hundreds of cycles), so the step issues them one per two S^T MFMAs instead of in
// a burst at the top of the iteration.  A step always issues one block's copies:
// when no whole block is due, the job re-copies the block being scored into its own
// slot (a whole block: only a request's last block can be partial, and it is never
// scored ahead of another block), which writes the bytes already there.
struct CopyJob {
  const uint8_t* src;  // first row of the block in the pool (wave-uniform)
  uint32_t dst;        // LDS address of this wave's share of the block's slot
};

template <class Kv>
__device__ __forceinline__ CopyJob copy_job(const uint8_t* src, uint8_t* slot) {
  return CopyJob{src, Kv::dst(slot)};
}

// ---- the software pipeline --------------------------------------------------------
// Iteration i of a piece runs the softmax step and O += P V of block i while the MFMA
// pipe computes this wave's half of S^T = K Q^T for block i + 1.  A wave pair owns 32
// query rows: each wave scores half of the 576-wide contraction, the halves of a
// block's S^T are swapped through LDS across the iteration barrier, and each wave
// accumulates O for its 256 of the 512 output columns.
//
// LDS operand reads run a fixed distance ahead of the MFMAs that consume them and
// sched_barrier pins the order of the interleaved MFMA, VALU and LDS work, so the
// compiler neither serialises each read with its MFMA nor hoists everything to the top.

// Own half of S^T for one staged block (the pipeline's first block).
template <class Kv>
__device__ __forceinline__ f32x16 qk_partial(const uint8_t* blk, const typename Kv::Bases& rb,
                                             const bf16x8* qreg) {
  KStream<Kv> ks{blk, &rb};
  ks.start();
  f32x16 s0 = {};
#pragma unroll
  for (int kk = 0; kk < Kv::kQSteps; ++kk) {
    s0 = mfma32(ks.next(kk), qreg[kk], s0);
    __builtin_amdgcn_sched_barrier(0);
  }
  return s0;
}

__device__ __forceinline__ void store_partial(f32x4* xs, const f32x16& s) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    xs[j * 64 + lane] = f32x4{s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]};
}

// One iteration.  s_own is this wave's half of block i's S^T (kept in registers) and
// `partner` the other wave's half in LDS.  When HAS_NEXT, this wave's half of block
// i + 1 replaces s_own and its copy in `own` (read by the partner), after a
// workgroup barrier that follows every wave's reads of block i's halves.  `lim` is
// the number of leading rows of block i this lane's query row may see; with a draft
// tree, rows from `drow0` on are draft rows (row drow0 + u is draft u), seen only
// where bit u of `tm` is set (drow0 >= 32 when the block holds no draft row).
//
// Both waves of a pair hold the full scores, but each computes the weights of one
// k-step of P only (C = wave % 2: kv rows 16 C .. 16 C + 15 in accumulator order)
// and hands them to the other through the other's S^T slot, which it has finished
// reading; the barrier after the S^T MFMAs publishes them.  Its own k-step is the
// first of its P V MFMAs, so the other's arrives under them.  Each wave's weight
// sums cover its k-step; the piece's epilogue adds the pair's.
template <bool HAS_NEXT, class Kv, int C>
__device__ __forceinline__ void pipe_step(const uint8_t* blk, const uint8_t* blk_next,
                                          const typename Kv::Bases& rb, const bf16x8* qreg,
                                          f32x16& s_own, f32x4* own, f32x4* partner,
                                          WaveState& ws, int lim, int drow0, uint64_t tm,
                                          float scale_log2, const CopyJob& job,
                                          const typename Kv::Offsets& so, bool full) {
  const int lane = threadIdx.x & 63;
  constexpr int NPV = 2 * kColTilesPerWave;  // 16 MFMAs: 2 k-steps x 8 column tiles
  static_assert(Kv::kQSteps >= 13, "the softmax step takes S^T slots 0..12");

  // `full` (wave-uniform): this block takes the row max, which needs all 32 scores
  // of a row; otherwise only this wave's k-step (S^T registers 8 C .. 8 C + 7) is summed
  f32x4 pr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pr[j] = partner[j * 64 + lane];
  KStream<Kv> kst{blk_next, &rb};
  if constexpr (HAS_NEXT) kst.start();
  __builtin_amdgcn_sched_barrier(0);

  f32x16 x;
  f32x16 n0 = {};
  float m_use = 0.0f, psum = 0.0f, mloc = 0.0f;
  bf16x8 p_own, p_other;  // P for k-step C (computed here) and k-step 1 - C (received)
  VStream<Kv, C> vst{blk, &rb};

  // ---- S^T of block i + 1 on the MFMA pipe, the softmax step of block i in between
#pragma unroll
  for (int kk = 0; kk < Kv::kQSteps; ++kk) {
    if constexpr (HAS_NEXT) {
      n0 = mfma32(kst.next(kk), qreg[kk], n0);
      if ((kk & 1) && (kk >> 1) < Kv::kCopies)
        dma16(job.src, so.off[kk >> 1], job.dst + (kk >> 1) * 1024);
    }
    if (kk == 0) {
      // full scores: own half + partner half (the same sum on both waves of the pair,
      // fp32 addition being commutative); the log2-domain scale is applied below
#pragma unroll
      for (int j = 2 * C; j < 2 * C + 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * j + e] = s_own[4 * j + e] + pr[j][e];
      if (full) {
#pragma unroll
        for (int j = 2 - 2 * C; j < 4 - 2 * C; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * j + e] = s_own[4 * j + e] + pr[j][e];
      }
    } else if (kk == 2) {
      if (__builtin_amdgcn_ballot_w64(lim < kKvBlock || drow0 < kKvBlock)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // branch-free: row r is seen if r < lim and, for a draft row, its bit is set
          const int r = acc_row(lane, i);
          const uint32_t bit = (uint32_t)(tm >> ((r - drow0) & 63)) & 1u;
          const uint32_t ok = (uint32_t)(r < lim) & ((uint32_t)(r < drow0) | bit);
          x[i] = ok ? x[i] : -INFINITY;
        }
      }
    } else if (kk == 4) {
      if (full) {
        // row max (a query row's 32 scores sit in lanes l and l + 32), in the log2
        // domain: scaling by a positive factor commutes with the max, rounding included
        mloc = x[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mloc = fmaxf(mloc, x[i]);
        mloc = pair32_max(mloc) * scale_log2;
        ws.m_seen = fmaxf(ws.m_seen, mloc);
        if (ws.m_ref == -INFINITY) ws.m_ref = mloc;  // a row's first visible block sets it
      }
      m_use = (ws.m_ref == -INFINITY) ? 0.0f : ws.m_ref;
    } else if (kk == 6 || kk == 8) {
      // this wave's k-step: S^T registers 8 C .. 8 C + 7
      const int i0 = 8 * C + (kk == 6 ? 0 : 4);
#pragma unroll
      for (int i = i0; i < i0 + 4; ++i) {
        x[i] = __builtin_amdgcn_exp2f(fmaf(x[i], scale_log2, -m_use));
        psum += x[i];
      }
    } else if (kk == 10) {
      // P as the A operand of O = P V: for k-step ks lane holds query row lane % 32 and
      // S^T registers 8 ks .. 8 ks + 7, i.e. kv rows 16 ks + 4 h + 0..3 and
      // 16 ks + 8 + 4 h + 0..3; the V operand is read in that same kv-row order.  O
      // is later divided by the sum of the rounded weights it was built from, so a
      // row dominated by one key returns that key's c_kv up to fp32 rounding rather
      // than up to bf16 rounding.
      ws.l_run += psum;
      if (!full) ws.p_hi = fmaxf(ws.p_hi, psum);  // every weight is <= its sum
#pragma unroll
      for (int k = 0; k < 8; ++k) p_own[k] = static_cast<__bf16>(x[8 * C + k]);
      // to the other wave: into its S^T slot, whose reads (above) this wave has issued
      // first, and LDS serves a wave's accesses in order
      *reinterpret_cast<bf16x8*>(partner + lane) = p_own;
      // sum of the rounded weights, two at a time (products with 1 are exact)
      const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
      float pbf = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; k += 2)
        pbf = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p_own[k], p_own[k + 1]}, ones, pbf, false);
      ws.l_bf += pbf;
    } else if (kk == 12) {
      vst.start();  // the first V operands of block i (this wave's k-step)
    }
    if (kk == Kv::kQSteps - 1) {
      // the weights are in every slot, and (when HAS_NEXT) block i's halves are read
      __syncthreads();
      p_other = *reinterpret_cast<const bf16x8*>(own + lane);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- O += P V, V = this wave's 256 c_kv columns of block i, read transposed; this
  // wave's k-step first
#pragma unroll
  for (int t = 0; t < NPV; ++t) {
    ws.acc[t & 7] = mfma32(t < 8 ? p_own : p_other, vst.next(t), ws.acc[t & 7]);
    if constexpr (HAS_NEXT) {
      if (t == 8) {  // block i + 1's half is complete; the received weights are read
        store_partial(own, n0);
        s_own = n0;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Normalises this wave's 32 rows x 256 columns and writes them: final O / LSE when
// the piece is the whole request, else a partial slot.  l_tot and l_bf are full row
// sums (per lane, row lane % 32).
__device__ __forceinline__ void write_rows(const SplitArgs& a, const WaveState& ws, float l_tot,
                                           float l_bf, int b, int m_slice, int row_in_tile,
                                           int c, bool whole, int slot) {
  const int lane = threadIdx.x & 63;
  const int M = a.M;
  const bool seen = l_tot > 0.0f;
  // O = kv_scale * sum(P V) / sum(P): an E4M3 pool's scale enters here and in the
  // score scale (1 for bf16)
  const float inv = (seen && l_bf > 0.0f) ? a.kv_scale / l_bf : 0.0f;
  const float lse2 = seen ? ws.m_ref + __builtin_amdgcn_logf(l_tot) : -INFINITY;
  float* base = whole ? a.O + ((size_t)b * M + m_slice) * kNope
                      : a.part_o + ((size_t)slot * a.slot_rows + row_in_tile) * kNope;
  const int col = 256 * c + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = acc_row(lane, i);
    const float inv_i = __shfl(inv, r, 64);
    if (m_slice + r < M) {
      float* rowp = base + (size_t)r * kNope + col;
      // streaming stores: the outputs are not read again by this kernel, and dirty
      // lines left in L2 would be written back at the kernel boundary
#pragma unroll
      for (int ct = 0; ct < kColTilesPerWave; ++ct)
        __builtin_nontemporal_store(ws.acc[ct][i] * inv_i, rowp + 32 * ct);
    }
  }
  if (c == 0 && lane < 32 && m_slice + lane < M) {
    if (whole)
      a.lse[(size_t)b * M + m_slice + lane] = lse2 * kLn2;
    else
      a.part_lse[(size_t)slot * a.slot_rows + row_in_tile + lane] = lse2;
  }
}

// Physical pages of 64 consecutive logical pages of one request, one per lane: a
// wave looks up page pg with a lane read and refills the window on its own (no LDS,
// no barrier).  Out-of-range ids are clamped to page 0 and flagged.
struct PageIds {
  int id;     // lane l: physical page of logical page first + l
  int first;  // wave-uniform
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

// Ring slot of block i.  The byte offset is passed through an empty asm so that the
// compiler keeps it a scalar added to a few per-lane bases, instead of strength-
// reducing i % kStagesN into one loop-carried register per LDS read.
template <class Kv>
__device__ __forceinline__ uint8_t* ring_slot(uint8_t* ring, int i) {
  uint32_t off = (uint32_t)(i % Kv::kStagesN) * Kv::kSlot;
  asm volatile("" : "+s"(off));
  return ring + off;
}

// Pool address of block i of the piece (logical page lo + i / 2, half i % 2) and the
// number of its rows inside the request.
template <class Kv>
__device__ __forceinline__ const uint8_t* block_source(const SplitArgs& a, PageIds& pi, int b,
                                                       int lo, int hi, int L, int i,
                                                       int& valid) {
  const int pg = lo + (i >> 1), half = i & 1;
  if (pg - pi.first >= 64 || pg < pi.first) load_page_ids(a, pi, b, pg, hi);
  const uint32_t phys = __builtin_amdgcn_readlane(pi.id, pg - pi.first);
  valid = min(kKvBlock, L - pg * kPage - half * kKvBlock);
  return reinterpret_cast<const uint8_t*>(a.kv_pool) +
         ((size_t)phys * Kv::kPageB + (size_t)half * Kv::kHalfB);
}

// Waits until at most `sets` blocks' worth of this wave's copies are in flight
// (copies complete in issue order; sets = 0..kMax, larger counts wait for kMax).
template <int kCopies, int kMax>
__device__ __forceinline__ void wait_copy_sets(int sets) {
  static_assert(kCopies * kMax <= 63 && kMax >= 1 && kMax <= 4, "vmcnt immediate");
  if (sets <= 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else if (kMax == 1 || sets == 1) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCopies) : "memory");
  } else if (kMax == 2 || sets == 2) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kCopies) : "memory");
  } else if (kMax == 3 || sets == 3) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * kCopies) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * kCopies) : "memory");
  }
}

// One piece: logical pages [lo, hi) of request b against M-tile mt.  The pages are
// walked as 32-row blocks through a ring of kStagesN slots: while block i is scored
// (softmax, P V) and block i + 1's S^T is computed, blocks i + 2 .. i + kStagesN - 1
// are in flight.
template <class Kv, int C>
__device__ __forceinline__ void run_piece(const SplitArgs& a, uint8_t* ring, f32x4* xbuf, int b,
                                          int L, int mt, int lo, int hi, bool whole, int slot) {
  constexpr int S = Kv::kStagesN;
  constexpr int AHEAD = S - 1;  // blocks copied ahead of the one being scored
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = wave >> 1, c = wave & 1;  // row slice of the M-tile; contraction / column half
  const int M = a.M;
  // drafts of this request: Sq, or q_lens[b] (query slots past it are padding that
  // sees nothing, so its rows come out as O = 0, LSE = -inf)
  int sq = a.Sq;
  if (a.q_lens) {
    // one value per request, kept in a scalar register like the other per-piece
    // bounds (an out-of-range count is reported by the kernel's prologue)
    const int want = __builtin_amdgcn_readfirstlane(a.q_lens[b]);
    sq = min(max(want, 1), min(a.Sq, max(L, 1)));
  }
  const int m_slice = mt * kMTile + p * kRowsPerWave;
  const int m_q = m_slice + (lane & 31);  // the query row this lane scores
  const bool q_ok = m_q < sq * a.H;
  const int t = q_ok ? m_q / a.H : 0;
  const int n_vis = !q_ok ? 0 : (a.causal ? L - sq + t + 1 : L);
  // rows the M-tile's last real query row sees: blocks past it are skipped by every
  // wave (a tile of padding rows sees none)
  const int m_last = min(sq * a.H, (mt + 1) * kMTile) - 1;
  const int n_vis_max = m_last < mt * kMTile ? 0 : (a.causal ? L - sq + m_last / a.H + 1 : L);
  const int nb = max(0, min(2 * (hi - lo), (n_vis_max + kKvBlock - 1) / kKvBlock - 2 * lo));

  // Q^T as the B operand of S^T = K Q^T: lane holds query row m_q, for k-step kk the
  // eight query elements from k = Kv::q_k(c, kk, lane / 32)
  bf16x8 qreg[Kv::kQSteps];
  {
    const int h = lane >> 5;
    const size_t qrow = (size_t)b * M + (q_ok ? m_q : 0);
#pragma unroll
    for (int kk = 0; kk < Kv::kQSteps; ++kk) {
      const int k0 = Kv::q_k(c, kk, h);
      bf16x8 v;
      if (!Kv::kRopeQ || k0 < kNope)
        v = *reinterpret_cast<const bf16x8*>(a.q_nope + qrow * kNope + k0);
      else if constexpr (Kv::kRopeQ)
        v = *reinterpret_cast<const bf16x8*>(a.q_rope + qrow * kRope + (k0 - kNope));
      qreg[kk] = q_ok ? v : bf16x8{};
    }
  }

  WaveState ws;
  ws.m_seen = -INFINITY;
  const typename Kv::Bases rb = Kv::bases(c);
  const typename Kv::Offsets so = Kv::offsets();
  PageIds pi;
  load_page_ids(a, pi, b, lo, hi);
  wait_vmem_all();  // queries and page ids are in before any block copy is counted

  f32x4* own = xbuf + wave * 4 * 64;  // this wave's S^T half (4 x 64 lanes x f32x4)
  f32x4* partner = xbuf + (wave ^ 1) * 4 * 64;
  auto lim_of = [&](int i) { return n_vis - (lo + (i >> 1)) * kPage - (i & 1) * kKvBlock; };
  // draft tree: this lane's ancestor bits (bits above its own draft ignored, its own
  // bit always set) and the block row where draft 0 sits
  uint64_t tm = 0;
  int d_first = 1 << 30;  // no tree: no block holds draft rows
  if (a.tree_mask) {
    d_first = L - sq;
    if (q_ok) tm = (a.tree_mask[(size_t)b * a.Sq + t] & ((2ull << t) - 1ull)) | (1ull << t);
  }
  auto drow_of = [&](int i) {
    const int r = d_first - (lo + (i >> 1)) * kPage - (i & 1) * kKvBlock;
    return a.tree_mask ? r : (1 << 30);
  };
  // copy sets issued after block i + 1's when iteration i starts: the prologue's
  // later blocks plus one set per step (a tail block copied at an iteration's top
  // only adds to that count)
  const int sets_after = min(nb, AHEAD) - 2;

  // At most three passes (rare): pass 0 takes a block's row max only where a row
  // lacks its reference, pass 1 takes every block's, pass 2 starts from the true
  // maxima that pass 1 found.  Formats without the lazy max start at pass 1.
  for (int pass = Kv::kLazyMax ? 0 : 1; pass < 3; ++pass) {
#pragma unroll
    for (int ct = 0; ct < kColTilesPerWave; ++ct) ws.acc[ct] = f32x16{};
    ws.m_ref = pass < 2 ? -INFINITY : ws.m_seen;
    ws.l_run = 0.0f;
    ws.l_bf = 0.0f;
    ws.p_hi = 0.0f;
    // the row max is due where a row has no reference yet and sees rows of the block
    auto full_max = [&](int i) {
      return !Kv::kLazyMax || pass > 0 ||
             __builtin_amdgcn_ballot_w64(ws.m_ref == -INFINITY && lim_of(i) > 0);
    };
    // Block j is copied into ring slot j % S during iteration j - AHEAD (the slot's
    // previous block, j - S, was finished in iteration j - S), its S^T halves are
    // computed in iteration j - 1 and its softmax and P V run in iteration j.  A
    // request's partial last block is copied at the top of iteration j - AHEAD
    // instead.  Prologue: blocks 0 .. AHEAD - 1 in flight, S^T halves of block 0.
    wait_vmem_all();  // no copy of an earlier pass is still landing in the ring
    const uint8_t* srcs[AHEAD];  // pool addresses of blocks i .. i + AHEAD - 1
#pragma unroll
    for (int j = 0; j < AHEAD; ++j) srcs[j] = nullptr;
#pragma unroll
    for (int j = 0; j < AHEAD; ++j) {
      if (j < nb) {
        int valid;
        srcs[j] = block_source<Kv>(a, pi, b, lo, hi, L, j, valid);
        Kv::stage(srcs[j], ring_slot<Kv>(ring, j), valid, so);
      }
    }
    wait_copy_sets<Kv::kCopies, AHEAD - 1>(min(nb, AHEAD) - 1);  // block 0 has landed
    __syncthreads();
    if (a.wg_time && threadIdx.x == 0 && pass == (Kv::kLazyMax ? 0 : 1))  // block 0 is in LDS
      a.wg_time[5 * (size_t)blockIdx.x + 2] = (int64_t)wall_clock64();
    f32x16 s_own = {};  // this wave's half of S^T of the block being scored
    if (nb > 0) {
      s_own = qk_partial<Kv>(ring_slot<Kv>(ring, 0), rb, qreg);
      store_partial(own, s_own);
    }
    int i = 0;
    for (; i + 1 < nb; ++i) {
      wait_copy_sets<Kv::kCopies, AHEAD - 2>(sets_after);  // block i + 1 has landed ...
      // ... in every wave; both S^T halves of block i are in LDS; every wave is done
      // with block i - 1, whose slot now receives block i + AHEAD
      __syncthreads();
      CopyJob job = copy_job<Kv>(srcs[0], ring_slot<Kv>(ring, i));  // same-data re-copy
      const uint8_t* src_new = nullptr;
      if (i + AHEAD < nb) {
        int valid;
        src_new = block_source<Kv>(a, pi, b, lo, hi, L, i + AHEAD, valid);
        if (valid == kKvBlock)
          job = copy_job<Kv>(src_new, ring_slot<Kv>(ring, i + AHEAD));
        else
          Kv::stage(src_new, ring_slot<Kv>(ring, i + AHEAD), valid, so);
      }
      pipe_step<true, Kv, C>(ring_slot<Kv>(ring, i), ring_slot<Kv>(ring, i + 1), rb, qreg,
                             s_own, own, partner, ws, lim_of(i), drow_of(i), tm, a.scale_log2,
                             job, so, full_max(i));
#pragma unroll
      for (int j = 0; j + 1 < AHEAD; ++j) srcs[j] = srcs[j + 1];
      srcs[AHEAD - 1] = src_new;
    }
    if (i < nb) {  // the last block (already in LDS): nothing left to score ahead or copy
      __syncthreads();
      pipe_step<false, Kv, C>(ring_slot<Kv>(ring, i), nullptr, rb, qreg, s_own, own, partner,
                              ws, lim_of(i), drow_of(i), tm, a.scale_log2, CopyJob{}, so,
                              full_max(i));
    }
    // a row whose scores outgrew its reference by more than the lazy bound (or a
    // weight sum past it, in a block without the max) forces another pass for the
    // whole workgroup; the flag lives in the exchange buffer
    const bool broke = (ws.m_ref != -INFINITY && ws.m_seen > ws.m_ref + kLazyRescale) ||
                       ws.p_hi > kLazyWeight;
    int* redo_flag = reinterpret_cast<int*>(xbuf);
    __syncthreads();  // every wave is done with the ring and the exchange buffer
    if (threadIdx.x == 0) *redo_flag = 0;
    __syncthreads();
    if (__builtin_amdgcn_ballot_w64(broke) && lane == 0) *redo_flag = 1;
    __syncthreads();
    const bool redo = *redo_flag != 0;
    __syncthreads();  // the flag has been read before the buffer is reused
    if (!redo) break;
  }

  if (a.wg_time && threadIdx.x == 0)  // the walk (and any re-walk) is over
    a.wg_time[5 * (size_t)blockIdx.x + 3] = (int64_t)wall_clock64();
  // the pair's weight sums: each wave summed the weights of its own k-step of P.  Both
  // waves add them in the same order (the C = 0 wave's first), so both normalise their
  // columns by the same sums.
  f32x2* sums = reinterpret_cast<f32x2*>(xbuf);  // free: every wave is past the last use
  sums[wave * 64 + lane] = f32x2{ws.l_run, ws.l_bf};
  __syncthreads();
  const f32x2 other = sums[(wave ^ 1) * 64 + lane];
  const float l_run = C == 0 ? ws.l_run + other[0] : other[0] + ws.l_run;
  const float l_bf = C == 0 ? ws.l_bf + other[1] : other[1] + ws.l_bf;
  write_rows(a, ws, pair32_sum(l_run), pair32_sum(l_bf), b, m_slice, p * kRowsPerWave, c,
             whole, slot);
}

// ---- combine ---------------------------------------------------------------------
// The partials of a split request are merged by their log-sum-exp.  The same row
// merges serve the separate combine kernels (after the split-KV kernel) and the
// single-pass kernel, whose workgroups past the split-KV ones wait for the pieces of
// their request first.

// Single pass: a merge waits until `expected` pieces of its (request, M-tile) have
// published their partials.  The split-KV workgroups never wait and, launched ahead
// of every merging workgroup of the grid, are all dispatched before any merging one;
// so every awaited piece runs.  The wait is still bounded (kMergeWaitTicks of the
// constant 100 MHz clock): past it the merge raises kFlagMergeWait and proceeds.
constexpr uint64_t kMergeWaitTicks = 100000000ull;  // one second

__device__ __forceinline__ void wait_pieces(const uint32_t* ctr, uint32_t expected,
                                            uint32_t* flags) {
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < expected) {
    __builtin_amdgcn_s_sleep(4);
    if (wall_clock64() - t0 > kMergeWaitTicks) {
      atomicOr(flags, kFlagMergeWait);
      break;
    }
  }
}

// Non-empty partitions among g0..g1: the pieces of a request that spans them.
__device__ __forceinline__ uint32_t pieces_of(int64_t T, int G, int g0, int g1, bool dense) {
  if (dense) return (uint32_t)(g1 - g0 + 1);
  uint32_t n = 0;
  for (int g = g0; g <= g1; ++g) n += part_begin(T, G, g) < part_begin(T, G, g + 1) ? 1u : 0u;
  return n;
}

// Single pass: one more row of M-tile (b, mt) is merged; the last of its rows
// returns both counters to zero for the next call (every merge of the tile has
// finished waiting by then).
__device__ __forceinline__ void row_merged(const CombineArgs& a, int idx, int mt) {
  const uint32_t rows = (uint32_t)min(a.M - mt * a.MT, a.MT);
  if (atomicAdd(a.done + idx, 1u) + 1u == rows) {
    atomicExch(a.arrive + idx, 0u);
    atomicExch(a.done + idx, 0u);
  }
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; ++w) r += red[w];
  return r;
}

// Many pieces per request (G >= 16 B): one workgroup merges folded query row `row`
// = (b, m), all 512 columns (half < 0) or one half of them (half = 0 or 1; the
// separate combine kernel runs two workgroups per row).  Thread t handles the pieces
// s with s % 4 == t / 64 and the four-column groups 4 (t % 64) and 256 + 4 (t % 64)
// (only the one in its half when half >= 0), so that each load instruction of a wave
// reads 1 KB of one partial row contiguously.  The partial outputs of a chunk of 64
// pieces (16 per thread) are all requested at once, before the row's log-sum-exp over
// the pieces is reduced, so that one memory round trip covers both; the four piece
// lanes are summed through LDS.  Every column is summed in the same order whatever
// `half` is.  prefix: kMaxBatch + 1 ints, red: 4 floats, part: 4 x 512 floats.
constexpr int kCombineLanes = kCombineThreads / 64;
constexpr int kCombineChunk = 16;  // pieces per thread per chunk

__device__ __forceinline__ void merge_row_group(const CombineArgs& a, int row, int* prefix,
                                                float* red, float* part, int half = -1) {
  build_page_prefix(a.seq_lens, a.B, a.Sq, a.max_pages, prefix, a.flags, false);
  const int64_t T = prefix[a.B];
  const int b = row / a.M, m = row - b * a.M;
  const int pb0 = prefix[b], pb1 = prefix[b + 1];
  if (pb1 <= pb0) return;
  const int g0 = part_of(T, a.G, pb0);
  const int g1 = part_of(T, a.G, pb1 - 1);
  if (g0 == g1) return;  // one partition held the whole request: already final
  const int mt = m / a.MT, ml = m - mt * a.MT;
  const int n = g1 - g0 + 1;
  // Partitions g0..g1 hold the request's pieces.  With more partitions than pages
  // some partitions are empty; they wrote nothing and carry no weight.  With at
  // least one page per partition (G <= T) none is empty and the 64-bit divisions
  // that find empty ones are skipped.
  const bool dense = (int64_t)a.G <= T;
  const int idx = b * a.n_mt + mt;
  if (a.arrive) {
    // acquire: one fence invalidates this CU's L1 and the XCD's L2 for all waves, and
    // the barrier orders it before every wave's reads of the partials
    if (threadIdx.x == 0) {
      wait_pieces(a.arrive + idx, pieces_of(T, a.G, g0, g1, dense), a.flags);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
  }
  auto lse_of = [&](int s) {
    const int g = g0 + s;
    if (!dense && part_begin(T, a.G, g) >= part_begin(T, a.G, g + 1)) return -INFINITY;
    const size_t slot = (size_t)(b + g) * a.n_mt + mt;
    return a.part_lse[slot * a.slot_rows + ml];
  };
  const int tid = threadIdx.x;
  const int cg = tid & 63, pl = tid >> 6;
  auto src_of = [&](int s) {
    const size_t slot = (size_t)(b + g0 + s) * a.n_mt + mt;
    return a.part_o + (slot * a.slot_rows + ml) * kNope + 4 * cg +
           (half > 0 ? kNope / 2 : 0);
  };

  f32x4 v0[kCombineChunk], v1[kCombineChunk];
  float lv[kCombineChunk];
  auto load_chunk = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kCombineChunk; ++u) {
      const int s = s0 + pl + kCombineLanes * u;
      lv[u] = -INFINITY;
      if (s < n) {
        const float* src = src_of(s);
        v0[u] = *reinterpret_cast<const f32x4*>(src);
        if (half < 0) v1[u] = *reinterpret_cast<const f32x4*>(src + kNope / 2);
        lv[u] = lse_of(s);
      }
    }
  };
  load_chunk(0);

  // the row's log2-sum-exp2 over its pieces
  float mx = -INFINITY;
  for (int s = tid; s < n; s += kCombineThreads) mx = fmaxf(mx, lse_of(s));
  mx = block_max(mx, red);
  float tot = 0.0f;
  if (mx != -INFINITY)
    for (int s = tid; s < n; s += kCombineThreads) tot += exp2f(lse_of(s) - mx);
  tot = block_sum(tot, red);
  const bool seen = tot > 0.0f;
  const float lse2 = seen ? mx + log2f(tot) : -INFINITY;

  f32x4 o0 = {}, o1 = {};
  auto accumulate = [&]() {
#pragma unroll
    for (int u = 0; u < kCombineChunk; ++u) {
      const float w = (seen && lv[u] != -INFINITY) ? exp2f(lv[u] - lse2) : 0.0f;
      // a zero-weight slot may hold stale data, even NaN: select, never multiply
      o0 = w != 0.0f ? o0 + w * v0[u] : o0;
      if (half < 0) o1 = w != 0.0f ? o1 + w * v1[u] : o1;
    }
  };
  accumulate();
  for (int s0 = kCombineLanes * kCombineChunk; s0 < n; s0 += kCombineLanes * kCombineChunk) {
    load_chunk(s0);
    accumulate();
  }

  *reinterpret_cast<f32x4*>(&part[pl * 512 + 4 * cg]) = o0;
  *reinterpret_cast<f32x4*>(&part[pl * 512 + 4 * cg + 256]) = o1;
  __syncthreads();
  if (pl == 0) {
#pragma unroll
    for (int q = 1; q < kCombineLanes; ++q) {
      o0 += *reinterpret_cast<const f32x4*>(&part[q * 512 + 4 * cg]);
      o1 += *reinterpret_cast<const f32x4*>(&part[q * 512 + 4 * cg + 256]);
    }
    float* dst = a.O + ((size_t)b * a.M + m) * kNope + 4 * cg +
                 (half > 0 ? kNope / 2 : 0);
    *reinterpret_cast<f32x4*>(dst) = o0;
    if (half < 0) *reinterpret_cast<f32x4*>(dst + kNope / 2) = o1;
    if (cg == 0 && half <= 0) a.lse[(size_t)b * a.M + m] = lse2 * kLn2;
  }
  if (a.arrive && tid == 0) row_merged(a, idx, mt);
}

// Few pieces per request: one wave merges folded query row `row`, with no LDS and no
// barriers.  The wave finds its request's page range by summing the clamped page
// counts itself, reduces the row's log-sum-exp over the pieces with lane shuffles,
// and lane l accumulates columns 4 l .. 4 l + 3 and 256 + 4 l .. 256 + 4 l + 3 over
// all pieces (each load instruction reads 1 KB of a partial row contiguously), four
// pieces' loads in flight at a time.
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}
__device__ __forceinline__ float wave_sumf(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

__device__ __forceinline__ void merge_row_wave(const CombineArgs& a, int64_t row) {
  const int lane = threadIdx.x & 63;
  const int b = (int)(row / a.M), m = (int)(row - (int64_t)b * a.M);
  int below = 0, total = 0;
  for (int j = lane; j < a.B; j += 64) {
    const int L = clamp_len(a.seq_lens[j], a.Sq, a.max_pages, a.flags, false);
    const int pages = (L + kPage - 1) / kPage;
    total += pages;
    if (j < b) below += pages;
  }
  const int64_t T = wave_sum(total);
  const int Lb = clamp_len(a.seq_lens[b], a.Sq, a.max_pages, a.flags, false);
  const int pb0 = wave_sum(below), pb1 = pb0 + (Lb + kPage - 1) / kPage;
  if (pb1 <= pb0) return;
  const int g0 = part_of(T, a.G, pb0);
  const int g1 = part_of(T, a.G, pb1 - 1);
  if (g0 == g1) return;  // one partition held the whole request: already final
  const int mt = m / a.MT, ml = m - mt * a.MT;
  const int n = g1 - g0 + 1;
  const bool dense = (int64_t)a.G <= T;  // then no partition is empty
  const int idx = b * a.n_mt + mt;
  if (a.arrive) {
    if (lane == 0) wait_pieces(a.arrive + idx, pieces_of(T, a.G, g0, g1, dense), a.flags);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the partials are read after this
  }
  auto lse_of = [&](int s) {
    const int g = g0 + s;
    if (!dense && part_begin(T, a.G, g) >= part_begin(T, a.G, g + 1)) return -INFINITY;
    const size_t slot = (size_t)(b + g) * a.n_mt + mt;
    return a.part_lse[slot * a.slot_rows + ml];
  };
  float mx = -INFINITY;
  for (int s = lane; s < n; s += 64) mx = fmaxf(mx, lse_of(s));
  mx = wave_max(mx);
  float tot = 0.0f;
  if (mx != -INFINITY)
    for (int s = lane; s < n; s += 64) tot += exp2f(lse_of(s) - mx);
  tot = wave_sumf(tot);
  const bool seen = tot > 0.0f;
  const float lse2 = seen ? mx + log2f(tot) : -INFINITY;

  f32x4 o0 = {}, o1 = {};
  constexpr int U = 4;
  for (int s0 = 0; s0 < n; s0 += U) {
    f32x4 v0[U], v1[U];
    float w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u;
      w[u] = 0.0f;
      if (s < n) {
        const size_t slot = (size_t)(b + g0 + s) * a.n_mt + mt;
        const float* src = a.part_o + (slot * a.slot_rows + ml) * kNope + 4 * lane;
        v0[u] = *reinterpret_cast<const f32x4*>(src);
        v1[u] = *reinterpret_cast<const f32x4*>(src + kNope / 2);
        const float l = lse_of(s);
        w[u] = (seen && l != -INFINITY) ? exp2f(l - lse2) : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // a zero-weight slot may hold stale data, even NaN: select, never multiply
      o0 = w[u] != 0.0f ? o0 + w[u] * v0[u] : o0;
      o1 = w[u] != 0.0f ? o1 + w[u] * v1[u] : o1;
    }
  }
  float* dst = a.O + ((size_t)b * a.M + m) * kNope + 4 * lane;
  *reinterpret_cast<f32x4*>(dst) = o0;
  *reinterpret_cast<f32x4*>(dst + kNope / 2) = o1;
  if (lane == 0) {
    a.lse[(size_t)b * a.M + m] = lse2 * kLn2;
    if (a.arrive) row_merged(a, idx, mt);
  }
}

// The merge arguments of a single-pass call.
__device__ __forceinline__ CombineArgs merge_args(const SplitArgs& s) {
  CombineArgs a;
  a.seq_lens = s.seq_lens;
  a.O = s.O;
  a.lse = s.lse;
  a.part_o = s.part_o;
  a.part_lse = s.part_lse;
  a.flags = s.flags;
  a.arrive = s.arrive;
  a.done = s.done;
  a.max_pages = s.max_pages;
  a.B = s.B;
  a.Sq = s.Sq;
  a.H = s.H;
  a.M = s.M;
  a.n_mt = s.n_mt;
  a.G = s.G;
  a.MT = kMTile;
  a.slot_rows = s.slot_rows;
  return a;
}

// Merging workgroup w of a single-pass call: row w (comb_rows == 0), or rows
// (4 w + wave) comb_rows .. + comb_rows, one wave each.
__device__ __forceinline__ void merge_role(const SplitArgs& s, int w, uint8_t* lds) {
  const CombineArgs a = merge_args(s);
  if (s.comb_rows == 0) {
    int* prefix = reinterpret_cast<int*>(lds);
    float* red = reinterpret_cast<float*>(lds + 8192);
    float* part = reinterpret_cast<float*>(lds + 8192 + 256);
    merge_row_group(a, w, prefix, red, part);
  } else {
    const int64_t rows = (int64_t)a.B * a.M;
    const int64_t r0 = ((int64_t)w * kWaves + (threadIdx.x >> 6)) * s.comb_rows;
    for (int64_t r = r0; r < r0 + s.comb_rows && r < rows; ++r) merge_row_wave(a, r);
  }
}

template <class Kv>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
splitkv_kernel(SplitArgs a) {
  // bf16: 4 x 36 KB ring + 16 KB exchange buffer = the whole 160 KB of LDS;
  // E4M3: 6 x 20 KB ring + 16 KB
  __shared__ __attribute__((aligned(16))) uint8_t ring[Kv::kStagesN * Kv::kSlot];
  __shared__ f32x4 xbuf[kWaves * 4 * 64];  // S^T halves exchanged by wave pairs
  static_assert(sizeof(f32x4) * kWaves * 4 * 64 >= (2 * kMaxBatch + 1) * sizeof(int),
                "the page prefix and lengths are built in the exchange buffer");

  if ((int)blockIdx.x >= a.n_split) {  // single pass: a merging workgroup
    merge_role(a, (int)blockIdx.x - a.n_split, ring);
    return;
  }
  // With several partitions, the M-tiles of one partition (and neighbouring
  // partitions) share an XCD and its L2.  With one partition every M-tile walks the
  // same pages anyway; launch order then spreads the causally longer last M-tiles
  // over all eight XCDs, heaviest first, instead of giving them all to one.
  const int lam = a.G > 1 ? xcd_logical_id(blockIdx.x, a.n_split)
                          : a.n_split - 1 - (int)blockIdx.x;
  const int g = lam / a.n_mt;
  const int mt = lam - g * a.n_mt;
  int64_t* tl = a.wg_time ? a.wg_time + 5 * (size_t)blockIdx.x : nullptr;
  if (tl && threadIdx.x == 0) tl[0] = (int64_t)wall_clock64();
  if (a.wg_trace && threadIdx.x == 0) {
    // where this workgroup actually runs: the XCC id register of the executing die
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(xcc));
    int32_t* rec = a.wg_trace + 3 * (size_t)blockIdx.x;
    rec[0] = (int32_t)xcc;
    rec[1] = g;
    rec[2] = mt;
  }

  // page prefix and clamped lengths of the batch, in the exchange buffer until the
  // first piece starts
  int* prefix = reinterpret_cast<int*>(xbuf);
  int* lens = prefix + kMaxBatch + 1;
  build_page_prefix(a.seq_lens, a.B, a.len_min, a.max_pages, prefix, a.flags, true, lens);
  if (tl && threadIdx.x == 0) tl[1] = (int64_t)wall_clock64();
  if (a.q_lens && threadIdx.x < 64) {  // per-request draft counts outside [1, min(Sq, L_b)]
    for (int j = threadIdx.x; j < a.B; j += 64) {
      const int q = a.q_lens[j];
      if (q < 1 || q > min(a.Sq, lens[j])) atomicOr(a.flags, kFlagBadSeqLen);
    }
  }
  const int64_t T = prefix[a.B];
  const int64_t p0 = part_begin(T, a.G, g);
  const int64_t p1 = part_begin(T, a.G, g + 1);
  // first request whose pages reach past p0
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid + 1] > p0) hi = mid; else lo = mid + 1;
  }
  int pb0 = prefix[lo];
  const int L_first = lens[lo];
  __syncthreads();  // the prefix has been read
  if (p0 >= p1) return;

  // walk the requests the partition touches; a request's page count is recomputed
  // from its clamped length (the same count the prefix was built from)
  for (int b = lo; b < a.B && pb0 < p1; ++b) {
    const int Lb = b == lo ? L_first : clamp_len(a.seq_lens[b], a.len_min, a.max_pages, a.flags,
                                                  false);
    const int pb1 = pb0 + (Lb + kPage - 1) / kPage;
    if (pb1 > pb0) {
      const int plo = (int)((p0 > pb0 ? p0 : pb0) - pb0);
      const int phi = (int)((p1 < pb1 ? p1 : pb1) - pb0);
      const bool whole = plo == 0 && phi == pb1 - pb0;
      // the two waves of a pair run the two k-step halves of P (wave-uniform branch)
      if ((threadIdx.x >> 6) & 1)
        run_piece<Kv, 1>(a, ring, xbuf, __builtin_amdgcn_readfirstlane(b),
                         __builtin_amdgcn_readfirstlane(Lb), mt,
                         __builtin_amdgcn_readfirstlane(plo), __builtin_amdgcn_readfirstlane(phi),
                         whole, (b + g) * a.n_mt + mt);
      else
        run_piece<Kv, 0>(a, ring, xbuf, __builtin_amdgcn_readfirstlane(b),
                         __builtin_amdgcn_readfirstlane(Lb), mt,
                         __builtin_amdgcn_readfirstlane(plo), __builtin_amdgcn_readfirstlane(phi),
                         whole, (b + g) * a.n_mt + mt);
      if (a.arrive && !whole) {
        // single pass: every wave's partial stores have reached L2 before the barrier;
        // one release fence then writes the XCD's L2 back (it covers all four waves)
        // before the piece is counted
        wait_vmem_all();
        __syncthreads();
        if (threadIdx.x == 0) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          atomicAdd(a.arrive + b * a.n_mt + mt, 1u);
        }
      }
      __syncthreads();  // LDS free before the next piece stages into it
    }
    pb0 = pb1;
  }
  if (tl) {  // every store of the workgroup is complete
    wait_vmem_all();
    __syncthreads();
    if (threadIdx.x == 0) tl[4] = (int64_t)wall_clock64();
  }
}

// ---- the separate combine kernels (two-pass calls) ----------------------------------
// two workgroups per row, one per half of the columns
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(CombineArgs a) {
  __shared__ int prefix[kMaxBatch + 1];
  __shared__ float red[kCombineLanes];
  __shared__ __attribute__((aligned(16))) float part[kCombineLanes * 512];
  merge_row_group(a, blockIdx.x >> 1, prefix, red, part, blockIdx.x & 1);
}

// four rows per workgroup, one wave each
constexpr int kRowsPerCombineGroup = kCombineThreads / 64;

__global__ void __launch_bounds__(kCombineThreads) combine_rows_kernel(CombineArgs a) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerCombineGroup + (threadIdx.x >> 6);
  if (row >= (int64_t)a.B * a.M) return;  // the whole wave
  merge_row_wave(a, row);
}

hipError_t launch_splitkv(const SplitArgs& a, hipStream_t stream) {
  const int64_t n_split = (int64_t)a.G * a.n_mt;
  int64_t nwg = n_split;
  if (a.arrive) {  // single pass: the merging workgroups follow the split-KV ones
    const int64_t rows = (int64_t)a.B * a.M;
    const int64_t per = (int64_t)kWaves * a.comb_rows;
    nwg += a.comb_rows == 0 ? rows : (rows + per - 1) / per;
  }
  if (n_split != a.n_split || nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidValue;
  if (a.kv_nope)
    hipLaunchKernelGGL(splitkv_kernel<NopeKv>, dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
  else if (a.kv_e4m3)
    hipLaunchKernelGGL(splitkv_kernel<E4m3Kv>, dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(splitkv_kernel<Bf16Kv>, dim3((unsigned)nwg), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// Zeroes n words: the single-pass arrival and merged-row counters, before each
// single-pass launch (a kernel rather than a memset node, so that a captured graph
// replays it like any other launch).
__global__ void __launch_bounds__(256) clear_words_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_clear_words(uint32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t groups = (n + 255) / 256;
  if (groups > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(clear_words_kernel, dim3((unsigned)groups), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.M;
  if (rows <= 0 || rows > 0x7fffffff) return hipErrorInvalidValue;
  // about G / B pieces per request: spread many over two workgroups, few over a wave
  if ((int64_t)a.G >= 16 * (int64_t)a.B) {
    if (rows > 0x3fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(2 * rows)), dim3(kCombineThreads), 0,
                       stream, a);
  } else {
    const int64_t groups = (rows + kRowsPerCombineGroup - 1) / kRowsPerCombineGroup;
    hipLaunchKernelGGL(combine_rows_kernel, dim3((unsigned)groups), dim3(kCombineThreads), 0,
                       stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla
