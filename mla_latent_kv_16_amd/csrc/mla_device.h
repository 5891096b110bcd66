// Device-side building blocks of the gfx950 MLA kernels: tile geometry, the LDS
// layout of a staged KV page, MFMA and LDS-transpose wrappers, cross-lane
// reductions, and the KV partition plan shared by the split-KV and combine passes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// ---- problem geometry -------------------------------------------------------
constexpr int kNope = 512;                     // latent c_kv width (also the value width)
constexpr int kRope = 64;                      // decoupled RoPE key width
constexpr int kRow = kNope + kRope;            // one cached latent row: 576 bf16
constexpr int kPage = 64;                      // rows per page
constexpr int kRowBytes = kRow * 2;            // 1152
constexpr int kChunks = kRowBytes / 16;        // 72 sixteen-byte chunks per row
constexpr int kPageBytes = kPage * kRowBytes;  // 73,728
constexpr int kMaxBatch = 1024;
constexpr uint32_t kFlagBadSeqLen = 1u;
constexpr uint32_t kFlagBadPageId = 2u;
constexpr uint32_t kFlagMergeWait = 4u;  // a merge gave up waiting for its pieces
constexpr int kHeaderBytes = 256;

// Split-KV pass: a workgroup is 4 waves and covers an M-tile of 64 folded query
// rows.  Waves 2 p and 2 p + 1 own rows 32 p .. 32 p + 31 (one column block of
// v_mfma_f32_32x32x16_bf16); wave 2 p + c scores contraction half c of the 576-wide
// rows and accumulates output columns 256 c .. 256 c + 255.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kMTile = 64;
constexpr int kKvBlock = 32;                       // kv rows per MFMA block (S^T tile rows)
constexpr int kQStepsPerWave = kRow / 16 / 2;      // 18 MFMA k-steps: half the 576-wide row
constexpr int kColTilesPerWave = kNope / 32 / 2;   // 8 output column tiles of 32
constexpr int kStageBytes = kKvBlock * kRowBytes;  // 36,864: half a page
constexpr int kStages = 4;                         // LDS ring depth (two blocks in flight)
constexpr int kStageCopiesPerWave = 9;             // 16-byte-per-lane copies per wave per block
constexpr int kCombineThreads = 256;

// E4M3 latent pools (one byte per element): a row is 576 bytes, a page 36,864 and a
// 32-row block 18,432 = 1,152 sixteen-byte chunks.  Each wave copies 5 KB of a block
// (4 x 5 KB = the block plus 2 KB of padding at the end of its slot), and the ring
// has six slots, so four blocks are in flight while two are being scored.
constexpr int kRowBytes8 = kRow;                               // 576
constexpr int kPageBytes8 = kPage * kRowBytes8;                // 36,864
constexpr int kChunks8 = kRowBytes8 / 16;                      // 36
constexpr int kBlockBytes8 = kKvBlock * kRowBytes8;            // 18,432
constexpr int kBlockChunks8 = kBlockBytes8 / 16;               // 1,152
constexpr int kStageCopies8 = 5;                               // 1 KB copies per wave per block
constexpr int kSlotBytes8 = kWaves * kStageCopies8 * 1024;     // 20,480
constexpr int kStages8 = 6;
constexpr int kKSteps8 = kQStepsPerWave / 2;                   // 9 sixteen-byte K reads per wave

// NoPE-MLA pools: rows are the 512-wide latent alone (1,024 bf16 bytes, 64 chunks).
constexpr int kNopeRowBytes = kNope * 2;                       // 1,024
constexpr int kNopePageBytes = kPage * kNopeRowBytes;          // 65,536
constexpr int kNopeBlockBytes = kKvBlock * kNopeRowBytes;      // 32,768: half a page
constexpr int kNopeCopies = kNopeBlockBytes / kWaves / 1024;   // 8 copies of 1 KB per wave
constexpr int kNopeQSteps = kNope / 16 / 2;                    // 16 MFMA k-steps per wave

// NoPE rows: 16-byte chunk c of row r sits at chunk position c ^ swzn(r), the xor
// touching the low four chunk bits.  Every 1,024-byte row starts on the same bank,
// so the xor value must differ across any 16 consecutive rows (the sixteen-byte K
// reads of 16 rows) and across the 4 rows of a transposed V read: the 4-bit row
// index rotated by two does both.
__device__ __forceinline__ int swzn(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// ---- LDS layout of one staged page ------------------------------------------
// Row r of the page occupies bytes [r * 1152, (r + 1) * 1152).  Its sixteen-byte
// chunk c sits at chunk position c ^ swz(r); the xor only touches the low three
// bits, so a chunk never leaves its aligned group of eight (72 = 9 * 8).  With 64
// four-byte banks, rows r and r + 1 start half a bank row apart, and swz spreads
// (a) the 16 rows a quarter-wave of ds_read_b128 reads at one chunk and (b) the
// 4 rows x 4 chunks a half-wave of ds_read_b64_tr_b16 reads over distinct banks.
__device__ __forceinline__ int swz(int r) {
  const int i = (r >> 1) & 7;  // index among same-parity rows of a 16-row block
  return ((i & 1) << 2) | (i & 2) | ((i >> 2) & 1);  // 3-bit bit reversal
}

// E4M3 rows: 16-byte chunk c of row r sits at chunk position c ^ swz8(r).  The xor
// only touches the low two chunk bits (a row's 36 chunks are nine aligned groups of
// four).  With 576-byte rows (9 x 64 bytes) the bank of a chunk repeats every four
// rows; swz8 takes bits 2 and 3 of the row so that the sixteen-byte K reads of 16
// consecutive rows and the transposed V reads (8 rows x 2 chunks per 32 lanes) hit
// distinct 16-byte bank groups.
__device__ __forceinline__ int swz8(int r) {
  return ((r >> 2) & 1) | ((((r >> 3) ^ (r >> 2)) & 1) << 1);
}

// ---- instruction wrappers ---------------------------------------------------
// 32x32x16 bf16 MFMA.  A [32 x 16]: lane l holds row l % 32, k = 8 (l / 32) + 0..7.
// B [16 x 32]: lane l holds column l % 32, the same k.  D [32 x 32]: lane l holds
// column l % 32 and rows 4 (l / 32) + 8 q + c in register 4 q + c.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const uint8_t* lds_base, int byte_off) {
  return *reinterpret_cast<const bf16x8*>(lds_base + byte_off);
}
__device__ __forceinline__ u32x4 lds_read_u128(const uint8_t* lds_base, int byte_off) {
  return *reinterpret_cast<const u32x4*>(lds_base + byte_off);
}

// LDS transpose read (gfx950): within each group of 16 lanes, when lane 4 r + c
// addresses the 8-byte word at columns [4 c, 4 c + 4) of row r (r, c = 0..3), lane n
// of the group receives column n of rows 0..3: the k-contiguous operand an MFMA
// needs from a row-major tile.
__device__ __forceinline__ bf16x4 lds_read_tr(const uint8_t* lds_base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(lds_base + byte_off));
}

// LDS transpose read of 8-bit data (gfx950): within each group of 16 lanes, lane n
// receives byte n % 8 of the 8-byte words addressed by lanes 2 j + n / 8, j = 0..7.
// When lane 2 j + e addresses columns [8 e, 8 e + 8) of row j, lane n gets column n
// of rows 0..7: eight consecutive k of one column, as an MFMA operand wants them.
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* lds_base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(lds_base + byte_off));
}

// Eight E4M3 codes (bytes 0..7 of w0, w1) to eight bf16 values, exactly: every E4M3
// value is a bf16 value (scale factor 1).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct global -> LDS copy of 16 bytes per lane: lane l reads sbase + voff and
// writes LDS bytes [lds + 16 l, lds + 16 l + 16).  sbase and lds are wave-uniform.
// Issued as inline asm so that the compiler does not tie later LDS reads of the
// *other* ring slots to these copies (it would wait for every copy in flight);
// completion is awaited explicitly with wait_vmem_all() before the barrier that
// publishes a slot.  The LDS address travels in M0: the operand is bound to M0 with
// a register constraint, so the compiler writes M0 itself and knows it is taken.  A
// write of M0 needs one wait state before a global load with the LDS bit reads it
// (the s_nop).  The base and the LDS address are passed through readfirstlane (as
// unsigned 32-bit halves) so that they are scalar operands even where the compiler
// cannot prove them uniform.
__device__ __forceinline__ void dma16(const void* sbase_in, uint32_t voff, uint32_t lds_in) {
  const uint64_t p = reinterpret_cast<uint64_t>(sbase_in);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  const void* sbase = reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_in);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "{m0}"(lds)
               : "memory");
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// v_permlane32_swap(x, x) leaves x[l % 32] in the first result and x[32 + l % 32]
// in the second, on every lane: the two halves of a 32x32 MFMA column.
__device__ __forceinline__ float pair32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- KV partition plan -------------------------------------------------------
// The batch's pages are concatenated in request order (request b owns
// [prefix[b], prefix[b+1])).  Partition g covers [T*g/G, T*(g+1)/G); a partition
// may span several requests and a request several partitions.  The piece
// (request b, partition g) writes partial slot b + g: for two pieces (b, g) and
// (b', g') with b + g = b' + g' and b < b', partition g' < g would have to reach
// past the end of request b while g starts before it, which contiguity forbids.
__device__ __forceinline__ int64_t part_begin(int64_t T, int G, int g) {
  return (T * g) / G;
}
// Partition holding concatenated page x: the largest g with part_begin(g) <= x.
__device__ __forceinline__ int part_of(int64_t T, int G, int64_t x) {
  return (int)(((x + 1) * G + T - 1) / T) - 1;
}

// Clamped visible length of request b; raises kFlagBadSeqLen for out-of-range input.
__device__ __forceinline__ int clamp_len(int L, int Sq, int max_pages, uint32_t* flags,
                                         bool report) {
  const int cap = max_pages * kPage;
  if (L < Sq || L > cap) {
    if (report) atomicOr(flags, kFlagBadSeqLen);
    L = L < 0 ? 0 : (L > cap ? cap : L);
  }
  return L;
}

// Fills prefix[0..B] (LDS) with the page prefix sums of the clamped lengths, and
// lens[0..B) with those lengths when lens is given.  Wave 0 scans; every thread of
// the workgroup must call it (it ends in a barrier).
__device__ inline void build_page_prefix(const int32_t* seq_lens, int B, int Sq, int max_pages,
                                         int* prefix, uint32_t* flags, bool report,
                                         int* lens = nullptr) {
  const int tid = threadIdx.x;
  if (tid < 64) {  // wave 0
    const int per = (B + 63) / 64;
    const int b0 = tid * per;
    const int b1 = min(B, b0 + per);
    int local = 0;
    for (int b = b0; b < b1; ++b) {
      const int L = clamp_len(seq_lens[b], Sq, max_pages, flags, report);
      local += (L + kPage - 1) / kPage;
    }
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (tid >= d) incl += v;
    }
    int run = incl - local;
    for (int b = b0; b < b1; ++b) {
      prefix[b] = run;
      const int L = clamp_len(seq_lens[b], Sq, max_pages, flags, false);
      if (lens) lens[b] = L;
      run += (L + kPage - 1) / kPage;
    }
    if (tid == 63) prefix[B] = incl;
  }
  __syncthreads();
}

// Logical workgroup id with all ids of one XCD contiguous.  Workgroups are handed
// to the eight XCDs round-robin by blockIdx (TokenSpeed review page, "Optimizing
// Attention on MI300X" entry): blockIdx x runs on XCD (x + o) % 8, where the offset
// o is wherever the dispatcher's rotation stood after earlier launches, so the ids
// with one value of x % 8 share an XCD.  Those ids are renumbered into one contiguous
// block, which keeps the M-tiles that share a KV range (and neighbouring ranges)
// inside one XCD's L2.  (Measured at the spec-decode shape with four M-tiles per
// range: 75% L2 hits and the KV fetched once, against 1% and four times over in
// launch order.)
__device__ __forceinline__ int xcd_logical_id(int x, int nwg) {
  const int xcd = x & 7, slot = x >> 3;
  const int per = nwg >> 3, rem = nwg & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

}  // namespace mla
