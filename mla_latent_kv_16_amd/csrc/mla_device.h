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
constexpr int kCombineThreads = 256;           // combine pass: 4 waves, one row each
constexpr int kMaxBatch = 1024;
constexpr uint32_t kFlagBadSeqLen = 1u;
constexpr uint32_t kFlagBadPageId = 2u;
constexpr int kHeaderBytes = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// Each wave owns 16 folded query rows and runs v_mfma_f32_16x16x32_bf16; a
// workgroup of NW = 4 or 8 waves covers an M-tile of 16 * NW folded rows.
constexpr int kRowsPerWave = 16;
constexpr int kQSteps = kRow / 32;     // 18 MFMA k-steps over the 576-wide row
constexpr int kDBlocks = kNope / 16;   // 32 output column blocks of 16
constexpr int kBlockRows = 32;         // kv rows per softmax block (2 per page)

// ---- LDS layout of one staged page ------------------------------------------
// Row r of the page occupies bytes [r * 1152, (r + 1) * 1152).  Its sixteen-byte
// chunk c sits at chunk position c ^ swz(r); the xor only touches the low three
// bits, so a chunk never leaves its aligned group of eight (72 = 9 * 8).  With 64
// four-byte banks, rows r and r + 1 start half a bank row apart, and swz spreads
// (a) the 16 rows a ds_read_b128 quarter-wave reads at one chunk and (b) the 8 rows
// x 2 chunks a half-wave of ds_read_b64_tr_b16 reads over distinct banks.
__device__ __forceinline__ int swz(int r) {
  const int i = (r >> 1) & 7;  // index among same-parity rows of a 16-row block
  return ((i & 1) << 2) | (i & 2) | ((i >> 2) & 1);  // 3-bit bit reversal
}

// ---- instruction wrappers ---------------------------------------------------
__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const uint8_t* lds_base, int byte_off) {
  return *reinterpret_cast<const bf16x8*>(lds_base + byte_off);
}

// LDS transpose read (gfx950): within each group of 16 lanes, lane 16G + n
// receives element (n % 4) of the 8-byte words addressed by lanes 16G + 4r + n / 4,
// r = 0..3.  Addressing four rows with lanes 4r + c gives every lane one column of
// a 4-row block, i.e. the k-contiguous operand an MFMA needs from a row-major tile.
__device__ __forceinline__ bf16x4 lds_read_tr(const uint8_t* lds_base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4_t*)(lds_base + byte_off));
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct global -> LDS copy of 16 bytes per lane: lane l reads sbase + voff and
// writes LDS bytes [lds + 16 l, lds + 16 l + 16).  sbase and lds are wave-uniform.
// Issued as inline asm so that the compiler does not tie later LDS reads of the
// *other* stage buffer to these copies (it would wait for every copy in flight);
// completion is awaited explicitly with wait_vmem_all() before the barrier that
// publishes a stage.  The kernels use no M0-relative instructions of their own.
__device__ __forceinline__ void dma16(const void* sbase, int voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory");
}

// s_waitcnt encodings (gfx9): vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Reductions over the four lanes l % 16 + 16 k that hold one S^T column.
// v_permlane32_swap(x, x) leaves x[l % 32] in the first result and x[32 + l % 32]
// in the second, on every lane.
__device__ __forceinline__ float pair32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  return fmaxf(x, __shfl_xor(x, 16, 64));
}
__device__ __forceinline__ float xor16_sum(float x) {
  return x + __shfl_xor(x, 16, 64);
}

__device__ __forceinline__ bf16x8 pack_bf16(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(v[i]);
  return r;
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

// Fills prefix[0..B] (LDS) with the page prefix sums of the clamped lengths.
// Wave 0 scans; every thread of the workgroup must call it (it ends in a barrier).
__device__ inline void build_page_prefix(const int32_t* seq_lens, int B, int Sq, int max_pages,
                                         int* prefix, uint32_t* flags, bool report) {
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
      run += (L + kPage - 1) / kPage;
    }
    if (tid == 63) prefix[B] = incl;
  }
  __syncthreads();
}

// Logical workgroup id with all ids of one XCD contiguous.  Workgroups are handed
// to the eight XCDs round-robin by blockIdx (TokenSpeed review page, "Optimizing
// Attention on MI300X" entry), so blockIdx x runs on XCD x % 8; the ids a given
// XCD runs are renumbered into one contiguous block, which keeps the M-tiles that
// share a KV range (and neighbouring ranges) inside one XCD's L2.
__device__ __forceinline__ int xcd_logical_id(int x, int nwg) {
  const int xcd = x & 7, slot = x >> 3;
  const int per = nwg >> 3, rem = nwg & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

}  // namespace mla
