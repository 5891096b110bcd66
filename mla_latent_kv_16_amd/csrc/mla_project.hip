// The two per-head GEMMs that bracket the latent attention (TokenSpeed review page,
// Attack 1, "absorb + project"): the key up-projection folded into the query before
// the decode, and the value up-projection applied to its latent output after it.
// Both are C[m, n] = sum_k A[m, k] W[n, k] for every head, on 32x32x16 bf16 MFMA
// with fp32 accumulation.  A workgroup takes one head and 32 rows; each of its four
// waves takes a quarter of the output columns.  W is stored n-major (its k run is
// contiguous), so every operand fragment is one sixteen-byte load per lane.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

// Eight consecutive A values of row m from k0: bf16 as stored, or fp32 rounded to
// bf16 (nearest, ties to even) for the MFMA.
__device__ __forceinline__ bf16x8 a_frag(const uint16_t* a, int64_t off) {
  return *reinterpret_cast<const bf16x8*>(a + off);
}
__device__ __forceinline__ bf16x8 a_frag(const float* a, int64_t off) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(a + off);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(a + off + 4);
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = static_cast<__bf16>(lo[i]);
    v[4 + i] = static_cast<__bf16>(hi[i]);
  }
  return v;
}

__device__ __forceinline__ void store_c(uint16_t* c, float v) {
  *c = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}
__device__ __forceinline__ void store_c(float* c, float v) { *c = v; }

// A: [rows, H, K] (row m of head h at (m H + h) K); W: [H, N, K]; C: [rows, H, N].
template <class TA, class TC, int K, int N>
__global__ void __launch_bounds__(kProjThreads) head_gemm_kernel(const TA* __restrict__ a,
                                                                 const uint16_t* __restrict__ w,
                                                                 TC* __restrict__ c, int rows,
                                                                 int H) {
  constexpr int kTiles = N / 32 / kWaves;  // 32-column tiles per wave
  static_assert(kTiles >= 1 && N % (32 * kWaves) == 0 && K % 16 == 0, "tile shape");
  const int h = blockIdx.y;
  const int m0 = blockIdx.x * 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = m0 + (lane & 31);
  const bool m_ok = m < rows;
  const int kh = 8 * (lane >> 5);  // this lane's k offset within a k-step
  const int64_t a_row = ((int64_t)(m_ok ? m : 0) * H + h) * K;
  const uint16_t* wh = w + (int64_t)h * N * K;
  f32x16 acc[kTiles];
#pragma unroll
  for (int j = 0; j < kTiles; ++j) acc[j] = f32x16{};
#pragma unroll 4
  for (int ks = 0; ks < K / 16; ++ks) {
    const int k = ks * 16 + kh;
    bf16x8 av = a_frag(a, a_row + k);
    if (!m_ok) av = bf16x8{};
#pragma unroll
    for (int j = 0; j < kTiles; ++j) {
      const int n = (wave * kTiles + j) * 32 + (lane & 31);
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(wh + (int64_t)n * K + k);
      acc[j] = mfma32(av, bv, acc[j]);
    }
  }
  // D register 4 q + e holds row 8 q + 4 (lane / 32) + e, column lane % 32
#pragma unroll
  for (int j = 0; j < kTiles; ++j) {
    const int n = (wave * kTiles + j) * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = m0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (r < rows) store_c(c + ((int64_t)r * H + h) * N + n, acc[j][i]);
    }
  }
}

hipError_t launch_absorb(const uint16_t* q_heads, const uint16_t* w_uk_t, uint16_t* q_lat,
                         int rows, int H, hipStream_t stream) {
  const dim3 grid((unsigned)((rows + 31) / 32), (unsigned)H);
  hipLaunchKernelGGL((head_gemm_kernel<uint16_t, uint16_t, kHeadDim, kNope>), grid,
                     dim3(kProjThreads), 0, stream, q_heads, w_uk_t, q_lat, rows, H);
  return hipGetLastError();
}

hipError_t launch_project(const float* O, const uint16_t* w_uv, float* out, int rows, int H,
                          hipStream_t stream) {
  const dim3 grid((unsigned)((rows + 31) / 32), (unsigned)H);
  hipLaunchKernelGGL((head_gemm_kernel<float, float, kNope, kHeadDim>), grid,
                     dim3(kProjThreads), 0, stream, O, w_uv, out, rows, H);
  return hipGetLastError();
}

}  // namespace mla
