// The two per-head GEMMs that bracket the latent attention (TokenSpeed review page,
// Attack 1, "absorb + project"): the key up-projection folded into the query before
// the decode, and the value up-projection applied to its latent output after it.
// Both are C[m, n] = sum_k A[m, k] W[n, k] for every head, on 32x32x16 bf16 MFMA
// with fp32 accumulation.  W is stored n-major (its k run is contiguous), so every
// operand fragment is one sixteen-byte load per lane.
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
// Workgroup (32-row tile, head h, 128-column chunk): the four waves split K, each
// computing all four 32-column tiles of the chunk over its quarter of K with every
// operand load issued up front (one memory round trip), then the four partial tiles
// are summed through LDS.  Decode shapes have few rows, so the latency of the load
// chain, not the MFMA rate, is what these kernels are sized for.
template <class TA, class TC, int K, int N>
__global__ void __launch_bounds__(kProjThreads) head_gemm_kernel(const TA* __restrict__ a,
                                                                 const uint16_t* __restrict__ w,
                                                                 TC* __restrict__ c, int rows,
                                                                 int H) {
  constexpr int kCols = 128;                 // columns per workgroup
  constexpr int kTiles = kCols / 32;         // 32-column tiles per wave
  constexpr int kSteps = K / 16 / kWaves;    // k-steps per wave
  static_assert(N % kCols == 0 && K % (16 * kWaves) == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) float part[kWaves - 1][kTiles][16][64];
  const int h = blockIdx.y;
  const int m0 = blockIdx.x * 32;
  const int n0 = blockIdx.z * kCols;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = m0 + (lane & 31);
  const bool m_ok = m < rows;
  const int kw = wave * kSteps * 16 + 8 * (lane >> 5);  // this lane's first k
  const int64_t a_row = ((int64_t)(m_ok ? m : 0) * H + h) * K;
  const uint16_t* wh = w + (int64_t)h * N * K;
  bf16x8 av[kSteps], bv[kSteps][kTiles];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    av[s] = a_frag(a, a_row + kw + 16 * s);
    if (!m_ok) av[s] = bf16x8{};
#pragma unroll
    for (int j = 0; j < kTiles; ++j)
      bv[s][j] = *reinterpret_cast<const bf16x8*>(
          wh + (int64_t)(n0 + 32 * j + (lane & 31)) * K + kw + 16 * s);
  }
  f32x16 acc[kTiles];
#pragma unroll
  for (int j = 0; j < kTiles; ++j) acc[j] = f32x16{};
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
#pragma unroll
    for (int j = 0; j < kTiles; ++j) acc[j] = mfma32(av[s], bv[s][j], acc[j]);
  // waves 1..3 hand their partial tiles to wave 0, which sums and writes them
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < kTiles; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) part[wave - 1][j][i][lane] = acc[j][i];
  }
  __syncthreads();
  if (wave == 0) {
    // D register 4 q + e holds row 8 q + 4 (lane / 32) + e, column lane % 32
#pragma unroll
    for (int j = 0; j < kTiles; ++j) {
      const int n = n0 + 32 * j + (lane & 31);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float v = acc[j][i] + part[0][j][i][lane] + part[1][j][i][lane] +
                        part[2][j][i][lane];
        const int r = m0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (r < rows) store_c(c + ((int64_t)r * H + h) * N + n, v);
      }
    }
  }
}

hipError_t launch_absorb(const uint16_t* q_heads, const uint16_t* w_uk_t, uint16_t* q_lat,
                         int rows, int H, hipStream_t stream) {
  const dim3 grid((unsigned)((rows + 31) / 32), (unsigned)H, kNope / 128);
  hipLaunchKernelGGL((head_gemm_kernel<uint16_t, uint16_t, kHeadDim, kNope>), grid,
                     dim3(kProjThreads), 0, stream, q_heads, w_uk_t, q_lat, rows, H);
  return hipGetLastError();
}

hipError_t launch_project(const float* O, const uint16_t* w_uv, float* out, int rows, int H,
                          hipStream_t stream) {
  const dim3 grid((unsigned)((rows + 31) / 32), (unsigned)H, kHeadDim / 128);
  hipLaunchKernelGGL((head_gemm_kernel<float, float, kNope, kHeadDim>), grid,
                     dim3(kProjThreads), 0, stream, O, w_uv, out, rows, H);
  return hipGetLastError();
}

}  // namespace mla
