// Achievable-peak microbenchmarks for MI355X, measured in the same run as the
// attention kernels so that their roofline fractions have a same-box denominator
// beside the spec-sheet one.  They are measurement support, not part of the
// attention path: nothing in libmla calls them.
//
//  stream_read_kernel   HBM read bandwidth with plain 16-byte vector loads over a
//                       large buffer (each byte read once per launch).
//  dma_stream_kernel    the load path the split-KV kernel itself uses: 16-byte
//                       direct global->LDS copies of 36 KB blocks into a four-slot
//                       LDS ring, one workgroup of four waves per compute unit, two
//                       blocks in flight, each workgroup streaming one contiguous
//                       range (the split-KV kernel's partition walk without the math).
//  mfma_kernel          dense bf16 matrix-core rate: four independent accumulation
//                       chains of v_mfma_f32_32x32x16_bf16 per wave on register
//                       operands, several waves per SIMD.
#include "../../include/mla_peaks.h"
#include "mla_device.h"

namespace {

using namespace mla;

constexpr int kPeakThreads = 256;

// A value the loads cannot be proven not to produce, so the compiler keeps them.
constexpr uint32_t kNever = 0x9E3779B9u;

__global__ void __launch_bounds__(kPeakThreads) stream_read_kernel(const u32x4* p, int64_t n16,
                                                                   uint32_t* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * kPeakThreads;
  int64_t i = (int64_t)blockIdx.x * kPeakThreads + threadIdx.x;
  // four loads in flight per lane
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == kNever) sink[blockIdx.x] = x;
}

// The split-KV kernel's staging, alone: block k of the workgroup's range goes to ring
// slot k % 4; wave w copies 9 KB of each 36 KB block as nine 16-byte-per-lane copies.
// Three blocks are issued ahead of the one being "consumed" (a barrier after its
// copies have landed), so at most 27 copies per wave are outstanding.
constexpr int kDmaSlot = kStageBytes;  // 36,864
constexpr int kDmaStages = 4;

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
dma_stream_kernel(const uint8_t* p, int64_t blocks_per_wg, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kDmaStages * kDmaSlot];
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint8_t* base = p + (size_t)blockIdx.x * blocks_per_wg * kDmaSlot;
  const uint32_t ring_lds = lds_addr(ring);
  uint32_t off[kStageCopiesPerWave];
#pragma unroll
  for (int i = 0; i < kStageCopiesPerWave; ++i)
    off[i] = wave * kStageCopiesPerWave * 1024 + i * 1024 + lane * 16;
  auto issue = [&](int64_t k) {
    const uint8_t* src = base + (size_t)k * kDmaSlot;
    const uint32_t dst = ring_lds + (uint32_t)(k % kDmaStages) * kDmaSlot +
                         wave * kStageCopiesPerWave * 1024;
#pragma unroll
    for (int i = 0; i < kStageCopiesPerWave; ++i) dma16(src, off[i], dst + i * 1024);
  };
  const int64_t ahead = blocks_per_wg < 3 ? blocks_per_wg : 3;
  for (int64_t k = 0; k < ahead; ++k) issue(k);
  uint32_t acc = 0;
  for (int64_t k = 0; k < blocks_per_wg; ++k) {
    // block k has landed once at most (blocks issued after it) sets are in flight
    const int64_t after = (k + 3 <= blocks_per_wg ? 3 : blocks_per_wg - k) - 1;
    if (after >= 2)
      asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else if (after == 1)
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // block k is in LDS for every wave; block k - 1's slot is free
    acc ^= *reinterpret_cast<const uint32_t*>(ring + (k % kDmaStages) * kDmaSlot + 4 * threadIdx.x);
    if (k + 3 < blocks_per_wg) issue(k + 3);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (acc == kNever) sink[blockIdx.x] = acc;
}

__global__ void __launch_bounds__(kThreads) mfma_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = static_cast<__bf16>(0.001f * (float)((lane + k) & 7));
    b[k] = static_cast<__bf16>(0.002f * (float)((lane * 3 + k) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(b, a, c1);
    c2 = mfma32(a, a, c2);
    c3 = mfma32(b, b, c3);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += c0[k] + c1[k] + c2[k] + c3[k];
  if (s == -1.0f) sink[blockIdx.x] = s;
}

}  // namespace

extern "C" {

int mla_peak_stream_read(const void* buf, size_t bytes, void* sink, int workgroups,
                         void* stream) {
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15) || bytes < 16 || workgroups < 1)
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kPeakThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf),
                     (int64_t)(bytes / 16), static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mla_peak_dma_stream(const void* buf, size_t bytes, void* sink, int workgroups,
                        void* stream) {
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15) || workgroups < 1) return -1;
  const int64_t blocks_per_wg = (int64_t)(bytes / kDmaSlot) / workgroups;
  if (blocks_per_wg < 1) return -1;
  hipLaunchKernelGGL(dma_stream_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(buf),
                     blocks_per_wg, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

size_t mla_peak_dma_stream_bytes(size_t bytes, int workgroups) {
  if (workgroups < 1) return 0;
  return (size_t)((int64_t)(bytes / kDmaSlot) / workgroups) * workgroups * kDmaSlot;
}

int mla_peak_mfma_bf16(int iters, void* sink, int workgroups, void* stream) {
  if (!sink || iters < 1 || workgroups < 1) return -1;
  hipLaunchKernelGGL(mfma_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), iters, static_cast<float*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

double mla_peak_mfma_bf16_flops(int iters, int workgroups) {
  // four MFMAs of 32 x 32 x 16 per iteration per wave, four waves per workgroup
  return (double)workgroups * kWaves * iters * 4 * (2.0 * 32 * 32 * 16);
}

}  // extern "C"
