// Writing the new tokens' latent rows into the paged pool (the cache write that
// precedes the decode: the rows a decode verifies as drafts are already in the
// pool).  One thread moves one sixteen-byte chunk (8 bf16) of a new row; the
// destination row comes from the block table exactly as the decode finds it.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

// OCP E4M3 code of a float: the nearest E4M3 value, ties to the even code,
// magnitudes past 448 (and non-finite inputs) saturated to +-448.  Normal results
// keep 3 mantissa bits, rounded to nearest-even at bit 20 of the fp32 pattern and
// re-biased from exponent 127 to 7; below 2^-6 the codes are the multiples of 2^-9.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__float2int_rn(a * 512.0f);  // exact scaling, ties to even
  } else {
    const uint32_t bits = __float_as_uint(a);
    const uint32_t r = (bits + 0x7FFFFu + ((bits >> 20) & 1u)) & 0xFFF00000u;
    code = ((((r >> 23) & 0xFFu) - 120u) << 3) | ((r >> 20) & 7u);
  }
  return code | sign;
}

__global__ void __launch_bounds__(kAppendThreads) kv_append_kernel(AppendArgs a) {
  const int64_t g = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
  const int64_t rows = (int64_t)a.B * a.Sq;
  if (g >= rows * kChunks) return;
  const int64_t row = g / kChunks;
  const int ch = (int)(g - row * kChunks);  // chunk of 8 values within the row
  const int b = (int)(row / a.Sq), t = (int)(row - (int64_t)b * a.Sq);
  const int L = a.seq_lens[b];
  if (L < a.Sq || L > a.max_pages * kPage) {  // nothing is written for such a request
    if (t == 0 && ch == 0) atomicOr(a.flags, kFlagBadSeqLen);
    return;
  }
  const int j = L - a.Sq + t;  // logical row of draft t
  const int page = a.block_table[(size_t)b * a.max_pages + j / kPage];
  if (page < 0 || (int64_t)page >= a.num_pages) {
    if (ch == 0) atomicOr(a.flags, kFlagBadPageId);
    return;
  }
  const size_t dst_row = (size_t)page * kPage + (j % kPage);
  const u32x4 v = *reinterpret_cast<const u32x4*>(a.kv_new + row * kRow + ch * 8);
  if (!a.e4m3) {
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.kv_pool) + dst_row * kRow + ch * 8) = v;
    return;
  }
  uint32_t out[2];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    uint32_t packed = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // value 4 w + k: half k % 2 of bf16 pair v[2 w + k / 2]
      const uint32_t pair = v[2 * w + (k >> 1)];
      const float x = __uint_as_float((k & 1) ? (pair & 0xFFFF0000u) : (pair << 16));
      packed |= e4m3_code(x * a.inv_scale) << (8 * k);
    }
    out[w] = packed;
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(a.kv_pool) + dst_row * kRow +
                                              ch * 8);
  dst[0] = out[0];
  dst[1] = out[1];
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const int64_t chunks = (int64_t)a.B * a.Sq * kChunks;
  const int64_t nwg = (chunks + kAppendThreads - 1) / kAppendThreads;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)nwg), dim3(kAppendThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
