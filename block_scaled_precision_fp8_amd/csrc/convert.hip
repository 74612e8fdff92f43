// Conversions around the FP8 path (fine-grained FP8 guide, sections 五 and 七):
//  * dequant_weight_kernel: fold the block scales (128 x 128 or 32 x 32) into the weights
//    (the dequantize-on-load step): bf16_rne(fl32(E4M3(code) * scale));
//  * pow2_to_ue8m0_kernel: power-of-two scales kept in float32 containers
//    -> the one-byte E8M0 form, exactly; any other value -> 0xFF (E8M0 NaN).
// Both are HBM-bound elementwise passes.
#include "bsfp8_internal.h"

namespace bsfp8 {
namespace detail {

// Eight codes per thread: one 8-byte load, one 16-byte store of bf16.
// E4M3 decode is the hardware conversion (exact for every finite code).
// lg = log2 of the block edge (7 for 128 x 128 blocks, 5 for 32 x 32).
template <int FMT>
__global__ __launch_bounds__(256) void dequant_weight_kernel(
    const uint8_t* __restrict__ wq, int64_t N, int64_t K, int64_t KB, int lg,
    const void* __restrict__ scale, uint16_t* __restrict__ w) {
  const int64_t per_row = K / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N * per_row) return;
  const int64_t n = i / per_row, k = (i - n * per_row) * 8;
  const int64_t sidx = (n >> lg) * KB + (k >> lg);
  float s;
  if (FMT == 0) {
    s = ((const float*)scale)[sidx];
  } else {
    // 2^(b-127): byte 0 is the subnormal 2^-127 (0x00400000); 0xFF is NaN
    const uint32_t b = ((const uint8_t*)scale)[sidx];
    s = __uint_as_float(b == 0 ? 0x00400000u : (b == 0xFF ? 0x7FC00000u : b << 23));
  }
  const uint2 c = *(const uint2*)(wq + n * K + k);
  float f[8];
  const uint32_t words[2] = {c.x, c.y};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[h], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[h], true);
    f[4 * h + 0] = lo[0]; f[4 * h + 1] = lo[1];
    f[4 * h + 2] = hi[0]; f[4 * h + 3] = hi[1];
  }
  uint4 o;
  uint32_t b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = f32_to_bf16(f[j] * s);
  o.x = b[0] | (b[1] << 16); o.y = b[2] | (b[3] << 16);
  o.z = b[4] | (b[5] << 16); o.w = b[6] | (b[7] << 16);
  *(uint4*)(w + n * K + k) = o;
}

// E8M0 byte 0 is 2^-127, an fp32 subnormal: its bits are 0x00400000.
__global__ __launch_bounds__(256) void pow2_to_ue8m0_kernel(const float* __restrict__ in,
                                                            int64_t n,
                                                            uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint32_t u = __float_as_uint(in[i]);
  const uint32_t ex = (u >> 23) & 0xFF, man = u & 0x7FFFFF;
  uint8_t b = 0xFF;
  if ((u >> 31) == 0) {
    if (ex >= 1 && ex <= 254 && man == 0) b = (uint8_t)ex;          // 2^(ex-127)
    else if (ex == 0 && man == 0x400000u) b = 0;                     // 2^-127
  }
  out[i] = b;
}

}  // namespace detail
using namespace detail;

hipError_t launch_dequant_weight(const uint8_t* wq, int64_t N, int64_t K, int fmt,
                                 const void* scale, uint16_t* w, hipStream_t s, int blk) {
  const int lg = blk == 32 ? 5 : 7;
  const int64_t KB = (K + blk - 1) / blk;
  const int64_t total = N * (K / 8);
  const dim3 grid((unsigned)((total + 255) / 256));
  if (fmt == 0)
    hipLaunchKernelGGL(dequant_weight_kernel<0>, grid, dim3(256), 0, s, wq, N, K, KB, lg, scale,
                       w);
  else
    hipLaunchKernelGGL(dequant_weight_kernel<1>, grid, dim3(256), 0, s, wq, N, K, KB, lg, scale,
                       w);
  return hipGetLastError();
}

hipError_t launch_pow2_to_ue8m0(const float* in, int64_t n, uint8_t* out, hipStream_t s) {
  hipLaunchKernelGGL(pow2_to_ue8m0_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     in, n, out);
  return hipGetLastError();
}

}  // namespace bsfp8
