// FP4-packed weights with UE8M0 block scales (the V4-style expert weights of
// the fine-grained FP8 guide, sections 一 and 6.1, consumed by its FP8
// activation x FP4 weight linear).  One 1 x 32 group along K per scale (the
// microscaling block):
//   e = ceil(log2(amax / 6)) clamped to [-127, 127] (0 for amax == 0),
//   stored as the byte e + 127;  code = E2M1(w * 2^-e), round to nearest
//   even, two codes per byte, element 2i in the low nibble.
// HBM-bound: 2 bytes read and 0.5 + 1/32 written per weight.
#include "bsfp8_internal.h"

namespace bsfp8 {
namespace mxd {

// e = ceil(log2(amax / 6)): amax = f * 2^E with f in [1, 2) and 6 = 1.5 * 2^2,
// so e = E - 2 when f <= 1.5, else E - 1.  Integer logic on the fp32 bits
// (subnormals normalised).
__device__ __forceinline__ int mx_exp(float amax) {
  uint32_t u = __float_as_uint(amax) & 0x7fffffffu;
  if (u == 0) return 0;
  int E;
  uint32_t frac;
  const uint32_t ef = u >> 23;
  if (ef == 0) {
    const int msb = 31 - __clz(u);
    E = msb - 149;
    frac = (u << (23 - msb)) & 0x7fffffu;
  } else {
    E = (int)ef - 127;
    frac = u & 0x7fffffu;
  }
  const int e = (frac <= 0x400000u) ? E - 2 : E - 1;   // 0x400000 = 0.5 * 2^23
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// One thread per 32-element group: four 16-byte bf16 loads, one 16-byte
// code store, one scale byte.
__global__ __launch_bounds__(256) void mxfp4_quant_weight_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, int64_t ldw, uint8_t* __restrict__ wq4,
    uint8_t* __restrict__ scale) {
  const int64_t G = K / 32;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N * G) return;
  const int64_t n = i / G, g = i - n * G;
  const uint16_t* src = w + n * ldw + g * 32;
  float f[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 v = ld_stream16(src + 8 * j);
    f[8 * j + 0] = bf16_lo(v.x); f[8 * j + 1] = bf16_hi(v.x);
    f[8 * j + 2] = bf16_lo(v.y); f[8 * j + 3] = bf16_hi(v.y);
    f[8 * j + 4] = bf16_lo(v.z); f[8 * j + 5] = bf16_hi(v.z);
    f[8 * j + 6] = bf16_lo(v.w); f[8 * j + 7] = bf16_hi(v.w);
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(f[j]));
  const int e = mx_exp(amax);
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t r = 0;
    // the conversion takes the values pre-scaled (exact) and a unit scale
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, ldexpf(f[8 * j + 0], -e), ldexpf(f[8 * j + 1], -e), 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, ldexpf(f[8 * j + 2], -e), ldexpf(f[8 * j + 3], -e), 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, ldexpf(f[8 * j + 4], -e), ldexpf(f[8 * j + 5], -e), 1.0f, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, ldexpf(f[8 * j + 6], -e), ldexpf(f[8 * j + 7], -e), 1.0f, 3);
    out[j] = r;
  }
  *(uint4*)(wq4 + n * (K / 2) + g * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  scale[n * G + g] = (uint8_t)(e + 127);
}

}  // namespace mxd
using namespace mxd;

hipError_t launch_mxfp4_quant_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                     uint8_t* wq4, uint8_t* scale, hipStream_t s) {
  const int64_t groups = N * (K / 32);
  hipLaunchKernelGGL(mxfp4_quant_weight_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256),
                     0, s, w, N, K, ldw, wq4, scale);
  return hipGetLastError();
}

}  // namespace bsfp8
