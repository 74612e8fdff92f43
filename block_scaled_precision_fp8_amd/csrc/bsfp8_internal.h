// Internal declarations shared by the HIP translation units of libbsfp8.so.
// Device helpers (bf16 <-> fp32, E4M3 packing, UE8M0 exponent) and the host
// launchers that the C-ABI layer (capi.hip) calls after argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsfp8 {

constexpr int kBlock = 128;        // weight block edge and act group width
constexpr float kE4M3Max = 448.0f; // largest finite OCP E4M3FN magnitude

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- device

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (data read once: non-temporal hint).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Four fp32 values -> four E4M3 bytes (little-endian in the result), round
// to nearest even, saturating at +-448.  The clamp makes the hardware
// conversion saturating; values in (448, 464) would round to 448 anyway.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  c = fminf(fmaxf(c, -kE4M3Max), kE4M3Max);
  d = fminf(fmaxf(d, -kE4M3Max), kE4M3Max);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

// e = ceil(log2(amax / 448)) clamped to [-127, 127]; 0 for amax == 0.
// amax = f * 2^E with f in [1, 2): e = E - 8 when f <= 1.75, else E - 7.
// Pure integer logic on the fp32 bits (subnormals normalised).
__device__ __forceinline__ int ue8m0_exp(float amax) {
  uint32_t u = __float_as_uint(amax) & 0x7fffffffu;
  if (u == 0) return 0;
  int E;
  uint32_t frac;
  uint32_t ef = u >> 23;
  if (ef == 0) {                      // subnormal: value = u * 2^-149
    int msb = 31 - __clz(u);          // position of the leading one
    E = msb - 149;
    frac = (u << (23 - msb)) & 0x7fffffu;
  } else {
    E = (int)ef - 127;
    frac = u & 0x7fffffu;
  }
  int e = (frac <= 0x600000u) ? E - 8 : E - 7;   // 0x600000 = 0.75 * 2^23
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Activation group codec (1 x 128 groups), one definition for every kernel
// that quantizes activations so their codes and scales agree bit for bit.
//   FLOAT: s = fl32(amax / 448) (1 for amax == 0), code = E4M3(fl32(x / s))
//   UE8M0: e = ue8m0_exp(amax), code = E4M3(x * 2^-e) (exact scaling)
__device__ __forceinline__ float act_scale_f32(float amax) {
  return (amax == 0.0f) ? 1.0f : amax / kE4M3Max;
}
template <int FMT>
__device__ __forceinline__ uint32_t act_encode4(float a, float b, float c, float d, float s,
                                                int e) {
  if (FMT == 0) return e4m3x4(a / s, b / s, c / s, d / s);
  return e4m3x4(ldexpf(a, -e), ldexpf(b, -e), ldexpf(c, -e), ldexpf(d, -e));
}

constexpr float kMinNormal = 0x1p-126f;   // smallest normal fp32

// fl32(x / s) for a NORMAL scale s from its reciprocal, in four operations
// per value instead of an IEEE division: q = RN(x' r), the residual
// x' - q s' (exact with an FMA) and q' = RN(q + residual r), Markstein's
// correction, which gives the correctly rounded quotient when r = RN(1 / s')
// and nothing underflows.  Two details make that hold for every x the
// activation codec meets:
//   * s < 2^-60: x and s are both multiplied by 2^64 first (exact; the
//     quotient is unchanged), so a subnormal x cannot leave a residual below
//     the smallest subnormal -- without this, x subnormal against a small
//     normal s rounded a tie the wrong way (an E4M3 code off by one);
//   * the result takes the sign of x: for x = -0 the correction step returns
//     +0 (-0 + +0), where the quotient is -0 (code 0x80).
// Against IEEE division (CPU emulation with exact rounding, every finite bf16
// x against 6000 scales from 448 * 2^-126 up): identical E4M3 codes; the fp32
// quotients differ only where they lie far below the smallest E4M3 subnormal
// (code +-0 either way).  Subnormal scales and the static scheme (x / s not
// bounded by 448) still divide directly.
struct RcpDiv {
  float s, r, m;   // rescaled scale, its correctly rounded reciprocal, the rescale
};
__device__ __forceinline__ RcpDiv rcp_div(float s) {
  const float m = s < 0x1p-60f ? 0x1p64f : 1.0f;
  const float sm = s * m;
  return RcpDiv{sm, 1.0f / sm, m};
}
__device__ __forceinline__ float div_by_rcp(float x, const RcpDiv& d) {
  const float xm = x * d.m;
  const float q = xm * d.r;
  const float res = fmaf(-q, d.s, xm);
  return copysignf(fmaf(res, d.r, q), x);
}
template <int FMT>
__device__ __forceinline__ uint32_t act_encode4_rcp(float a, float b, float c, float d,
                                                    const RcpDiv& dv, int e) {
  if (FMT == 0)
    return e4m3x4(div_by_rcp(a, dv), div_by_rcp(b, dv), div_by_rcp(c, dv), div_by_rcp(d, dv));
  return e4m3x4(ldexpf(a, -e), ldexpf(b, -e), ldexpf(c, -e), ldexpf(d, -e));
}

// Buffer resource over [base, base + bytes): loads past the end return 0,
// which handles ragged M, N and K edges without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
constexpr uint32_t kOOB = 0x80000000u;   // an offset past any buffer's end

#define BSFP8_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0): this wave's LDS stores are done (s_barrier alone
// does not wait for them on gfx950)
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}

// ---------------------------------------------------------------- host

// static_scale: null for dynamic 1x128 groups, else the device address of
// one calibrated per-tensor scale (fp32, or the E8M0 byte).
hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            int fmt, uint8_t* xq, void* scale, hipStream_t s,
                            const void* static_scale = nullptr, int group_k = 128);
hipError_t launch_dequant_weight(const uint8_t* wq, int64_t N, int64_t K, int fmt,
                                 const void* scale, uint16_t* w, hipStream_t s, int blk = 128);
hipError_t launch_pow2_to_ue8m0(const float* in, int64_t n, uint8_t* out, hipStream_t s);
hipError_t launch_mxfp4_quant_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                     uint8_t* wq4, uint8_t* scale, hipStream_t s);
hipError_t launch_quant_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                               int fmt, uint8_t* wq, void* scale, hipStream_t s,
                               int block = 128);

struct GemmArgs {
  const uint8_t* xq;
  const void* xs;          // [M][KB] fp32 or u8
  const uint8_t* wq;       // [E][N][K]
  const void* ws;          // [E][NB][KB]
  const uint16_t* bias;    // [N] or null
  uint16_t* y;             // [M][N]
  int64_t M, N, K;
  int fmt;
  const int32_t* seg;      // grouped: [E+1] device offsets, else null
  int E;
  void* workspace;
  size_t workspace_bytes;
  // fused act quant (fp8_linear decode path): bf16 input, else null; xstat
  // is the static scheme's calibrated scale (device fp32 or E8M0 byte), or
  // null for dynamic 1 x 128 groups
  const uint16_t* x_bf16;
  int64_t ldx;
  const void* xstat;
  // MXFP4 weights: wq (N, K/2) E2M1 codes, ws (N, K/32) E8M0 bytes
  bool w4;
  // grouped gate/up GEMM with the SiLU-mul requant epilogue: h codes
  // (M, N/2) and scales (M, N/256); y is then the optional bf16 h
  uint8_t* hq;
  void* hs;
  // weight block edge = activation group width: 128, or 32 for (32, 32)
  int blk = 128;
};

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
size_t fp8_fp4_workspace_bytes(int64_t M, int64_t N, int64_t K);
int gemm_kind(int64_t M, int64_t N, int64_t K, int* splits);   // a bsfp8_gemm_kind
size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int blk = 128);
bool linear_fused(int64_t M, int64_t N, int64_t K);   // fp8_linear quantizes inside the GEMM
bool linear_xq(int64_t M, int64_t N, int64_t K);      // ... inside the large-M GEMM (M > 16)
size_t grouped_workspace_bytes(int64_t T, int64_t N, int64_t K, int E);
hipError_t launch_block_gemm(const GemmArgs& a, hipStream_t s);
hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t s);
hipError_t launch_grouped_silu_mul_quant(const GemmArgs& a, hipStream_t s);

// C-ABI helpers shared by the entry points of capi.hip and noalloc.hip:
// the once-per-device gfx950 / stream-device check, and fp8_linear's
// host-only argument checks (*need: its workspace bytes) and launches.
int32_t check_device(void* stream);
int32_t linear_checks(const void* x, int64_t ldx, const void* wq, const void* w_scale_inv,
                      const void* bias, const void* y, int64_t M, int64_t N, int64_t K,
                      int32_t block_n, int32_t block_k, int32_t act_scheme, int32_t scale_fmt,
                      const void* act_scale, size_t* need);
int32_t linear_launch(const void* x, int64_t ldx, const void* wq, const void* w_scale_inv,
                      const void* bias, void* y, int64_t M, int64_t N, int64_t K, int32_t blk,
                      int32_t act_scheme, int32_t scale_fmt, const void* act_scale,
                      void* workspace, size_t workspace_bytes, void* stream);

size_t fp4_quant_workspace_bytes(int64_t R, int64_t K);
size_t fp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_fp4_quant(const uint16_t* x, int64_t R, int64_t K, int dynamic,
                            uint8_t* q4, uint8_t* gs, float* ts, void* ws, hipStream_t s);
hipError_t launch_fp4_gemm(const uint8_t* xq, const uint8_t* xs, const float* xt,
                           const uint8_t* wq, const uint8_t* wsc, const float* wt,
                           uint16_t* y, int64_t M, int64_t N, int64_t K, void* ws,
                           size_t ws_bytes, hipStream_t s);

}  // namespace bsfp8
