// NVFP4-style path for gfx950: quantization and GEMM.
//
// The NVFP4 page (Mistral-Medium-3.5-128B-NVFP4, config_groups group_1)
// stores the MLP projections' weights and input activations as 4-bit floats
// in 16-element groups.  Each group carries an E4M3 scale and each tensor an
// fp32 scale g:
//   g   = fl32(amax_tensor / 2688)         (1.0 for an all-zero tensor)
//   sg  = E4M3(fl32(amax_group / fl32(6 g)))
//   eff = fl32(dec(sg) * g),  code = E2M1(fl32(x / eff))   (0 when eff == 0)
// Codes are packed two per byte, element 2i in the low nibble.
//
// GEMM: an E2M1 value (<= 2 significant bits) times an E4M3 group scale
// (<= 4 significant bits) needs at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16.  Operands are dequantized to fp16
// in registers (hardware fp4 -> fp16 convert, then one packed fp16 multiply
// by the group scale) and multiplied with fp16 MFMAs accumulating in fp32;
// the two tensor scales are applied once in the epilogue.  The scaled
// f8f6f4 MFMA cannot be used here: its block scales are powers of two on
// 32-element blocks, while these group scales are E4M3 values on 16.
//
// Kernels:
//   fp4_amax_kernel        per-block partial max |x| (dynamic tensor scale)
//   fp4_quant_kernel       tensor scale from the partials, then one 16-element
//                          group per lane
//   fp4_gemm_stream_kernel M <= 64: weight-streaming split-K, W dequantized
//                          straight from global memory
//   fp4_gemm_lds_kernel    larger M: 128 x 128 tiles, both operands
//                          dequantized once per workgroup into fp16 LDS tiles,
//                          eight waves (two per SIMD)
//   fp4_splitk_reduce      fp32 partials -> bf16
#include <type_traits>

#include "bsfp8_internal.h"

namespace bsfp8 {
namespace fp4d {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kAmaxBlocks = 1024;

__device__ __forceinline__ float amax_bf16x8(uint4 v) {
  float a = fabsf(bf16_lo(v.x));
  a = fmaxf(a, fabsf(bf16_hi(v.x)));
  a = fmaxf(a, fabsf(bf16_lo(v.y)));
  a = fmaxf(a, fabsf(bf16_hi(v.y)));
  a = fmaxf(a, fabsf(bf16_lo(v.z)));
  a = fmaxf(a, fabsf(bf16_hi(v.z)));
  a = fmaxf(a, fabsf(bf16_lo(v.w)));
  a = fmaxf(a, fabsf(bf16_hi(v.w)));
  return a;
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// Partial max |x| over a grid-stride slice of the tensor, four independent
// 16-byte loads per lane per step (64 KB in flight per CU at four
// workgroups; one load per step left the pass latency-bound).  Plain
// (cached) loads: the quantization pass reads x again right after, and finds
// much of it in the last-level cache (8-10% faster than streaming loads at
// 4096 x 12288 and 4096 x 28672).  Rows are dense (K elements each,
// K % 32 == 0).
constexpr int kAmaxUnroll = 4;
__global__ __launch_bounds__(256) void fp4_amax_kernel(const uint16_t* __restrict__ x,
                                                       int64_t n8, float* __restrict__ part) {
  __shared__ float red[4];
  float a = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (kAmaxUnroll - 1) * stride < n8; i += kAmaxUnroll * stride) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) v[u] = *(const uint4*)(x + (i + u * stride) * 8);
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) a = fmaxf(a, amax_bf16x8(v[u]));
  }
  for (; i < n8; i += stride) a = fmaxf(a, amax_bf16x8(*(const uint4*)(x + i * 8)));
  a = block_max(a, red);
  if (threadIdx.x == 0) part[blockIdx.x] = a;
}

// One lane per 16-element group.  The tensor scale is either reduced from
// the partial maxima (every block reduces them the same way, so every block
// gets the same g) or read from *tscale.
__global__ __launch_bounds__(256) void fp4_quant_kernel(
    const uint16_t* __restrict__ x, int64_t groups, const float* __restrict__ part, int nparts,
    float* __restrict__ tscale, uint8_t* __restrict__ q4, uint8_t* __restrict__ gs) {
  __shared__ float red[4];
  float g;
  if (part != nullptr) {
    float a = 0.0f;
    for (int i = threadIdx.x; i < nparts; i += 256) a = fmaxf(a, part[i]);
    a = block_max(a, red);
    g = (a == 0.0f) ? 1.0f : a / 2688.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *tscale = g;
  } else {
    g = *tscale;
  }
  const float den = 6.0f * g;
  for (int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x; gi < groups;
       gi += (int64_t)gridDim.x * 256) {
    const uint4 v0 = ld_stream16(x + gi * 16);
    const uint4 v1 = ld_stream16(x + gi * 16 + 8);
    const float a = fmaxf(amax_bf16x8(v0), amax_bf16x8(v1));
    // group scale: E4M3 of a / (6 g), saturating, round to nearest even
    float sgf = a / den;
    sgf = fminf(sgf, kE4M3Max);
    const uint32_t sg = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sgf, 0.0f, 0, false) & 0xffu;
    const float eff = __builtin_amdgcn_cvt_f32_fp8((int)sg, 0) * g;
    float f[16];
    f[0] = bf16_lo(v0.x); f[1] = bf16_hi(v0.x); f[2] = bf16_lo(v0.y); f[3] = bf16_hi(v0.y);
    f[4] = bf16_lo(v0.z); f[5] = bf16_hi(v0.z); f[6] = bf16_lo(v0.w); f[7] = bf16_hi(v0.w);
    f[8] = bf16_lo(v1.x); f[9] = bf16_hi(v1.x); f[10] = bf16_lo(v1.y); f[11] = bf16_hi(v1.y);
    f[12] = bf16_lo(v1.z); f[13] = bf16_hi(v1.z); f[14] = bf16_lo(v1.w); f[15] = bf16_hi(v1.w);
    uint2 codes = make_uint2(0, 0);
    if (eff > 0.0f) {
      // E2M1 encode of fl32(x / eff): the hardware convert with a unit scale
      // rounds to nearest even and saturates at 6; element 2i -> low nibble.
      // Dynamic tensor scale: |x / eff| stays below 16 (eff follows the
      // group amax), where the reciprocal form with its correction gives
      // the same codes as IEEE division (checked on the CPU with exact fp32
      // rounding: every finite bf16 x with |x| <= 16 eff against 3000 scales
      // over the whole positive range, none differ); a static tensor scale
      // does not bound the quotient, so that case divides.
      float q[16];
      if (part != nullptr) {
        const RcpDiv dv = rcp_div(eff);
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = div_by_rcp(f[i], dv);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = f[i] / eff;
      }
      uint32_t lo = 0, hi = 0;
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, q[0], q[1], 1.0f, 0);
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, q[2], q[3], 1.0f, 1);
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, q[4], q[5], 1.0f, 2);
      lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, q[6], q[7], 1.0f, 3);
      hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, q[8], q[9], 1.0f, 0);
      hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, q[10], q[11], 1.0f, 1);
      hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, q[12], q[13], 1.0f, 2);
      hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, q[14], q[15], 1.0f, 3);
      codes = make_uint2(lo, hi);
    }
    *(uint2*)(q4 + gi * 8) = codes;
    gs[gi] = (uint8_t)sg;
  }
}

// ---------------------------------------------------------------- GEMM

// LDS reads through restrict-qualified pointers: the alias scope tells the
// compiler they do not touch the buffers the in-flight LDS-DMA writes, so it
// does not wait for that DMA before them
__device__ __forceinline__ uint4 read_u128(const uint8_t* __restrict__ p, int off) {
  return *(const uint4*)(p + off);
}
__device__ __forceinline__ uint32_t read_u16(const uint8_t* __restrict__ p, int off) {
  return *(const uint16_t*)(p + off);
}
// compile-time loop: f(std::integral_constant<int, 0>) .. f(<N - 1>)
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}


// Eight E2M1 codes (one 32-bit word, element 0 in the low nibble) times one
// group scale -> eight fp16 values, exact.
__device__ __forceinline__ half8 dequant8(uint32_t w, _Float16 s) {
  const half2v s2 = {s, s};
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t byte) {
  return (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

__device__ __forceinline__ void store4_bf16(uint16_t* y, int64_t N, int64_t m, int64_t n, v4f v) {
  uint2 o;
  o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
  o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
  *(uint2*)(y + m * N + n) = o;
}

// A 128-wide K block of one row: 64 bytes of codes + 8 group-scale bytes.
// Lane (l16, g4) owns K [32 g4, 32 g4 + 32): 16 code bytes (4 words) and 2
// scale bytes.  MFMA step t (0..3) uses word t: K [32 g4 + 8 t, + 8), group
// 2 g4 + t / 2 -- the same K assignment for both operands.
struct Frag128 {
  uint4 codes;
  uint32_t scales;   // two scale bytes in bits [15:0]
};

__device__ __forceinline__ Frag128 load_frag128(const uint8_t* q4, const uint8_t* gs, int64_t row,
                                                int64_t K, int64_t kb, int g4, bool valid) {
  Frag128 f;
  f.codes = make_uint4(0, 0, 0, 0);
  f.scales = 0;
  const int64_t k0 = kb * 128 + 32 * g4;
  if (valid && k0 < K) {
    f.codes = *(const uint4*)(q4 + row * (K / 2) + k0 / 2);
    f.scales = *(const uint16_t*)(gs + row * (K / 16) + k0 / 16);
  }
  return f;
}

__device__ __forceinline__ half8 frag_step(const Frag128& f, int t) {
  const uint32_t w = t == 0 ? f.codes.x : t == 1 ? f.codes.y : t == 2 ? f.codes.z : f.codes.w;
  return dequant8(w, e4m3_to_f16((f.scales >> (8 * (t >> 1))) & 0xffu));
}

constexpr int kStreamWaves = 4;
template <int MT> constexpr int kStreamBlocks = MT == 4 ? 2 : 4;

// S8 (K a multiple of 128, so a row's 8 scale bytes of a K block are 8-byte
// aligned): lane g4 < U loads all 8 weight-scale bytes of block kb + g4 in
// one load and the lanes of a row exchange them, one request per row per
// round of U blocks instead of one per row and block (the scales' own lines
// would otherwise double the requests of the weight stream)
template <int MT, bool S8>
__global__ __launch_bounds__(64 * kStreamWaves) void fp4_gemm_stream_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
    const float* __restrict__ xt, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ ws, const float* __restrict__ wt, uint16_t* __restrict__ y,
    float* __restrict__ part, int M, int64_t N, int64_t K, int kb_per_split) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int64_t n0 = ((int64_t)blockIdx.x * kStreamWaves + wave) * 16;
  if (n0 >= N) return;
  const int64_t KB = (K + 127) / 128;
  const int64_t kb0 = (int64_t)blockIdx.y * kb_per_split;
  const int64_t kb1 = min(KB, kb0 + kb_per_split);
  const bool nvalid = n0 + l16 < N;
  v4f acc[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  // K blocks per round of loads: each wave walks its split in rounds whose
  // latency is exposed, so fewer, wider rounds where registers allow
  constexpr int U = kStreamBlocks<MT>;
  for (int64_t kb = kb0; kb < kb1; kb += U) {
    // the weight fragments (HBM) and the activation fragments (L2) of U
    // blocks, all issued before any is used so their latencies overlap
    Frag128 fw[U], fx[U][MT];
    uint2 wsc8 = make_uint2(0, 0), xsc8[MT];
    if constexpr (S8) {
      if (nvalid && g4 < U && kb + g4 < kb1)
        wsc8 = *(const uint2*)(ws + (n0 + l16) * (K / 16) + (kb + g4) * 8);
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        xsc8[j] = make_uint2(0, 0);
        if (j * 16 + l16 < M && g4 < U && kb + g4 < kb1)
          xsc8[j] = *(const uint2*)(xs + (int64_t)(j * 16 + l16) * (K / 16) + (kb + g4) * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (S8) {
        fw[u].codes = make_uint4(0, 0, 0, 0);
        fw[u].scales = 0;
        const int64_t k0 = (kb + u) * 128 + 32 * g4;
        if (nvalid && kb + u < kb1 && k0 < K)
          fw[u].codes = *(const uint4*)(wq + (n0 + l16) * (K / 2) + k0 / 2);
      } else {
        fw[u] = load_frag128(wq, ws, n0 + l16, K, kb + u, g4, nvalid && kb + u < kb1);
      }
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        if constexpr (S8) {
          fx[u][j].codes = make_uint4(0, 0, 0, 0);
          fx[u][j].scales = 0;
          const int64_t k0 = (kb + u) * 128 + 32 * g4;
          if (j * 16 + l16 < M && kb + u < kb1 && k0 < K)
            fx[u][j].codes = *(const uint4*)(xq + (int64_t)(j * 16 + l16) * (K / 2) + k0 / 2);
        } else {
          fx[u][j] = load_frag128(xq, xs, j * 16 + l16, K, kb + u, g4,
                                  j * 16 + l16 < M && kb + u < kb1);
        }
      }
    }
    if constexpr (S8) {
      // this lane's two bytes of block kb + u: bytes 2 g4, 2 g4 + 1 of the
      // 8 held by lane (l16, u)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t lo = __shfl(wsc8.x, l16 + 16 * u);
        const uint32_t hi = __shfl(wsc8.y, l16 + 16 * u);
        fw[u].scales = ((g4 < 2 ? lo : hi) >> (16 * (g4 & 1))) & 0xffffu;
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          const uint32_t xl = __shfl(xsc8[j].x, l16 + 16 * u);
          const uint32_t xh = __shfl(xsc8[j].y, l16 + 16 * u);
          fx[u][j].scales = ((g4 < 2 ? xl : xh) >> (16 * (g4 & 1))) & 0xffffu;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kb + u >= kb1) break;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const half8 a = frag_step(fw[u], t);
#pragma unroll
        for (int j = 0; j < MT; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, frag_step(fx[u][j], t), acc[j], 0, 0, 0);
      }
    }
  }
  const float gg = (*xt) * (*wt);
  const int64_t n = n0 + 4 * g4;
  if (n >= N) return;
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int m = j * 16 + l16;
    if (m >= M) continue;
    const v4f v = acc[j] * gg;
    if (part == nullptr) store4_bf16(y, N, m, n, v);
    else *(float4*)(part + ((int64_t)blockIdx.y * M + m) * N + n) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

__global__ __launch_bounds__(256) void fp4_splitk_reduce(const float* __restrict__ part, int splits,
                                                         int64_t MN, int64_t N,
                                                         uint16_t* __restrict__ y) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= MN) return;
  float4 s = *(const float4*)(part + i4);
  for (int k = 1; k < splits; ++k) {
    const float4 t = *(const float4*)(part + (int64_t)k * MN + i4);
    s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
  }
  const int64_t m = i4 / N, n = i4 - m * N;
  store4_bf16(y, N, m, n, v4f{s.x, s.y, s.z, s.w});
}

// Large-M kernel: 128 x 128 output tile, WAVES_M x WAVES_N waves (wave tile
// (128 / WAVES_M) x (128 / WAVES_N)), K step 128.  Every K block: each
// thread loads a slice of one row of codes + scales of X and of W (global ->
// registers, two blocks ahead), dequantizes them to fp16 and stores them to
// LDS; rows are 256 bytes (16 chunks of 8 halves) with chunk c stored at
// c ^ (row & 15), so the 16 rows of a fragment read hit 16 different bank
// groups.  The fp16 tiles take 128 KB of LDS (one workgroup per CU); eight
// waves put two on each SIMD, so one wave's dequantization, LDS traffic and
// barrier wait overlap the other's MFMAs.
constexpr int kLdsBM = 128, kLdsBN = 128;

template <int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void fp4_gemm_lds_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
    const float* __restrict__ xt, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ ws, const float* __restrict__ wt, uint16_t* __restrict__ y,
    int64_t M, int64_t N, int64_t K) {
  constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  constexpr int WM = kLdsBM / WAVES_M, WN = kLdsBN / WAVES_N;
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int LPR = THREADS / 128;          // loader threads per row
  constexpr int KPT = 128 / LPR;              // K elements per loader thread
  constexpr int CPT = KPT / 8;                // 8-value chunks (code words) per thread
  static_assert(LPR == 2 || LPR == 4 || LPR == 8, "loader layout");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(kLdsBM + kLdsBN) * 256];
  const int64_t MT = (M + kLdsBM - 1) / kLdsBM;
  const int64_t NT = (N + kLdsBN - 1) / kLdsBN;
  // XCD-aware order, M tiles fastest within groups of 8
  const int bid = blockIdx.x;
  const int per_xcd = (int)(gridDim.x / 8);
  const int t = (bid & 7) * per_xcd + (bid >> 3);
  if (t >= MT * NT) return;
  constexpr int GM = 8;
  const int group = t / (GM * (int)NT);
  const int first_m = group * GM;
  const int gsz = min((int)MT - first_m, GM);
  const int in = t - group * GM * (int)NT;
  const int64_t m0 = (int64_t)(first_m + in % gsz) * kLdsBM;
  const int64_t n0 = (int64_t)(in / gsz) * kLdsBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int64_t KB = (K + 127) / 128;

  // loader role: row r (0..127), slice h: K [KPT h, KPT h + KPT) of the block
  const int lr = tid / LPR, lh = tid % LPR;
  const bool xrow_ok = m0 + lr < M, wrow_ok = n0 + lr < N;
  // two register sets of loaded codes (one 32-bit word per 8 values) and
  // group-scale bytes (one per 16 values), for blocks kb and kb + 1
  uint32_t xcs[2][CPT], wcs[2][CPT];
  uint32_t xscs[2] = {0, 0}, wscs[2] = {0, 0};
  auto gload = [&](int64_t kb, auto set_c) {
    constexpr int st = decltype(set_c)::value;
    uint32_t* xc = xcs[st];
    uint32_t* wc = wcs[st];
    uint32_t& xsc = xscs[st];
    uint32_t& wsc = wscs[st];
    const int64_t k0 = kb * 128 + KPT * lh;
#pragma unroll
    for (int i = 0; i < CPT; ++i) xc[i] = wc[i] = 0;
    xsc = wsc = 0;
    // K % 32 == 0: each 32-value quarter (and so each 16-value slice) is
    // wholly in or out of range; a 64-value slice may end after its first
    // quarter
    if (kb >= KB || k0 >= K) return;
    auto ld = [&](const uint8_t* q, const uint8_t* gs, int64_t row, uint32_t* c, uint32_t& sc) {
      const uint8_t* p = q + row * (K / 2) + k0 / 2;
      const uint8_t* sp = gs + row * (K / 16) + k0 / 16;
      if constexpr (CPT >= 4) {
#pragma unroll
        for (int i = 0; i < CPT / 4; ++i) {
          if (k0 + 32 * i >= K) break;
          const uint4 v = *(const uint4*)(p + 16 * i);
          c[4 * i] = v.x; c[4 * i + 1] = v.y; c[4 * i + 2] = v.z; c[4 * i + 3] = v.w;
          sc |= (uint32_t)(sp[2 * i] | (sp[2 * i + 1] << 8)) << (16 * i);
        }
      } else {
        const uint2 v = *(const uint2*)p;
        c[0] = v.x; c[1] = v.y;
        sc = sp[0];
      }
    };
    if (xrow_ok) ld(xq, xs, m0 + lr, xc, xsc);
    if (wrow_ok) ld(wq, ws, n0 + lr, wc, wsc);
  };
  // dequantize this thread's KPT elements of each operand into LDS buffer b
  auto dstore = [&](int b, auto set_c) {
    constexpr int st = decltype(set_c)::value;
    const uint32_t* xc = xcs[st];
    const uint32_t* wc = wcs[st];
    const uint32_t xsc = xscs[st], wsc = wscs[st];
    uint8_t* sx = lds[b];
    uint8_t* sw = lds[b] + kLdsBM * 256;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {        // chunk c: 8 values, group c / 2
      const uint32_t xw = xc[c];
      const uint32_t ww = wc[c];
      const half8 hx = dequant8(xw, e4m3_to_f16((xsc >> (8 * (c >> 1))) & 0xffu));
      const half8 hw = dequant8(ww, e4m3_to_f16((wsc >> (8 * (c >> 1))) & 0xffu));
      const int chunk = lh * CPT + c;
      const int phys = chunk ^ (lr & 15);
      *(half8*)(sx + lr * 256 + phys * 16) = hx;
      *(half8*)(sw + lr * 256 + phys * 16) = hw;
    }
  };

  v4f acc[NI][MI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  gload(0, S0{});
  gload(1, S1{});
  dstore(0, S0{});
  __syncthreads();
  // block kb: LDS buffer kb & 1 holds it, register set kb & 1 refills with
  // block kb + 2, register set (kb + 1) & 1 holds block kb + 1 for the store
  auto iter = [&](int64_t kb, auto b_c) {
    constexpr int b = decltype(b_c)::value;
    gload(kb + 2, b_c);
    const uint8_t* sx = lds[b];
    const uint8_t* sw = lds[b] + kLdsBM * 256;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {        // MFMA K step: chunks 4 ks + g4
      half8 bx[MI], aw[NI];
      const int chunk = 4 * ks + g4;
#pragma unroll
      for (int j = 0; j < MI; ++j) {
        const int r = wm * WM + j * 16 + l16;
        bx[j] = *(const half8*)(sx + r * 256 + ((chunk ^ (r & 15)) * 16));
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = wn * WN + i * 16 + l16;
        aw[i] = *(const half8*)(sw + r * 256 + ((chunk ^ (r & 15)) * 16));
      }
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < MI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw[i], bx[j], acc[i][j], 0, 0, 0);
    }
    if (kb + 1 < KB) dstore(b ^ 1, std::integral_constant<int, b ^ 1>{});
    __syncthreads();
  };
  for (int64_t kb = 0; kb < KB; kb += 2) {
    iter(kb, S0{});
    if (kb + 1 < KB) iter(kb + 1, S1{});
  }

  // bf16 epilogue through LDS (the loop ended with a barrier after its last
  // fragment reads): waves write their tiles row-major, 16-byte chunks
  // swizzled by row, then every thread stores whole chunks, 16 lanes to a
  // 256-byte row, so the output leaves in full lines
  const float gg = (*xt) * (*wt);
  constexpr int CPR = kLdsBN / 8;              // 16-byte chunks per output row
  uint8_t* ot = lds[0];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int col = wn * WN + i * 16 + 4 * g4;
#pragma unroll
    for (int j = 0; j < MI; ++j) {
      const int row = wm * WM + j * 16 + l16;
      const v4f v = acc[i][j] * gg;
      uint2 o;
      o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
      o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
      const int c = col >> 3;
      *(uint2*)(ot + row * (kLdsBN * 2) + ((c ^ (row & (CPR - 1))) << 4) + ((col >> 2) & 1) * 8) = o;
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kLdsBM * CPR / THREADS; ++p) {
    const int L = p * THREADS + tid;
    const int row = L / CPR, c = L % CPR;
    const int64_t m = m0 + row, n = n0 + c * 8;
    if (m < M && n < N)
      *(uint4*)(y + m * N + n) = *(const uint4*)(ot + row * (kLdsBN * 2) + ((c ^ (row & (CPR - 1))) << 4));
  }
}

// ------------------------------------------------------------------------
// Large-M NVFP4 GEMM on staged codes (K % 128 == 0).  fp4_gemm_lds_kernel
// keeps both operands in LDS as fp16, four times the bytes of the codes: per
// 128-wide K block its dequantized stores and fragment reads move about
// 256 KB through LDS against about 1000 cycles of fp16 MFMA work, and the
// kernel runs at about a third of the fp16 peak.  Here LDS holds the raw
// operands -- E2M1 codes, 64 bytes per row and K block, and E4M3 group
// scales, 8 bytes -- in a four-stage pipeline filled by LDS-DMA, and each
// wave dequantizes its fragments in registers after reading them (hardware
// fp4 -> fp16 convert, one packed multiply by the group scale; exact, as in
// fp4_gemm_lds_kernel): about 55 KB of LDS traffic per K block.
//   tiles of 128 x 128 (four waves of 64 x 64, two workgroups per CU) or
//   256 x 256 (eight waves of 64 x 128, one workgroup per CU; the kernel is
//   bound by the dequantization on the vector ALU, and a wave's weight
//   fragment then feeds eight MFMAs instead of four);
//   lane (l16, g4) reads 16 contiguous code bytes of a row -- K
//   [32 g4, 32 g4 + 32) of the block -- and feeds 8 of them to each of the
//   four 16x16x32 MFMA steps (step s: K [32 g4 + 8 s, + 8)), the same K
//   assignment for both operands; its two group scales are bytes 2 g4 and
//   2 g4 + 1 of the row's eight;
//   LDS rows of 64 bytes: lane chunk c of row r sits at chunk c ^ ((r >> 1)
//   & 3), so the 16 rows of a fragment read hit distinct banks (the DMA
//   stays contiguous: the swizzle is applied to its source offsets).
// ------------------------------------------------------------------------
constexpr int kDmaStages = 4;
constexpr int kDmaLoads = 6;                                 // DMA ops per lane per stage

// Tile BM x BN with WAVES_M x WAVES_N waves of (BM / WAVES_M) x (BN /
// WAVES_N); a stage holds both operands' codes (64 bytes per row) and group
// scales (8 bytes per row) of one K block.  Either tile forms every output
// from the same MFMA sequence over K, so both give the same bits.
template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 512 / (64 * WAVES_M * WAVES_N))
void fp4_gemm_dma_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
    const float* __restrict__ xt, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ ws, const float* __restrict__ wt, uint16_t* __restrict__ y,
    int64_t M, int64_t N, int64_t K) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int WAVES = WAVES_M * WAVES_N, THREADS = 64 * WAVES;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, MI = WM / 16, NI = WN / 16;
  constexpr int XCODES = BM * 64, WCODES = BN * 64;           // codes per stage
  constexpr int XSC = BM * 8, WSC = BN * 8;                   // group scales per stage
  constexpr int STAGE = XCODES + WCODES + XSC + WSC;
  constexpr int CJ = XCODES / (THREADS * 16);                 // 16-byte code loads per lane
  static_assert(BM == BN && CJ * THREADS * 16 == XCODES && XSC == THREADS * 4,
                "square tile, whole code chunks and one scale dword per lane");
  static_assert(2 * CJ + 2 == kDmaLoads, "DMA ops per lane per stage");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kDmaStages * STAGE];
  const int64_t MT = (M + BM - 1) / BM;
  const int64_t NT = (N + BN - 1) / BN;
  // XCD-aware order, M tiles fastest within groups of 8 (as fp4_gemm_lds_kernel)
  const int bid = blockIdx.x;
  const int per_xcd = (int)(gridDim.x / 8);
  const int t = (bid & 7) * per_xcd + (bid >> 3);
  if (t >= MT * NT) return;
  constexpr int GM = 8;
  const int group = t / (GM * (int)NT);
  const int first_m = group * GM;
  const int gsz = min((int)MT - first_m, GM);
  const int in = t - group * GM * (int)NT;
  const int64_t m0 = (int64_t)(first_m + in % gsz) * BM;
  const int64_t n0 = (int64_t)(in / gsz) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int KB = (int)(K / 128);
  const int64_t KH = K / 2, KG = K / 16;            // code and scale bytes per row
  const int64_t mrows = min((int64_t)BM, M - m0), nrows = min((int64_t)BN, N - n0);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xq + m0 * KH, mrows * KH);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wq + n0 * KH, nrows * KH);
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(xs + m0 * KG, mrows * KG);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(ws + n0 * KG, nrows * KG);
  const float gg = (*xt) * (*wt);

  // stage kb into buffer b: codes (lane chunk q: row q >> 2, LDS chunk q & 3
  // holding code chunk (q & 3) ^ ((row >> 1) & 3)), then scales (row q >> 1,
  // dword q & 1); rows past the tile and blocks past K read zeros
  auto issue = [&](int kb, int b) __attribute__((always_inline)) {
    uint8_t* st = lds + b * STAGE;
    const uint32_t kc = (uint32_t)kb * 64, ks = (uint32_t)kb * 8;
    const bool kin = kb < KB;
#pragma unroll
    for (int j = 0; j < CJ; ++j) {
      const int q = (j * WAVES + wave) * 64 + lane;
      const int row = q >> 2, c = (q & 3) ^ ((row >> 1) & 3);
      const uint32_t off = kin ? (uint32_t)(row * KH) + kc + c * 16 : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, BSFP8_LDS(st + (j * WAVES + wave) * 1024), 16,
                                               off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, BSFP8_LDS(st + XCODES + (j * WAVES + wave) * 1024), 16, off, 0, 0, 0);
    }
    const int q = wave * 64 + lane;
    const uint32_t so = kin ? (uint32_t)((q >> 1) * KG) + ks + (q & 1) * 4 : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rxs, BSFP8_LDS(st + XCODES + WCODES + wave * 256), 4,
                                             so, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rws, BSFP8_LDS(st + XCODES + WCODES + XSC + wave * 256), 4, so, 0, 0, 0);
  };

  v4f acc[NI][MI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // one K block from buffer b: 16 code bytes and two scale bytes per row
  // (BM > 128: the code words are read per step, 4 bytes per fragment, so
  // that the 64 x 128 accumulators and the fragments fit two waves per SIMD)
  auto compute = [&](int b) __attribute__((always_inline)) {
    const uint8_t* st = lds + b * STAGE;
    constexpr bool WIDE = BM <= 128;
    uint4 xc[WIDE ? MI : 1], wc[WIDE ? NI : 1];
    uint32_t xsc[MI], wsc[NI];
    // row r = (first row of the wave) + 16 f + l16: the swizzle (r >> 1) & 3
    // is that of l16 for every fragment f, so fragment f sits 1024 f bytes
    // (codes) and 128 f bytes (scales) past fragment 0
    const int sw = (g4 ^ ((l16 >> 1) & 3)) << 4;
    const int xo0 = (wm * WM + l16) * 64 + sw, wo0 = (wn * WN + l16) * 64 + sw;
    const int xs0 = (wm * WM + l16) * 8 + 2 * g4, ws0 = (wn * WN + l16) * 8 + 2 * g4;
    int xo[MI], wo[NI];
#pragma unroll
    for (int j = 0; j < MI; ++j) {
      xo[j] = xo0 + j * 1024;
      if constexpr (WIDE) xc[j] = read_u128(st, xo[j]);
      xsc[j] = read_u16(st + XCODES + WCODES, xs0 + j * 128);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      wo[i] = wo0 + i * 1024;
      if constexpr (WIDE) wc[i] = read_u128(st + XCODES, wo[i]);
      wsc[i] = read_u16(st + XCODES + WCODES + XSC, ws0 + i * 128);
    }
    auto word = [&](const uint4* c, const uint8_t* base, int off, int s) __attribute__((always_inline)) {
      if constexpr (WIDE) return s == 0 ? c->x : s == 1 ? c->y : s == 2 ? c->z : c->w;
      else return *(const uint32_t*)(base + off + 4 * s);
    };
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8 bx[MI];
#pragma unroll
      for (int j = 0; j < MI; ++j) {
        const uint32_t w = word(&xc[WIDE ? j : 0], st, xo[j], s);
        bx[j] = dequant8(w, e4m3_to_f16((xsc[j] >> (8 * (s >> 1))) & 0xffu));
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const uint32_t w = word(&wc[WIDE ? i : 0], st + XCODES, wo[i], s);
        const half8 aw = dequant8(w, e4m3_to_f16((wsc[i] >> (8 * (s >> 1))) & 0xffu));
#pragma unroll
        for (int j = 0; j < MI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, bx[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  // prologue: stages 0..2; then per block: its stage has landed (the two
  // newer ones may still fly: loads retire in issue order), everyone's has
  // and everyone is done reading the buffer refilled next, refill, multiply
  issue(0, 0);
  issue(1, 1);
  issue(2, 2);
  for (int kb0 = 0; kb0 < KB; kb0 += kDmaStages) {
    static_for<kDmaStages>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      const int kb = kb0 + s;
      if (kb >= KB) return;
      wait_vmcnt<2 * kDmaLoads>();
      wait_lgkmcnt0();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(kb + 3, (s + 3) % kDmaStages);
      compute(s);
    });
  }
  // drain: no DMA may land in LDS once it holds the output tile
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  __syncthreads();

  // bf16 epilogue through LDS (as fp4_gemm_lds_kernel)
  constexpr int CPR = BN / 8;                  // 16-byte chunks per output row
  static_assert(BM * BN * 2 <= kDmaStages * STAGE, "output tile fits the stage buffers");
  uint8_t* ot = lds;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int col = wn * WN + i * 16 + 4 * g4;
#pragma unroll
    for (int j = 0; j < MI; ++j) {
      const int row = wm * WM + j * 16 + l16;
      const v4f v = acc[i][j] * gg;
      uint2 o;
      o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
      o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
      const int c = col >> 3;
      *(uint2*)(ot + row * (BN * 2) + ((c ^ (row & (CPR - 1))) << 4) + ((col >> 2) & 1) * 8) = o;
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < BM * CPR / THREADS; ++p) {
    const int L = p * THREADS + tid;
    const int row = L / CPR, c = L % CPR;
    const int64_t m = m0 + row, n = n0 + c * 8;
    if (m < M && n < N)
      *(uint4*)(y + m * N + n) = *(const uint4*)(ot + row * (BN * 2) + ((c ^ (row & (CPR - 1))) << 4));
  }
#endif
}

constexpr int kFp4WavesN = 4;   // 2 x 4 waves of 64 x 32 (two per SIMD)

constexpr int64_t kStreamMaxM = 64;

int fp4_splits(int64_t N, int64_t K) {
  const int64_t KB = (K + 127) / 128;
  const int64_t wg_n = (N + 16 * kStreamWaves - 1) / (16 * kStreamWaves);
  int64_t want = (2048 + wg_n - 1) / wg_n;
  int64_t max_by_depth = KB / 4;
  int64_t s = want < max_by_depth ? want : max_by_depth;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

void fp4_split_plan(int64_t N, int64_t K, int* kbps, int* real) {
  const int64_t KB = (K + 127) / 128;
  const int s = fp4_splits(N, K);
  *kbps = (int)((KB + s - 1) / s);
  *real = (int)((KB + *kbps - 1) / *kbps);
}

}  // namespace fp4d
using namespace fp4d;

size_t fp4_quant_workspace_bytes(int64_t, int64_t) { return kAmaxBlocks * sizeof(float); }

size_t fp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || M > kStreamMaxM) return 0;
  int kbps, real;
  fp4_split_plan(N, K, &kbps, &real);
  return real > 1 ? (size_t)real * M * N * sizeof(float) : 0;
}

hipError_t launch_fp4_quant(const uint16_t* x, int64_t R, int64_t K, int dynamic, uint8_t* q4,
                            uint8_t* gs, float* ts, void* ws, hipStream_t s) {
  const int64_t n8 = R * K / 8;
  const int64_t groups = R * K / 16;
  float* part = nullptr;
  int nparts = 0;
  if (dynamic) {
    part = (float*)ws;
    int64_t nb = (n8 + 256 * 8 - 1) / (256 * 8);
    if (nb > kAmaxBlocks) nb = kAmaxBlocks;
    if (nb < 1) nb = 1;
    nparts = (int)nb;
    hipLaunchKernelGGL(fp4_amax_kernel, dim3(nparts), dim3(256), 0, s, x, n8, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int64_t nb = (groups + 255) / 256;
  if (nb > 8192) nb = 8192;
  hipLaunchKernelGGL(fp4_quant_kernel, dim3((unsigned)nb), dim3(256), 0, s, x, groups, part,
                     nparts, ts, q4, gs);
  return hipGetLastError();
}

hipError_t launch_fp4_gemm(const uint8_t* xq, const uint8_t* xs, const float* xt,
                           const uint8_t* wq, const uint8_t* wsc, const float* wt, uint16_t* y,
                           int64_t M, int64_t N, int64_t K, void* ws, size_t, hipStream_t s) {
  if (M > kStreamMaxM) {
    int64_t tiles = ((M + kLdsBM - 1) / kLdsBM) * ((N + kLdsBN - 1) / kLdsBN);
    tiles = (tiles + 7) / 8 * 8;
    if (K % 128 == 0) {   // staged codes, dequantized per fragment
      // 256 x 256 tiles (one workgroup per CU, 1.15-1.2x the rate of a
      // 128 x 128 tile pair in a round of the Llama-sized MLP) when their
      // rounds over the 256 CUs take no longer: a round of big tiles costs
      // about 1.75 rounds of 512 small ones, and up to 256 small tiles run
      // one per CU at about 0.56 of a round
      const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
      const int64_t rb = (big + 255) / 256, rs = (tiles + 511) / 512;
      if (tiles > 256 && 7 * rb <= 4 * rs) {
        const int64_t bt = (big + 7) / 8 * 8;
        hipLaunchKernelGGL((fp4_gemm_dma_kernel<256, 256, 4, 2>), dim3((unsigned)bt), dim3(512), 0,
                           s, xq, xs, xt, wq, wsc, wt, y, M, N, K);
      } else {
        hipLaunchKernelGGL((fp4_gemm_dma_kernel<128, 128, 2, 2>), dim3((unsigned)tiles), dim3(256),
                           0, s, xq, xs, xt, wq, wsc, wt, y, M, N, K);
      }
    } else
      hipLaunchKernelGGL((fp4_gemm_lds_kernel<2, kFp4WavesN>), dim3((unsigned)tiles),
                         dim3(64 * 2 * kFp4WavesN), 0, s, xq, xs, xt, wq, wsc, wt, y, M, N, K);
    return hipGetLastError();
  }
  int kbps, real;
  fp4_split_plan(N, K, &kbps, &real);
  float* part = real > 1 ? (float*)ws : nullptr;
  dim3 grid((unsigned)((N + 16 * kStreamWaves - 1) / (16 * kStreamWaves)), real);
  const int Mi = (int)M;
#define BSFP8_FP4S(MT)                                                                         \
  if (K % 128 == 0)                                                                            \
    hipLaunchKernelGGL((fp4_gemm_stream_kernel<MT, true>), grid, dim3(64 * kStreamWaves), 0, s, \
                       xq, xs, xt, wq, wsc, wt, y, part, Mi, N, K, kbps);                       \
  else                                                                                         \
    hipLaunchKernelGGL((fp4_gemm_stream_kernel<MT, false>), grid, dim3(64 * kStreamWaves), 0,   \
                       s, xq, xs, xt, wq, wsc, wt, y, part, Mi, N, K, kbps)
  if (M <= 16) {
    BSFP8_FP4S(1);
  } else if (M <= 32) {
    BSFP8_FP4S(2);
  } else {
    BSFP8_FP4S(4);
  }
#undef BSFP8_FP4S
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || part == nullptr) return e;
  const int64_t MN = M * N;
  hipLaunchKernelGGL(fp4_splitk_reduce, dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256), 0, s,
                     part, real, MN, N, y);
  return hipGetLastError();
}

}  // namespace bsfp8

