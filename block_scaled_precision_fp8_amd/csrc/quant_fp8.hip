// FP8 quantization kernels for gfx950.
//
//  * quant_act_kernel:    per-token 1x128 dynamic activation groups
//                         (fine-grained FP8 guide, section 一, second bullet)
//  * quant_weight_kernel: per 128x128 weight blocks
//                         (same section, first bullet; scale tensor shape
//                         (ceil(N/128), ceil(K/128)) from its third paragraph)
//
// Both are HBM-bound codecs: 2 bytes read and 1 byte written per element
// plus one scale per group.  Every read is a coalesced 16-byte load of eight
// bf16 values; every write is an 8-byte store of eight E4M3 codes.
//
// Scale formats (section 七 of the guide; readings for the open points):
//   FLOAT: s = fl32(amax / 448) (1.0 for amax == 0), code = E4M3(fl32(x / s))
//          with the correctly rounded fp32 quotient (reciprocal plus one
//          exact correction for a normal s, IEEE division otherwise).
//   UE8M0: s = 2^e, e = ceil(log2(amax / 448)) clamped to [-127, 127] (fp32
//          scales round *up* to UE8M0), code = E4M3(x * 2^-e) (exact scaling).
#include "bsfp8_internal.h"

namespace bsfp8 {
namespace detail {

constexpr int kActUnroll = 4;   // loads in flight per lane
constexpr int kActRows = 2;     // row sets per workgroup

struct Unpacked { float f[8]; };

__device__ __forceinline__ Unpacked unpack8(uint4 v) {
  Unpacked u;
  u.f[0] = bf16_lo(v.x); u.f[1] = bf16_hi(v.x);
  u.f[2] = bf16_lo(v.y); u.f[3] = bf16_hi(v.y);
  u.f[4] = bf16_lo(v.z); u.f[5] = bf16_hi(v.z);
  u.f[6] = bf16_lo(v.w); u.f[7] = bf16_hi(v.w);
  return u;
}

__device__ __forceinline__ float amax8(const Unpacked& u) {
  float a = fabsf(u.f[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) a = fmaxf(a, fabsf(u.f[i]));
  return a;
}

// Encode eight values of one group with the group's scale.  Returns the
// codes packed little-endian; writes the stored scale representation.
// fp32 scales divide by the correctly rounded reciprocal with one exact
// correction (div_by_rcp: the same E4M3 codes as IEEE x / s for a normal s,
// at four operations per value instead of an IEEE division each); a
// subnormal scale divides directly.
template <int FMT>
__device__ __forceinline__ uint2 encode8(const Unpacked& u, float amax, float* s_f32, int* s_exp) {
  const float s = FMT == 0 ? act_scale_f32(amax) : 0.0f;
  const int e = FMT == 0 ? 0 : ue8m0_exp(amax);
  *s_f32 = s;
  *s_exp = e;
  uint2 r;
  if (FMT == 0 && s >= kMinNormal) {
    const RcpDiv dv = rcp_div(s);
    r.x = act_encode4_rcp<FMT>(u.f[0], u.f[1], u.f[2], u.f[3], dv, e);
    r.y = act_encode4_rcp<FMT>(u.f[4], u.f[5], u.f[6], u.f[7], dv, e);
  } else {
    r.x = act_encode4<FMT>(u.f[0], u.f[1], u.f[2], u.f[3], s, e);
    r.y = act_encode4<FMT>(u.f[4], u.f[5], u.f[6], u.f[7], s, e);
  }
  return r;
}

// One 16-lane quarter-wave owns 128 consecutive values of one row: each lane
// holds eight consecutive bf16 values (one 16-byte load).  A workgroup of 16
// quarters covers QG consecutive 128-value chunks of RQ rows (QG * RQ = 16)
// and walks ROWS such row sets (kActRows = 2: many small workgroups keep more
// loads in flight across the chip than 8 row sets did -- 12-14% faster at
// 8192 x 4096 and 2048 x 14336 with fp32 scales, within 3% either way with
// UE8M0), with up to kActUnroll loads issued before use.
// GK is the group width: 128 (the quarter-wave is one group) or 32 (four
// lanes per group, for (32, 32) weight blocks); G counts 128-value chunks,
// GS the stored scales per row.
// STATIC: one calibrated scale for the whole tensor, read from `sscale`
// (fp32, or the E8M0 byte), replaces the group amax.
template <int FMT, bool STATIC, int GK, int ROWS>
__global__ __launch_bounds__(256) void quant_act_kernel(
    const uint16_t* __restrict__ x, int M, int K, int64_t ldx, int G, int qg_log2,
    uint8_t* __restrict__ xq, void* __restrict__ scale, const void* sscale) {
  static_assert(GK == 128 || GK == 32, "group width");
  constexpr int LPG = GK / 8;                // lanes per group
  const int GS = (K + GK - 1) / GK;
  const int tid = threadIdx.x;
  const int l16 = tid & 15;
  const int q = tid >> 4;
  const int QG = 1 << qg_log2;
  const int RQ = 16 >> qg_log2;
  const int g = blockIdx.x * QG + (q & (QG - 1));
  const int k0 = g * kBlock + l16 * 8;
  const bool gvalid = g < G;
  const bool kvalid = gvalid && k0 < K;
  constexpr int UN = ROWS < kActUnroll ? ROWS : kActUnroll;
  for (int mb = blockIdx.y; mb * (RQ * ROWS) < M; mb += gridDim.y) {
  const int mbase = mb * (RQ * ROWS) + (q >> qg_log2);
#pragma unroll
  for (int jb = 0; jb < ROWS; jb += UN) {
    uint4 v[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int m = mbase + RQ * (jb + u);
      v[u] = make_uint4(0, 0, 0, 0);
      if (kvalid && m < M)
        v[u] = ld_stream16(x + (int64_t)m * ldx + k0);
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int m = mbase + RQ * (jb + u);
      const Unpacked f = unpack8(v[u]);
      float sf = 0.0f;
      int se = 0;
      uint2 codes;
      if constexpr (STATIC) {
        if (FMT == 0) sf = *(const float*)sscale;
        else se = (int)*(const uint8_t*)sscale - 127;
        codes.x = act_encode4<FMT>(f.f[0], f.f[1], f.f[2], f.f[3], sf, se);
        codes.y = act_encode4<FMT>(f.f[4], f.f[5], f.f[6], f.f[7], sf, se);
      } else {
        float amax = amax8(f);
#pragma unroll
        for (int o = 1; o < LPG; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
        codes = encode8<FMT>(f, amax, &sf, &se);
      }
      if (m < M) {
        if (kvalid) *(uint2*)(xq + (int64_t)m * K + k0) = codes;
        // the group's first lane stores its scale (a group exists when its
        // first element is in range)
        if (kvalid && (l16 & (LPG - 1)) == 0) {
          const int64_t gi = (int64_t)m * GS + k0 / GK;
          if (FMT == 0) ((float*)scale)[gi] = sf;
          else ((uint8_t*)scale)[gi] = (uint8_t)(se + 127);
        }
      }
    }
  }
  }
}

// One workgroup per 128x128 tile of W.  Thread t loads column chunk
// (t % 16) of rows (t / 16) + 16 i, i = 0..7: each wave reads four full
// 256-byte row segments per load instruction.  BLK = 128: the tile is one
// weight block.  BLK = 32: the tile holds 4 x 4 blocks of 32 x 32; block
// (rb, cb) is rows 32 rb + {r0, r0 + 16} (loads 2 rb and 2 rb + 1) and
// column chunks 4 cb .. 4 cb + 3, so its amax gathers over lanes xor 1, 2
// (chunks), xor 16, 32 (rows within a wave) and the four waves.
template <int FMT, int BLK = 128>
__global__ __launch_bounds__(256) void quant_weight_kernel(
    const uint16_t* __restrict__ w, int N, int K, int64_t ldw, int KB,
    uint8_t* __restrict__ wq, void* __restrict__ scale) {
  static_assert(BLK == 128 || BLK == 32, "block size");
  constexpr int NSB = kBlock / BLK;          // blocks per tile side
  __shared__ float red[4][NSB][NSB];
  const int kb = blockIdx.x, nb = blockIdx.y;
  const int t = threadIdx.x;
  const int ch = t & 15, r0 = t >> 4;
  const int k0 = kb * kBlock + ch * 8;
  const bool kvalid = k0 < K;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int n = nb * kBlock + r0 + 16 * i;
    v[i] = make_uint4(0, 0, 0, 0);
    if (kvalid && n < N)
      v[i] = ld_stream16(w + (int64_t)n * ldw + k0);
  }
  // per block row rb (loads i with i * NSB / 8 == rb): lane-local amax, then
  // over the lanes and waves that share the block
  float amax[NSB];
#pragma unroll
  for (int rb = 0; rb < NSB; ++rb) amax[rb] = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax[i * NSB / 8] = fmaxf(amax[i * NSB / 8], amax8(unpack8(v[i])));
  const int cb = ch / (16 / NSB);
#pragma unroll
  for (int rb = 0; rb < NSB; ++rb) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      if (BLK == 32 && (o == 4 || o == 8)) continue;    // keep column blocks apart
      amax[rb] = fmaxf(amax[rb], __shfl_xor(amax[rb], o, 64));
    }
    if ((t & 63) == cb * (16 / NSB)) red[t >> 6][rb][cb] = amax[rb];
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < NSB; ++rb)
    amax[rb] = fmaxf(fmaxf(red[0][rb][cb], red[1][rb][cb]), fmaxf(red[2][rb][cb], red[3][rb][cb]));

  float sf[NSB];
  int se[NSB];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rb = i * NSB / 8;
    const int n = nb * kBlock + r0 + 16 * i;
    const uint2 codes = encode8<FMT>(unpack8(v[i]), amax[rb], &sf[rb], &se[rb]);
    if (kvalid && n < N) *(uint2*)(wq + (int64_t)n * K + k0) = codes;
  }
  // one thread per block stores its scale: rows r0 == 0, first chunk of cb
  if (r0 == 0 && (ch % (16 / NSB)) == 0 && kvalid) {
    const int KS = (K + BLK - 1) / BLK;
#pragma unroll
    for (int rb = 0; rb < NSB; ++rb) {
      const int nbs = nb * NSB + rb, kbs = kb * NSB + cb;
      if (nbs * BLK >= N) continue;
      const int64_t gi = (int64_t)nbs * KS + kbs;
      if (FMT == 0) ((float*)scale)[gi] = sf[rb];
      else ((uint8_t*)scale)[gi] = (uint8_t)(se[rb] + 127);
    }
  }
}

}  // namespace detail
using namespace detail;

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int fmt,
                            uint8_t* xq, void* scale, hipStream_t s, const void* static_scale,
                            int group_k) {
  const int G = (int)((K + kBlock - 1) / kBlock);
  int qg_log2 = 0;
  while ((1 << qg_log2) < G && qg_log2 < 4) ++qg_log2;
  const int QG = 1 << qg_log2, RQ = 16 >> qg_log2;
  int64_t gy = (M + RQ * kActRows - 1) / (RQ * kActRows);
  if (gy > 65535) gy = 65535;
  dim3 grid((G + QG - 1) / QG, (unsigned)gy);
#define BSFP8_ACT(F, S, GK)                                                                        \
  hipLaunchKernelGGL((quant_act_kernel<F, S, GK, kActRows>), grid, dim3(256), 0, s, x, (int)M,  \
                     (int)K, ldx, G, qg_log2, xq, scale, static_scale)
  if (static_scale) {
    if (fmt == 0) BSFP8_ACT(0, true, 128); else BSFP8_ACT(1, true, 128);
  } else if (group_k == 32) {
    if (fmt == 0) BSFP8_ACT(0, false, 32); else BSFP8_ACT(1, false, 32);
  } else {
    if (fmt == 0) BSFP8_ACT(0, false, 128); else BSFP8_ACT(1, false, 128);
  }
#undef BSFP8_ACT
  return hipGetLastError();
}

hipError_t launch_quant_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, int fmt,
                               uint8_t* wq, void* scale, hipStream_t s, int block) {
  const int KB = (int)((K + kBlock - 1) / kBlock);
  const int NB = (int)((N + kBlock - 1) / kBlock);
  dim3 grid(KB, NB);
#define BSFP8_WQ(F, B)                                                                        \
  hipLaunchKernelGGL((quant_weight_kernel<F, B>), grid, dim3(256), 0, s, w, (int)N, (int)K, ldw, \
                     KB, wq, scale)
  if (block == 32) {
    if (fmt == 0) BSFP8_WQ(0, 32); else BSFP8_WQ(1, 32);
  } else {
    if (fmt == 0) BSFP8_WQ(0, 128); else BSFP8_WQ(1, 128);
  }
#undef BSFP8_WQ
  return hipGetLastError();
}

}  // namespace bsfp8
