// Block-scaled FP8 GEMM kernels for gfx950 (CDNA4).
//
//   Y[m][n] = bf16( sum_kb S_a[m][kb] S_w[n/128][kb] sum_{k in kb} Xq[m][k] Wq[n][k] + bias[n] )
//
// The activation groups and weight blocks share the 128-wide K blocks, so
// the product runs block by block (fine-grained FP8 guide, section 一).  On
// gfx950 one V_MFMA_SCALE_F32_16X16X128_F8F6F4 consumes exactly one 128-deep
// K block of a 16x16 output tile, so each MFMA result is one fp32 partial
// sum that gets one scale:
//   * fp32 scales: tmp = MFMA(Wfrag, Xfrag, 0); acc += tmp * (S_a * S_w).
//     W is the MFMA A operand (output rows = n) and X the B operand (output
//     columns = m), so every lane's four accumulators share one token m and
//     one 128-row weight block: one scale product per lane per K block.
//   * UE8M0 scales: the power-of-two scales are passed straight to the MFMA
//     as its E8M0 block-scale operands (exact), and the MFMA accumulates in
//     place: no vector ALU work in the K loop at all.
//
// Kernels:
//   gemm_lds_kernel     M > 16: workgroup tile BM x BN, operands staged in
//                       LDS (double-buffered, XOR-swizzled 16-byte chunks),
//                       XCD-aware tile order, optional split-K into fp32
//                       partials.  Also serves the MoE grouped GEMM through
//                       a device-built tile table.
//   gemm_decode_kernel  M <= 16: weight-streaming kernel, one launch, with
//                       the activation quantization fused for fp8_linear.
//   splitk_reduce_kernel  fp32 partials -> bf16 (+ bias).
#include <algorithm>
#include <type_traits>

#include "bsfp8.h"
#include "bsfp8_internal.h"

namespace bsfp8 {
namespace detail {

constexpr int kRowBytes = 128;   // one K block of FP8 codes

__device__ __forceinline__ v8i join(uint4 a, uint4 b) {
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

// compile-time loop: f(std::integral_constant<int, 0>) .. f(<N - 1>)
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

template <int FMT>
__device__ __forceinline__ float load_scale(const void* p, int64_t idx) {
  if (FMT == 0) return ((const float*)p)[idx];
  return __int_as_float(((const uint8_t*)p)[idx]);   // carries the byte
}

__device__ __forceinline__ float e8m0_f32(uint32_t b) {
  return __uint_as_float(b == 0 ? 0x00400000u : b << 23);   // 2^(b - 127)
}

// MFMA step for one 16x16 tile and one K block.
template <int FMT>
__device__ __forceinline__ v4f mfma_step(v4f acc, const v8i& a, const v8i& b, float sa,
                                         float sw) {
  if (FMT == 0) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    v4f t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 127, 0, 127);
    const float c = sa * sw;
    acc[0] = fmaf(t[0], c, acc[0]);
    acc[1] = fmaf(t[1], c, acc[1]);
    acc[2] = fmaf(t[2], c, acc[2]);
    acc[3] = fmaf(t[3], c, acc[3]);
    return acc;
  } else {
    // A = W (scale S_w), B = X (scale S_a); E8M0 bytes in bits [7:0].
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        a, b, acc, 0, 0, 0, __float_as_int(sw), 0, __float_as_int(sa));
  }
}

// MFMA step with an MXFP4 weight fragment (A operand, format E2M1: 16
// bytes per lane in the low half of the register block) and its lane's
// E8M0 block scale (the 32 weights this lane carries); X stays FP8.
template <int FMT>
__device__ __forceinline__ v4f mfma_step_w4(v4f acc, const v8i& a, const v8i& b, float sa,
                                            int sw4) {
  if (FMT == 0) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    v4f t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 4, 0, 0, sw4, 0, 127);
    acc[0] = fmaf(t[0], sa, acc[0]);
    acc[1] = fmaf(t[1], sa, acc[1]);
    acc[2] = fmaf(t[2], sa, acc[2]);
    acc[3] = fmaf(t[3], sa, acc[3]);
    return acc;
  } else {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 4, 0, 0, sw4, 0,
                                                            __float_as_int(sa));
  }
}

// bf16 epilogue for four consecutive n of one row m.
__device__ __forceinline__ void store_out4(uint16_t* y, int64_t N, int64_t m, int64_t n, v4f v,
                                           const uint16_t* bias) {
  if (bias) {
    const uint2 b = *(const uint2*)(bias + n);
    v[0] += bf16_lo(b.x); v[1] += bf16_hi(b.x);
    v[2] += bf16_lo(b.y); v[3] += bf16_hi(b.y);
  }
  uint2 o;
  o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
  o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
  *(uint2*)(y + m * N + n) = o;
}

// ------------------------------------------------------------------------
// Large-M kernel.
// ------------------------------------------------------------------------
struct Tile {
  int64_t m0, mlim;   // rows [m0, min(m0 + BM, mlim))
  int64_t n0;
  int expert;
  int split;          // K split (dense split-K launches), else 0
  bool valid;
};

template <int BM, int BN>
__device__ __forceinline__ Tile dense_tile(int64_t M, int64_t N, int splits) {
  const int MT = (int)((M + BM - 1) / BM), NT = (int)((N + BN - 1) / BN);
  const int T = MT * NT;
  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so
  // bid -> (xcd, slot) and consecutive logical tiles go to one XCD.
  const int bid = blockIdx.x;
  const int per_xcd = (int)(gridDim.x / 8);
  int t = (bid & 7) * per_xcd + (bid >> 3);
  Tile tl;
  tl.valid = t < T * splits;
  tl.expert = 0;
  // K splits outermost: the tiles of one split run together
  tl.split = t / T;
  t -= tl.split * T;
  // grouped order: groups of 8 M tiles, M fastest, so 8 x k tiles that run
  // together share their X rows and W columns.
  constexpr int GM = 8;
  const int group = t / (GM * NT);
  const int first_m = group * GM;
  const int gsz = min(MT - first_m, GM);
  const int in = t - group * GM * NT;
  const int tm = first_m + (gsz > 0 ? in % gsz : 0);
  const int tn = gsz > 0 ? in / gsz : 0;
  tl.m0 = (int64_t)tm * BM;
  tl.mlim = M;
  tl.n0 = (int64_t)tn * BN;
  return tl;
}

// Grouped tile table, built by every workgroup in LDS from the device
// segment offsets: expert e owns mt_e = ceil(rows_e / BM) M tiles and all NT
// N tiles; tiles are numbered expert by expert, then N tile, then M tile
// (M fastest, so the M tiles of one expert's weight tile run together).
// gsel picks the experts a launch covers: 0 all, 1 those with more than
// kSmallSegment rows, 2 the others (each class runs on its own tile shape).
// XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so
// workgroup b takes logical tile (b % 8) ceil(total / 8) + b / 8 -- each XCD
// a contiguous eighth of the (device-known) tile count -- and the M tiles
// of one weight tile, and the N tiles of one expert, meet in one L2 (dealt
// in launch order they landed on different XCDs and re-read the weights
// from HBM: 12.1 GB read for 7.5 GB of gate/up experts).  The grid is the
// host's upper bound on the count, a multiple of 8.
constexpr int kSmallSegment = 128;

template <int BM, int BN, int THREADS>
__device__ __forceinline__ Tile grouped_tile(const int32_t* __restrict__ seg, int E, int64_t N,
                                             int* s_pref, int gsel) {
  const int NT = (int)((N + BN - 1) / BN);
  // per-expert M-tile counts, then an inclusive scan (Hillis-Steele).
  for (int e = threadIdx.x; e < E; e += THREADS) {
    const int rows = seg[e + 1] - seg[e];
    const bool take = gsel == 0 || ((rows > kSmallSegment) == (gsel == 1));
    s_pref[e + 1] = take ? (rows + BM - 1) / BM : 0;
  }
  if (threadIdx.x == 0) s_pref[0] = 0;
  __syncthreads();
  for (int d = 1; d < E; d <<= 1) {
    int v[4];
    int c = 0;
    for (int e = threadIdx.x; e < E; e += THREADS, ++c)
      v[c] = (e >= d) ? s_pref[e + 1 - d] : 0;
    __syncthreads();
    c = 0;
    for (int e = threadIdx.x; e < E; e += THREADS, ++c) s_pref[e + 1] += v[c];
    __syncthreads();
  }
  Tile tl;
  tl.split = 0;
  const int total = s_pref[E] * NT;
  const int per_xcd = (total + 7) / 8;
  const int bid = blockIdx.x;
  const int t = (bid & 7) * per_xcd + (bid >> 3);
  tl.valid = (bid >> 3) < per_xcd && t < total;
  tl.expert = 0;
  tl.m0 = 0; tl.mlim = 0; tl.n0 = 0;
  if (!tl.valid) return tl;
  // binary search: largest e with s_pref[e] * NT <= t
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] * NT <= t) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int mt_e = s_pref[e + 1] - s_pref[e];
  const int local = t - s_pref[e] * NT;
  const int tn = local / mt_e, tm = local - tn * mt_e;
  tl.expert = e;
  tl.m0 = (int64_t)seg[e] + (int64_t)tm * BM;
  tl.mlim = seg[e + 1];
  tl.n0 = (int64_t)tn * BN;
  return tl;
}

// One fragment read from LDS.  The restrict-qualified pointer gives the
// loads alias-scope information; without it the compiler assumes they may
// read what the in-flight LDS-DMA of the next stage writes and waits for
// that DMA first, which would serialise the prefetch with the MFMAs.
__device__ __forceinline__ v8i read_frag(const uint8_t* __restrict__ row, int ch0, int ch1) {
  return join(*(const uint4*)(row + ch0), *(const uint4*)(row + ch1));
}
// an MXFP4 weight fragment: one 16-byte chunk per lane.  Like read_frag, it
// reads through a restrict-qualified pointer: the alias scope that gives
// the load lets the compiler see that it does not read the stage the DMA
// in flight writes (a plain dereference made it wait for all of that DMA
// before every W4 fragment read).
__device__ __forceinline__ v8i read_frag_w4(const uint8_t* __restrict__ row, int chw) {
  return join(*(const uint4*)(row + chw), make_uint4(0, 0, 0, 0));
}
// a staged scale, read the same way (no wait for the in-flight DMA)
__device__ __forceinline__ float read_scale(const float* __restrict__ p, int idx) { return p[idx]; }
__device__ __forceinline__ uint32_t read_byte(const uint8_t* __restrict__ p, int idx) { return p[idx]; }
__device__ __forceinline__ uint32_t read_u32(const uint8_t* __restrict__ p, int off) {
  return *(const uint32_t*)(p + off);
}
__device__ __forceinline__ long read_u64(const uint8_t* __restrict__ p, int off) {
  return *(const long*)(p + off);
}
__device__ __forceinline__ float4 read_scale4(const uint8_t* __restrict__ p, int off) {
  return *(const float4*)(p + off);
}

// SiLU(gate) * up with the 1 x 128 requantization, for a gate/up tile of
// the grouped GEMM (the step between an MoE expert's gate/up and down
// GEMMs).  Waves wn < WAVES_N / 2 hold the gate values of h columns
// c0 + (wn WN .. wn WN + WN), wave wn + WAVES_N / 2 the up values of the same
// columns in the same lane layout: the up waves hand their accumulators over
// through the (drained) LDS stage buffers, each gate lane forms
// h = silu(g) u in fp32 and rounds it to bf16, and the 128 columns of a token
// row -- one activation group -- are quantized with the activation codec:
// amax over the lanes (and waves) that share the row, then the scale and the
// codes fp8_quant_act would write for that bf16 row.  h_bf16 (nullable)
// receives the rounded h.
template <int FMT, int WAVES_M, int WAVES_N, int WM, int WN>
__device__ __forceinline__ void swiglu_epilogue(v4f (&acc)[WN / 16][WM / 16], uint8_t* lds,
                                                const Tile& tl, int wm, int wn, int lane,
                                                int64_t I, int64_t c0, uint16_t* h_bf16,
                                                uint8_t* hq, void* hs) {
  constexpr int NI = WN / 16, MI = WM / 16;
  constexpr int HALF = WAVES_N / 2;
  constexpr int XCH = WAVES_M * HALF * NI * MI * 64 * 16;   // bytes of handed-over tiles
  const int l16 = lane & 15, g4 = lane >> 4;
  const bool upw = wn >= HALF;
  const int pair = wm * HALF + (wn % HALF);
  v4f* xch = (v4f*)lds + (int64_t)pair * NI * MI * 64;
  float* amx = (float*)(lds + XCH);                    // [WAVES_M][HALF][MI][16]
  __syncthreads();        // every DMA landed, every fragment read done
  if (upw) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j) xch[(i * MI + j) * 64 + lane] = acc[i][j];
  }
  __syncthreads();
  // h of one accumulator tile: bf16(silu(g) * u), as a float
  auto h4 = [&](int i, int j) -> v4f {
    const v4f u = xch[(i * MI + j) * 64 + lane];
    v4f h;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float g = acc[i][j][q];
      h[q] = __uint_as_float(f32_to_bf16(g / (1.0f + expf(-g)) * u[q]) << 16);
    }
    return h;
  };
  // pass 1: the row maxima of |h| (acc stays read-only: both passes form h)
  float amax[MI];
#pragma unroll
  for (int j = 0; j < MI; ++j) amax[j] = 0.0f;
  if (!upw) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int j = 0; j < MI; ++j) {
        const v4f h = h4(i, j);
        amax[j] = fmaxf(amax[j], fmaxf(fmaxf(fabsf(h[0]), fabsf(h[1])),
                                       fmaxf(fabsf(h[2]), fabsf(h[3]))));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < MI; ++j) {
      amax[j] = fmaxf(amax[j], __shfl_xor(amax[j], 16));
      amax[j] = fmaxf(amax[j], __shfl_xor(amax[j], 32));
    }
    if (HALF > 1 && g4 == 0) {
#pragma unroll
      for (int j = 0; j < MI; ++j) amx[((wm * HALF + wn) * MI + j) * 16 + l16] = amax[j];
    }
  }
  if constexpr (HALF > 1) {
    __syncthreads();
    if (!upw) {
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int h2 = 0; h2 < HALF; ++h2)
          amax[j] = fmaxf(amax[j], amx[((wm * HALF + h2) * MI + j) * 16 + l16]);
    }
  }
  if (upw) return;
  // pass 2: scales, codes, stores
  const int64_t G = I / 128;
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    const int64_t m = tl.m0 + wm * WM + j * 16 + l16;
    if (m >= tl.mlim) continue;
    const float s = FMT == 0 ? act_scale_f32(amax[j]) : 0.0f;
    const int e = FMT == 0 ? 0 : ue8m0_exp(amax[j]);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int64_t c = c0 + wn * WN + i * 16 + 4 * g4;
      const v4f v = h4(i, j);
      *(uint32_t*)(hq + m * I + c) = act_encode4<FMT>(v[0], v[1], v[2], v[3], s, e);
      if (h_bf16) {
        uint2 o;
        o.x = (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xffff0000u);
        o.y = (__float_as_uint(v[2]) >> 16) | (__float_as_uint(v[3]) & 0xffff0000u);
        *(uint2*)(h_bf16 + m * I + c) = o;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (wn == 0 && g4 == 0) {
      if (FMT == 0) ((float*)hs)[m * G + c0 / 128] = s;
      else ((uint8_t*)hs)[m * G + c0 / 128] = (uint8_t)(e + 127);
    }
  }
}

// Workgroup tile BM x BN = (WAVES_M * WM) x (WAVES_N * WN), K step 128 (one
// scale block).  Operands go global -> LDS directly (buffer_load ... lds,
// 16 bytes per lane), double-buffered; in LDS every 128-byte row keeps
// its eight 16-byte chunks XOR-swizzled by ((row >> 1) & 7).  The LDS has
// 64 four-byte banks (two 128-byte rows per sweep); a fragment read has 16
// lanes on 16 consecutive rows and one logical chunk, so (row parity,
// physical chunk) must be distinct over any 16 consecutive rows -- which
// this swizzle gives.  Each wave
// computes a WM (m) x WN (n) tile with 16x16x128 MFMAs: W is the A operand,
// X the B operand.
//
// W4: W holds MXFP4 codes (N, K/2) with one E8M0 scale per 1 x 32 group
// (N, K/32).  A W row is then 64 bytes per K block, four 16-byte chunks
// swizzled by ((row >> 2) & 3) (four rows per bank sweep); lane (l16, g4)
// takes chunk g4, the weights K 32 g4 .. 32 g4 + 31, which the MFMA pairs
// with the X chunks g4 and g4 + 4 of the FP8 operand (the lane layout of
// the FP4 x FP8 form, checked on the GPU), and passes its own group's scale.
template <int FMT, int WAVES_M, int WAVES_N, int WM, int WN, bool GROUPED, bool W4 = false,
          bool SWIGLU = false, bool SA = false, bool SW4 = false, bool XQ = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void gemm_lds_kernel(
    const uint8_t* __restrict__ xq, const void* __restrict__ xs, const uint8_t* __restrict__ wq,
    const void* __restrict__ wsc, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int64_t M, int64_t N, int64_t K, const int32_t* __restrict__ seg, int E, int gsel,
    float* __restrict__ part, int kbps, uint8_t* __restrict__ hq, void* __restrict__ hs,
    const uint16_t* __restrict__ xb, int64_t ldx) {
  // The body exists only in the device pass; the host pass needs nothing
  // but the launch stub of each instantiation.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int STAGES = 2;
  constexpr int WAVES = WAVES_M * WAVES_N;
  constexpr int THREADS = 64 * WAVES;
  constexpr int BM = WAVES_M * WM, BN = WAVES_N * WN;
  constexpr int MI = WM / 16, NI = WN / 16;
  static_assert(WN == 64 || WN == 128, "a wave's N range lies inside one weight block");
  static_assert(!SWIGLU || (GROUPED && !W4 && WAVES_N % 2 == 0 && WAVES_N / 2 * WN == 128),
                "SiLU-mul tiles: 128 gate rows then the 128 matching up rows");
  constexpr int kWRow = W4 ? 64 : kRowBytes;   // W bytes per row per K block
  constexpr int XJ = BM * 8 / THREADS;      // DMA loads per lane per stage (X)
  constexpr int WJ = BN * (kWRow / 16) / THREADS;   // (W)
  static_assert(XJ * THREADS == BM * 8 && WJ * THREADS == BN * (kWRow / 16), "tile / thread mismatch");
  constexpr int XBYTES = BM * kRowBytes;
  constexpr int STAGE = BM * kRowBytes + BN * kWRow;
  constexpr int SB = FMT == 0 ? 4 : 1;      // bytes per scale
  // The activation scales of tiles of at least 128 rows are staged through
  // LDS, SCH K blocks per chunk (8 fp32 or 16 UE8M0 scales, SROW bytes): one
  // row's chunk is one request, where loading each row's scale block by
  // block costs a request per row and K block (the rows of one K block are
  // a row stride apart).  UE8M0 rows are K/128 bytes apart: their chunks
  // are dword-aligned only when K/128 and the split length are multiples of
  // 4, so the launcher picks the staged instantiation (SA) then and the
  // per-block loads otherwise.  (A runtime choice between the two would
  // make the compiler wait for every load of the step before using the
  // per-block scales, the next stage's DMA included.)
  // XQ: X arrives as bf16 and is quantized here, one K block at a time
  // (fp8_linear's fused large-M form): each stage's 1 x 128 act groups are
  // loaded into registers with the weight DMA, encoded with the activation
  // codec once they land, and written to the stage's X tile and to a
  // per-stage scale row in LDS.  xs is then null (dynamic groups) or the
  // static scheme's calibrated scale.
  static_assert(!XQ || (!GROUPED && !W4 && !SWIGLU && !SA && BM == 128 && THREADS == 512),
                "fused act quant: dense 128 x 256 tiles");
  constexpr int XQJ = XQ ? BM * 16 / THREADS : 1;   // 16-byte bf16 loads per lane per stage
  constexpr bool SCL = !XQ && BM >= 128 && (FMT == 0 || (SA && !SWIGLU));
  constexpr int SCH = FMT == 0 ? 8 : 16;
  constexpr int SROW = SCH * SB;            // bytes per row per chunk
  constexpr int SDW = SROW / 4;             // dword loads per row per chunk
  constexpr int SBUF = BM * SROW;           // bytes per chunk buffer
  constexpr int SJ = SCL ? BM * SDW / (64 * WAVES) : 0;   // chunk DMA loads per lane
  static_assert(!SCL || SJ * 64 * WAVES == BM * SDW, "scale chunk / thread mismatch");
  // MXFP4 weight scales (SW4, K a multiple of 128 so every row's 4 bytes per
  // K block are dword-aligned) are staged the same way, 8 K blocks (32 bytes)
  // per weight row per chunk, instead of one byte load per lane, subtile and
  // K block (16 rows, so 16 requests, per load)
  static_assert(!SW4 || W4, "staged MXFP4 scales need MXFP4 weights");
  constexpr int WCH = 8;
  constexpr int WBUF = BN * 32;
  constexpr int WSJ = SW4 ? BN * 8 / (64 * WAVES) : 0;
  static_assert(!SW4 || WSJ * 64 * WAVES == BN * 8, "weight-scale chunk / thread mismatch");
  __shared__ __attribute__((aligned(1024)))
  uint8_t lds[STAGES * STAGE + (SCL ? 2 * SBUF : 0) + (SW4 ? 2 * WBUF : 0) + (XQ ? 2 * BM * 4 : 0)];
  uint8_t* const sbuf = lds + STAGES * STAGE;
  uint8_t* const wbuf = sbuf + (SCL ? 2 * SBUF : 0);
  float* const sxq = (float*)(wbuf + (SW4 ? 2 * WBUF : 0));   // XQ: [2][BM] scales
  static_assert(!GROUPED || STAGES * STAGE >= 1025 * 4, "tile table fits the stage buffers");
  static_assert(!SWIGLU || WAVES_M * (WAVES_N / 2) * MI * NI * 1024 +
                               (WAVES_N > 2 ? WAVES_M * (WAVES_N / 2) * MI * 64 : 0) <=
                           STAGES * STAGE,
                "the up tiles and row maxima fit the stage buffers");

  Tile tl;
  // the grouped tile table lives in the stage buffers until the tile is known
  if (GROUPED) tl = grouped_tile<BM, BN, THREADS>(seg, E, N, (int*)lds, gsel);
  else tl = dense_tile<BM, BN>(M, N, part ? (int)(((K + 127) / 128 + kbps - 1) / kbps) : 1);
  if (!tl.valid) return;
  if (GROUPED) __syncthreads();            // every lookup done before the first DMA

  const int KB = (int)((K + 127) / 128);
  // this workgroup's K blocks [kb_begin, kb_end): all of K, or its split
  const int kb_begin = part ? tl.split * kbps : 0;
  const int kb_end = part ? min(KB, kb_begin + kbps) : KB;
  const int64_t NB = (N + 127) / 128;
  const int64_t KW = W4 ? K / 2 : K;         // W bytes per row
  const int64_t G32 = K / 32;                // MXFP4 scales per row
  // this tile's expert: weights (E, N, KW), FP8 block scales (E, NB, KB) or
  // MXFP4 group scales (E, N, K/32)
  const uint8_t* wbase = wq + (int64_t)tl.expert * N * KW;
  const uint8_t* wsb = (const uint8_t*)wsc + (int64_t)tl.expert * NB * KB * SB;
  const uint8_t* wsb4 = (const uint8_t*)wsc + (int64_t)tl.expert * N * G32;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int l16 = lane & 15, g4 = lane >> 4;

  const int64_t mrows = min((int64_t)BM, tl.mlim - tl.m0);
  const int64_t nrows = min((int64_t)BN, N - tl.n0);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xq + tl.m0 * K, mrows * K);
  // SWIGLU: N = 2 I weight rows, gate rows [0, I) then up rows [I, 2 I); an
  // N tile at n0 = 256 t covers h columns [128 t, 128 t + 128): its rows
  // [0, 128) are gate rows 128 t + r, rows [128, 256) the up rows I + 128 t + r
  const int64_t I = N / 2, c0 = tl.n0 / 2;
  auto wrow_of = [&](int r) -> int64_t { return r < 128 ? c0 + r : I + c0 + (r - 128); };
  const __amdgpu_buffer_rsrc_t rw = SWIGLU ? make_rsrc(wbase, N * K)
                                           : make_rsrc(wbase + tl.n0 * KW, nrows * KW);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc((const uint8_t*)xs + tl.m0 * KB * SB,
                                               mrows * KB * SB);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(wsb, NB * KB * SB);

  // per-lane DMA source for LDS chunk q of a tile: row q / 8 holds, in its
  // physical chunk q % 8, the logical chunk (q % 8) ^ ((row >> 1) & 7)
  auto dma_src = [&](int q, int64_t rows, uint32_t kbyte) -> uint32_t {
    const int row = q >> 3, c = (q & 7) ^ ((row >> 1) & 7);
    const uint32_t kc = kbyte + c * 16;
    return (row < rows && kc < (uint32_t)K) ? (uint32_t)(row * K) + kc : kOOB;
  };
  // the same for W rows of a gate/up tile (rows from both halves of W)
  auto dma_src_gu = [&](int q, uint32_t kbyte) -> uint32_t {
    const int row = q >> 3, c = (q & 7) ^ ((row >> 1) & 7);
    const uint32_t kc = kbyte + c * 16;
    return kc < (uint32_t)K ? (uint32_t)(wrow_of(row) * K) + kc : kOOB;
  };
  // the same for a 64-byte MXFP4 W row: four chunks, swizzle (row >> 2) & 3
  auto dma_src4 = [&](int q, int64_t rows, int kb) -> uint32_t {
    const int row = q >> 2, c = (q & 3) ^ ((row >> 2) & 3);
    const uint32_t kc = (uint32_t)kb * 64 + c * 16;
    return (row < rows && kc < (uint32_t)KW) ? (uint32_t)(row * KW) + kc : kOOB;
  };
  // MXFP4 weight scales: lane row of each 16-row subtile, group 4 kb + g4
  const __amdgpu_buffer_rsrc_t rsw4 = make_rsrc(wsb4 + tl.n0 * G32, W4 ? nrows * G32 : 0);
  // scale sources: this lane's token rows, and this wave's weight block
  uint32_t saoff[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int r = wm * WM + i * 16 + l16;
    saoff[i] = r < mrows ? (uint32_t)(r * KB * SB) : kOOB;
  }
  const int64_t nwave = tl.n0 + wn * WN;
  const int64_t nwave_w = SWIGLU ? wrow_of(wn * WN) : nwave;   // its first weight row
  const uint32_t swoff = nwave < N ? (uint32_t)((nwave_w >> 7) * KB * SB) : kOOB;

  float sa_reg[STAGES][MI];
  float sw_reg[STAGES];
  int sw4_reg[STAGES][W4 && !SW4 ? NI : 1];
  // XQ: the next stage's bf16 X, 16 bytes per load; lane t takes row q / 16,
  // 8-value chunk q % 16 of the K block (q = j THREADS + t), so the 16 lanes
  // of a row are one quarter-wave
  u32x4 xr[XQJ];
  const uint16_t* const xrow = XQ ? xb + tl.m0 * ldx : nullptr;   // this tile's first row

  // issue one stage: X and W tiles into LDS buffer `buf`, scales into
  // registers; exactly LOADS vector-memory ops per lane, in this order.
  // part 1 issues the X tile only, part 2 the rest (0: all).
  auto issue = [&](int kb, int buf, int part = 0) {
    uint8_t* sx = lds + buf * STAGE;
    uint8_t* sw = sx + XBYTES;
    const uint32_t kbyte = (uint32_t)kb * 128;
    if constexpr (XQ) {
#pragma unroll
      for (int j = 0; j < XQJ; ++j) {
        const int q = j * THREADS + (int)threadIdx.x;
        const int row = q >> 4;
        const int64_t k = (int64_t)kbyte + (q & 15) * 8;
        xr[j] = u32x4{0u, 0u, 0u, 0u};
        if (row < mrows && k < K) xr[j] = *(const u32x4*)(xrow + row * ldx + k);
      }
    } else if (part != 2) {
#pragma unroll
      for (int j = 0; j < XJ; ++j) {
        const int q = (j * WAVES + wave) * 64 + lane;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, BSFP8_LDS(sx + (j * WAVES + wave) * 1024),
                                                 16, dma_src(q, mrows, kbyte), 0, 0, 0);
      }
    }
    if (part == 1) return;
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
      const int q = (j * WAVES + wave) * 64 + lane;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, BSFP8_LDS(sw + (j * WAVES + wave) * 1024), 16,
          W4 ? dma_src4(q, nrows, kb) : SWIGLU ? dma_src_gu(q, kbyte) : dma_src(q, nrows, kbyte),
          0, 0, 0);
    }
    if constexpr (SCL) {
      // at the first K block of a chunk: rows x SCH scales into its buffer,
      // row-major (lane q: row q / SDW, dword q % SDW of the row's chunk;
      // blocks past the end load other rows' scales or zeros and are never
      // read)
      const int rel = kb - kb_begin;
      if (rel % SCH == 0) {
        uint8_t* dst = sbuf + ((rel / SCH) & 1) * SBUF;
#pragma unroll
        for (int j = 0; j < SJ; ++j) {
          const int q = (j * WAVES + wave) * 64 + lane;
          const int row = q / SDW;
          const uint32_t off =
              row < mrows ? (uint32_t)((row * KB + kb) * SB + (q % SDW) * 4) : kOOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, BSFP8_LDS(dst + (j * WAVES + wave) * 256), 4,
                                                   off, 0, 0, 0);
        }
      }
    } else if constexpr (!XQ) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const uint32_t off = saoff[i] == kOOB ? kOOB : saoff[i] + kb * SB;
        if (FMT == 0) sa_reg[buf][i] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsa, off, 0, 0));
        else sa_reg[buf][i] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b8(rsa, off, 0, 0));
      }
    }
    if constexpr (SW4) {
      const int rel = kb - kb_begin;
      if (rel % WCH == 0) {
        uint8_t* dst = wbuf + ((rel / WCH) & 1) * WBUF;
#pragma unroll
        for (int j = 0; j < WSJ; ++j) {
          const int q = (j * WAVES + wave) * 64 + lane;
          const int row = q >> 3;
          const uint32_t off = row < nrows ? (uint32_t)(row * G32 + kb * 4 + (q & 7) * 4) : kOOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw4, BSFP8_LDS(dst + (j * WAVES + wave) * 256), 4,
                                                   off, 0, 0, 0);
        }
      }
    } else if constexpr (W4) {
#pragma unroll
      for (int ii = 0; ii < NI; ++ii) {
        const int r = wn * WN + ii * 16 + l16;
        const int64_t gi = (int64_t)kb * 4 + g4;
        const uint32_t off = (r < nrows && gi < G32) ? (uint32_t)(r * G32 + gi) : kOOB;
        sw4_reg[buf][ii] = (int)__builtin_amdgcn_raw_buffer_load_b8(rsw4, off, 0, 0);
      }
    } else {
      const uint32_t off = swoff == kOOB ? kOOB : swoff + kb * SB;
      if (FMT == 0) sw_reg[buf] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsw, off, 0, 0));
      else sw_reg[buf] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b8(rsw, off, 0, 0));
    }
  };

  // fragment: 16 rows x 128 codes; lane (l16, g4) takes row l16 and the
  // 16-byte chunks g4 and g4 + 4 of the K block as its 32 MFMA bytes.  The
  // same permutation of K on both operands leaves every dot product the
  // same, and all four 32-element scale sub-blocks of a row carry the one
  // block scale.  With chunks {0,1,2,3} then {4,5,6,7} across the four
  // lane groups the fragment reads have no LDS bank conflicts; chunks
  // {0,2,4,6} conflict two ways.  Fragment rows start at multiples of 16,
  // so a row's swizzle ((row >> 1) & 7) is the lane's (l16 >> 1): two
  // per-lane chunk offsets serve every fragment.
  const int ch0 = (g4 ^ (l16 >> 1)) << 4;
  const int ch1 = ((g4 + 4) ^ (l16 >> 1)) << 4;
  const int chw = (g4 ^ ((l16 >> 2) & 3)) << 4;   // MXFP4 W rows: chunk g4
  // a W fragment: FP8 rows as X, MXFP4 rows one 16-byte chunk per lane
  auto wfrag = [&](const uint8_t* row) -> v8i {
    if constexpr (W4) return read_frag_w4(row, chw);
    else return read_frag(row, ch0, ch1);
  };

  v4f acc[NI][MI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // One K block: issue the next stage's DMA, read this stage's fragments
  // (they may interleave freely with the MFMAs), run the MFMAs.
  auto step = [&](auto buf_c, int kb_next) {
    constexpr int buf = decltype(buf_c)::value;
    const int kb_cur = kb_next - 1;
    const uint8_t* sx = lds + buf * STAGE + (wm * WM + l16) * kRowBytes;
    const uint8_t* swl = lds + buf * STAGE + XBYTES + (wn * WN + l16) * kWRow;
    // 256 x 256 tiles and grouped tiles: every wave issues the next stage's
    // X tile here and its W tile and scales after its first MFMA group, so
    // no wave waits behind its whole share of the stage's DMA before its
    // first MFMAs (same bits; 2-5% on the dense Llama and DeepSeek shapes,
    // 2-3% with MXFP4 weights, 6% on the MXFP4 MoE experts, 0-1% on the
    // FP8 ones; 2% slower on dense 128 x 256 MXFP4 and 64-row tiles, 3-4%
    // on dense 128 x 256 FP8 tiles at M = 128, which keep one issue point.
    // Half the waves issuing all of theirs after the first group: 1-4%;
    // after the second group, the stage lands late: fp32 scales 1.7x slower)
    constexpr bool LATE = !XQ && ((BM == 256 && BN == 256) || GROUPED);
    issue(kb_next, buf ^ 1, LATE ? 1 : 0);
    float sa[MI];
    float sw = W4 ? 0.0f : sw_reg[buf];
    if (FMT == 1) sw = __int_as_float(__float_as_int(sw) & 0xff);
    int sw4[W4 ? NI : 1];
    if constexpr (SW4) {
      // this lane's group byte (g4) of K block kb_cur for each of its subtile rows
      const int rel = kb_cur - kb_begin;
      const uint8_t* wsc4 = wbuf + ((rel / WCH) & 1) * WBUF + (rel % WCH) * 4 + g4;
#pragma unroll
      for (int ii = 0; ii < NI; ++ii) sw4[ii] = (int)read_byte(wsc4, (wn * WN + ii * 16 + l16) * 32);
    } else if constexpr (W4) {
#pragma unroll
      for (int ii = 0; ii < NI; ++ii) sw4[ii] = sw4_reg[buf][ii] & 0xff;
    }
    if constexpr (XQ) {
      // the scales this workgroup derived for the stage's rows
#pragma unroll
      for (int j = 0; j < MI; ++j) {
        sa[j] = read_scale(sxq + buf * BM, wm * WM + j * 16 + l16);
        if (FMT == 1) sa[j] = __int_as_float(__float_as_int(sa[j]) & 0xff);
      }
    } else if constexpr (SCL) {
      // this block's scales of the lane's token rows, from the chunk buffer
      const int rel = kb_cur - kb_begin;
      const uint8_t* sc = sbuf + ((rel / SCH) & 1) * SBUF + (rel % SCH) * SB;
#pragma unroll
      for (int j = 0; j < MI; ++j) {
        const int o = (wm * WM + j * 16 + l16) * SROW;
        sa[j] = FMT == 0 ? read_scale((const float*)sc, o / 4)
                         : __int_as_float((int)read_byte(sc, o));
      }
    } else {
#pragma unroll
      for (int j = 0; j < MI; ++j) {
        sa[j] = sa_reg[buf][j];
        if (FMT == 1) sa[j] = __int_as_float(__float_as_int(sa[j]) & 0xff);
      }
    }
    v8i bx[MI];
#pragma unroll
    for (int j = 0; j < MI; ++j) bx[j] = read_frag(sx + j * 16 * kRowBytes, ch0, ch1);
    // W fragments in groups of NG 16-row subtiles, read one group ahead:
    // group g + 1 is in flight while the MFMAs of group g run.  Scheduling
    // fences keep that order (and bound the live fragments).  The dense
    // 256 x 256 UE8M0 tile (no promotion FMAs) takes one subtile per group
    // and interleaves each MFMA with one fragment read (3.4% faster over the
    // DeepSeek-sized shapes, 8% at 4096 x 18432 x 7168; with fp32 scales the
    // two-subtile groups measured best).
    constexpr bool ONE = FMT == 1 && BM == 256 && !GROUPED && !W4 && !SWIGLU && !XQ;
    constexpr int NG = ONE ? 1 : 2;
    constexpr int NGR = NI / NG;
    v8i aw[2][NG];
#pragma unroll
    for (int ii = 0; ii < NG; ++ii) aw[0][ii] = wfrag(swl + ii * 16 * kWRow);
    static_for<NGR>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g + 1 < NGR) {
#pragma unroll
        for (int ii = 0; ii < NG; ++ii)
          aw[(g + 1) & 1][ii] = wfrag(swl + ((g + 1) * NG + ii) * 16 * kWRow);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ii = 0; ii < NG; ++ii)
#pragma unroll
        for (int j = 0; j < MI; ++j) {
          if constexpr (W4)
            acc[g * NG + ii][j] = mfma_step_w4<FMT>(acc[g * NG + ii][j], aw[g & 1][ii], bx[j], sa[j],
                                                    sw4[g * NG + ii]);
          else
            acc[g * NG + ii][j] = mfma_step<FMT>(acc[g * NG + ii][j], aw[g & 1][ii], bx[j], sa[j], sw);
        }
      if constexpr (ONE) {
#pragma unroll
        for (int i = 0; i < NG * MI; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (LATE && g == 0) {
        issue(kb_next, buf ^ 1, 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  };

  // XQ: encode the landed bf16 stage with the activation codec (the codes
  // and scales fp8_quant_act writes for these rows and K block) into the X
  // tile of buffer `buf` (row-swizzled 16-byte chunks, as the DMA lays them
  // out) and its scale row
  auto xquant = [&](int buf) {
    uint8_t* sxl = lds + buf * STAGE;
    float* sq = sxq + buf * BM;
#pragma unroll
    for (int j = 0; j < XQJ; ++j) {
      const int q = j * THREADS + (int)threadIdx.x;
      const int row = q >> 4, c16 = q & 15;
      const u32x4 v = xr[j];
      float f[8];
      f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
      f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
      uint2 codes;
      float sv;
      if constexpr (FMT == 0) {
        // static scheme (xs carries the calibrated scale): x / s is not
        // bounded by 448 and may overflow, so it divides directly too
        const float sc = xs ? *(const float*)xs : act_scale_f32(amax);
        if (xs || !(sc >= kMinNormal)) {
          // subnormal scale: direct division (see div_by_rcp)
          codes.x = act_encode4<0>(f[0], f[1], f[2], f[3], sc, 0);
          codes.y = act_encode4<0>(f[4], f[5], f[6], f[7], sc, 0);
        } else {
          const RcpDiv dv = rcp_div(sc);
          codes.x = act_encode4_rcp<0>(f[0], f[1], f[2], f[3], dv, 0);
          codes.y = act_encode4_rcp<0>(f[4], f[5], f[6], f[7], dv, 0);
        }
        sv = sc;
      } else {
        const int e = xs ? (int)*(const uint8_t*)xs - 127 : ue8m0_exp(amax);
        codes.x = act_encode4<1>(f[0], f[1], f[2], f[3], 0.0f, e);
        codes.y = act_encode4<1>(f[4], f[5], f[6], f[7], 0.0f, e);
        sv = __int_as_float(e + 127);
      }
      const int pc = (c16 >> 1) ^ ((row >> 1) & 7);
      *(uint2*)(sxl + row * kRowBytes + pc * 16 + (c16 & 1) * 8) = codes;
      if (c16 == 0) sq[row] = sv;
    }
  };

  // prologue: the first stage
  issue(kb_begin, 0);

  // Main loop, unrolled by two so every register / buffer index is static.
  // Each step issues the next stage unconditionally (a stage past the end of
  // K loads zeros: its offsets are out of range; past the end of a split it
  // loads the next split's first block, which is never used).
  for (int kb0 = kb_begin;; kb0 += 2) {
    bool last = false;
    static_for<2>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if (last) return;
      const int kb = kb0 + s;
      // stage kb landed (own loads), then everyone's loads landed and
      // everyone is done reading the buffer about to be refilled
      wait_vmcnt<0>();
      if constexpr (XQ) {
        xquant(s);
        asm volatile("" ::: "memory");
        wait_lgkmcnt0();
      }
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      step(std::integral_constant<int, s>{}, kb + 1);
      last = kb + 1 >= kb_end;
    });
    if (last) break;
  }
  // drain: no DMA may land in LDS after this workgroup has finished
  wait_vmcnt<0>();

  if constexpr (SWIGLU) {
    swiglu_epilogue<FMT, WAVES_M, WAVES_N, WM, WN>(acc, lds, tl, wm, wn, lane, I, c0, y, hq, hs);
    return;
  }

  // bf16 epilogue through LDS when the stage buffers hold the whole output
  // tile: waves write their tiles (bias added, rounded) row-major with 16-byte
  // chunks swizzled by row, then every thread stores whole 16-byte chunks, 32
  // lanes to a 512-byte row, so the output leaves in full lines
  constexpr int CPR = BN / 8;                 // 16-byte chunks per output row
  if constexpr (BM * BN * 2 <= STAGES * STAGE) {
    if (part == nullptr) {
      __syncthreads();                        // every fragment read of the last stage done
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int col = wn * WN + i * 16 + 4 * g4;
        const int64_t n = tl.n0 + col;
#pragma unroll
        for (int j = 0; j < MI; ++j) {
          const int row = wm * WM + j * 16 + l16;
          v4f v = acc[i][j];
          if (bias && n < N) {
            const uint2 b = *(const uint2*)(bias + n);
            v[0] += bf16_lo(b.x); v[1] += bf16_hi(b.x);
            v[2] += bf16_lo(b.y); v[3] += bf16_hi(b.y);
          }
          uint2 o;
          o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
          o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
          const int c = col >> 3;
          *(uint2*)(lds + row * (BN * 2) + ((c ^ (row & (CPR - 1))) << 4) + ((col >> 2) & 1) * 8) = o;
        }
      }
      __syncthreads();
      // non-temporal stores: the output is not read again by this launch, and
      // kept out of L2 it does not evict the operand panels the other tiles
      // of the XCD still read (0-1.8% on the Llama and DeepSeek shapes)
#pragma unroll
      for (int p = 0; p < BM * CPR / THREADS; ++p) {
        const int L = p * THREADS + (int)threadIdx.x;
        const int row = L / CPR, c = L % CPR;
        const int64_t n = tl.n0 + c * 8;
        if (row < mrows && n < N) {
          const uint4 v = *(const uint4*)(lds + row * (BN * 2) + ((c ^ (row & (CPR - 1))) << 4));
          __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w},
                                      (u32x4*)(y + (tl.m0 + row) * N + n));
        }
      }
      return;
    }
  }

  // epilogue: lane holds n = nwave + 16 i + 4 g4 + {0..3} for token m_j
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int64_t n = nwave + i * 16 + 4 * g4;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < MI; ++j) {
      const int64_t m = tl.m0 + wm * WM + j * 16 + l16;
      if (m >= tl.mlim) continue;
      if (part) {
        float* p = part + ((int64_t)tl.split * M + m) * N + n;
        *(float4*)p = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      } else {
        store_out4(y, N, m, n, acc[i][j], bias);
      }
    }
  }
#endif

}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int64_t MN, int64_t N,
                                                            const uint16_t* __restrict__ bias,
                                                            uint16_t* __restrict__ y) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= MN) return;
  float4 s = *(const float4*)(part + i4);
  for (int k = 1; k < splits; ++k) {
    const float4 t = *(const float4*)(part + (int64_t)k * MN + i4);
    s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
  }
  const int64_t m = i4 / N, n = i4 - m * N;
  store_out4(y, N, m, n, v4f{s.x, s.y, s.z, s.w}, bias);
}

// ------------------------------------------------------------------------
// Decode kernel (M <= 16): one workgroup owns 16 weight rows over the whole
// K range and its kDecodeWaves waves take the K blocks round-robin.  Each
// lane streams its 32 weight bytes per block straight from HBM with
// kDecodeDepth blocks of loads in flight, the quantized activation
// fragment (one token row per lane column) and both block scales are
// fetched together with those weights, and the waves' partial 16 x 16
// tiles are summed through LDS: one launch, no workspace.  FUSED: the 1x128
// activation quantization runs in the same launch -- each lane encodes its
// 32 activations of the block with the group amax gathered from the four
// lanes that share its row, to the codes fp8_quant_act writes (the fp32
// division by the scale done as a multiply by the correctly rounded
// reciprocal plus one exact correction).  Every workgroup quantizes all of
// X, so the re-quantization grows with N K: the fused form is used up to
// N K = 2^24 and K = 6144 only (measured against the separate quantization
// launch plus the unfused kernel, which wins from N K = 6144 x 4096 and at
// K = 7168 with 16 tokens).
// ------------------------------------------------------------------------
constexpr int kDecodeWaves = 16;
constexpr int kDecodeDepth = 2;

// W4: W holds MXFP4 codes (N, K/2) with E8M0 scales per 1 x 32 group
// (N, K/32): each lane streams 16 weight bytes and one scale byte per block
// and takes the X chunks g4 and g4 + 4 (the FP4 x FP8 lane pairing of the
// scaled MFMA).  The kernel is bound by the latency of each workgroup's one
// round of loads, not by bytes, so MXFP4 rows run at about the FP8 time.
// XB (plain FP8 weights, from 8 tokens): every load of a block goes out
// unconditionally through a buffer resource (out-of-range offsets read
// zeros) instead of behind a branch per load, and the activation loads are
// held ahead of the weight loads: with no branch between them the compiler
// knows how many loads are in flight at each use, so the fused encoding waits
// for its activations alone and runs under the weight loads (behind branches
// it waited for all of them first).
// B32: (32, 32) weight blocks with 1 x 32 act groups.  A lane's 32 weight
// and activation bytes of a block are exactly the 32-wide group g4, so the
// block runs as four MFMAs whose weight operand keeps only group g's lanes,
// each promoted by s_a[m, g] s_w[n/32, g] in fp32 (UE8M0 bytes decoded to
// their powers of two); the extra MFMAs are free in this HBM-bound kernel.
// the activation scales of at most 16 tokens, staged whole (SXL) when they fit
constexpr int kDecodeXsBytes = 16384;

template <int FMT, bool FUSED, bool W4 = false, bool B32 = false, bool SXL = false,
          bool SWL = false, bool XB = true>
__global__ __launch_bounds__(64 * kDecodeWaves) void gemm_decode_kernel(
    const uint8_t* __restrict__ xq, const void* __restrict__ xs,
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wq,
    const void* __restrict__ wsc, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int M, int64_t N, int64_t K, const void* __restrict__ xstat) {
  static_assert(!SXL || !FUSED, "staged activation scales: quantized X");
  __shared__ v4f red[kDecodeWaves][64];
  // SXL: the M x KB activation scales, read once (contiguous) instead of one
  // scale per token row per K block, which cost as many requests as the
  // X codes themselves
  __shared__ __attribute__((aligned(16))) uint8_t sxs[SXL ? kDecodeXsBytes : 16];
  // SWL (MXFP4 weights, K a multiple of 128): the workgroup's 16 rows of E8M0
  // group scales are one contiguous span of 16 K/32 bytes, copied once
  // instead of one byte per lane per K block (as many requests as the codes)
  // (B32: the tile's one row of (32, 32)-block scales, GS entries)
  static_assert(!SWL || W4 || B32, "staged weight scales: MXFP4 or (32, 32) blocks");
  __shared__ __attribute__((aligned(16))) uint8_t sws[SWL ? kDecodeXsBytes : 16];
  const int lane = threadIdx.x & 63;
  constexpr bool PLAIN = !W4 && !B32 && XB;
  const int wave = PLAIN ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t nrow = n0 + l16;
  const bool nvalid = nrow < N;
  const bool mvalid = l16 < M;             // this lane's token row (B column)
  const int KB = (int)((K + 127) / 128);
  const int64_t nblk = n0 >> 7;
  constexpr int SBX = FMT == 0 ? 4 : 1;
  const int64_t GS = (K + 31) / 32;        // B32: scale groups per row
  if constexpr (SXL) {
    // M x KB scales (M x GS with 1 x 32 groups), <= kDecodeXsBytes (launcher)
    const int nbytes = M * (int)(B32 ? GS : KB) * SBX;
    for (int i = threadIdx.x * 4; i < nbytes; i += 64 * kDecodeWaves * 4) {
      if (i + 4 <= nbytes) {
        *(uint32_t*)(sxs + i) = *(const uint32_t*)((const uint8_t*)xs + i);
      } else {
        for (int b = i; b < nbytes; ++b) sxs[b] = ((const uint8_t*)xs)[b];
      }
    }
    __syncthreads();
  }
  const int64_t KW = W4 ? K / 2 : K;       // W bytes per row
  const int64_t G32 = K / 32;
  const int64_t nb32 = n0 >> 5;            // B32: this tile's weight block row
  if constexpr (SWL && W4) {
    const int nwords = (int)(min((int64_t)16, N - n0) * G32 / 4);   // K % 128 == 0
    const uint32_t* src = (const uint32_t*)((const uint8_t*)wsc + n0 * G32);
    for (int i = threadIdx.x; i < nwords; i += 64 * kDecodeWaves) ((uint32_t*)sws)[i] = src[i];
    __syncthreads();
  } else if constexpr (SWL && B32) {
    const int nbytes = (int)GS * SBX;
    const uint8_t* src = (const uint8_t*)wsc + nb32 * GS * SBX;
    for (int i = threadIdx.x; i < nbytes; i += 64 * kDecodeWaves) sws[i] = src[i];
    __syncthreads();
  }
  const uint8_t* wrow = wq + nrow * KW;
  // PLAIN (FP8 weights in 128-blocks): every load of a block is issued
  // unconditionally through a buffer resource (out-of-range offsets read
  // zeros), so no load sits behind a branch and the compiler's count of the
  // loads in flight stays exact: the encoding of a block then waits for its
  // activations only, not for every weight load issued after them
  const int64_t wrows = min((int64_t)16, N - n0);
  const __amdgpu_buffer_rsrc_t rwb = make_rsrc(wq + n0 * KW, PLAIN ? wrows * KW : 0);
  const uint32_t wlo = (uint32_t)(l16 * KW);
  const __amdgpu_buffer_rsrc_t rxb = make_rsrc(FUSED ? (const void*)x : (const void*)xq,
                                               FUSED ? (int64_t)M * ldx * 2 : (int64_t)M * K);
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(xs, (int64_t)M * KB * SBX);
  // this lane's X elements of a block: two runs of 16 starting at kx0, kx1
  const int kx0 = W4 ? 16 * g4 : 32 * g4;
  const int kx1 = W4 ? 64 + 16 * g4 : 32 * g4 + 16;

  constexpr int DEPTH = kDecodeDepth;
  constexpr int XD = FUSED ? 1 : DEPTH;    // X fragments prefetched with W
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int kb0 = wave; kb0 < KB; kb0 += kDecodeWaves * DEPTH) {
    uint4 wa[DEPTH], wb[DEPTH];
    int sw4[DEPTH];
    float swb[DEPTH];
    uint4 xa[XD], xb[XD];
    float sx[XD];
    // FUSED: this lane's 32 bf16 activations of each block, issued before
    // the weights: loads complete in issue order, so encoding them then
    // waits for them alone, while the weight loads are still in flight
    uint4 xv[FUSED ? DEPTH : 1][4];
    if constexpr (FUSED) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int kb = kb0 + u * kDecodeWaves;
        const int64_t k0 = (int64_t)kb * 128 + kx0, k1 = (int64_t)kb * 128 + kx1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t k = (i < 2 ? k0 : k1) + 8 * (i & 1);
          if constexpr (PLAIN) {
            const uint32_t o = (kb < KB && mvalid && k < K) ? (uint32_t)(((int64_t)l16 * ldx + k) * 2) : kOOB;
            const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rxb, o, 0, 0);
            xv[u][i] = make_uint4(t.x, t.y, t.z, t.w);
          } else {
            xv[u][i] = make_uint4(0, 0, 0, 0);
            if (kb < KB && mvalid && k < K) xv[u][i] = *(const uint4*)(x + (int64_t)l16 * ldx + k);
          }
        }
      }
    }
    // keep the activation loads ahead of the weight loads in issue order
    if constexpr (FUSED && PLAIN) __builtin_amdgcn_sched_barrier(0);
    // B32: the four groups' scales (fp32), or this lane's group's bytes
    float sx4[B32 ? DEPTH : 1][4], sw32[B32 ? DEPTH : 1][4];
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int kb = kb0 + u * kDecodeWaves;
      wa[u] = make_uint4(0, 0, 0, 0);
      wb[u] = make_uint4(0, 0, 0, 0);
      sw4[u] = 127;
      // the weight block scale: with fp32 scales it multiplies this lane's
      // OUTPUT column (token l16), so every lane needs it, whatever its row
      swb[u] = (FMT == 0) ? 0.f : __int_as_float(127);
      // a uniform address (kb, nblk): a scalar load, clamped in range
      if (PLAIN) swb[u] = load_scale<FMT>(wsc, min(nblk * KB + kb, ((N + 127) / 128) * KB - 1));
      else if (!W4 && !B32 && kb < KB) swb[u] = load_scale<FMT>(wsc, nblk * KB + kb);
      if constexpr (B32) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t gi = (int64_t)kb * 4 + g;
          const bool ok = kb < KB && gi < GS;
          float w = 0.f, x = 0.f;
          if (ok) {
            if constexpr (SWL)
              w = FMT == 0 ? ((const float*)sws)[gi] : __int_as_float((int)sws[gi]);
            else
              w = load_scale<FMT>(wsc, nb32 * GS + gi);
          }
          if (ok && mvalid) {
            if constexpr (SXL)
              x = FMT == 0 ? ((const float*)sxs)[l16 * GS + gi] : __int_as_float((int)sxs[l16 * GS + gi]);
            else
              x = load_scale<FMT>(xs, (int64_t)l16 * GS + gi);
          }
          if (FMT == 1) {
            w = ok ? e8m0_f32(__float_as_uint(w)) : 0.f;
            x = (ok && mvalid) ? e8m0_f32(__float_as_uint(x)) : 0.f;
          }
          sw32[u][g] = w;
          sx4[u][g] = x;
        }
      }
      if (kb < KB && nvalid) {
        if constexpr (W4) {
          // this lane's 32 weights (group 4 kb + g4) and their scale byte
          const int64_t kw = (int64_t)kb * 64 + g4 * 16;
          if (kw < KW) {
            wa[u] = ld_stream16(wrow + kw);
            sw4[u] = SWL ? (int)sws[l16 * G32 + (int64_t)kb * 4 + g4]
                         : (int)((const uint8_t*)wsc)[nrow * G32 + (int64_t)kb * 4 + g4];
          }
        } else if constexpr (!PLAIN) {
          const int64_t k = (int64_t)kb * 128 + g4 * 32;
          if (k < K) wa[u] = ld_stream16(wrow + k);
          if (k + 16 < K) wb[u] = ld_stream16(wrow + k + 16);
        }
      }
      if constexpr (PLAIN) {
        const int64_t k = (int64_t)kb * 128 + g4 * 32;
        const bool kin = kb < KB;
        u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rwb, kin && k < K ? wlo + (uint32_t)k : kOOB, 0, 2);
        wa[u] = make_uint4(t.x, t.y, t.z, t.w);
        t = __builtin_amdgcn_raw_buffer_load_b128(rwb, kin && k + 16 < K ? wlo + (uint32_t)k + 16 : kOOB, 0, 2);
        wb[u] = make_uint4(t.x, t.y, t.z, t.w);
      }
      if constexpr (!FUSED) {
        // the quantized X fragment and its scale (L2-resident), issued with
        // the weight loads so their latencies overlap
        xa[u] = make_uint4(0, 0, 0, 0);
        xb[u] = make_uint4(0, 0, 0, 0);
        sx[u] = (FMT == 0) ? 0.f : __int_as_float(127);
        if constexpr (PLAIN) {
          const int64_t k0 = (int64_t)kb * 128 + kx0, k1 = (int64_t)kb * 128 + kx1;
          const bool ok = kb < KB && mvalid;
          const uint32_t xo = (uint32_t)(l16 * K);
          u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rxb, ok && k0 < K ? xo + (uint32_t)k0 : kOOB, 0, 0);
          xa[u] = make_uint4(t.x, t.y, t.z, t.w);
          t = __builtin_amdgcn_raw_buffer_load_b128(rxb, ok && k1 < K ? xo + (uint32_t)k1 : kOOB, 0, 0);
          xb[u] = make_uint4(t.x, t.y, t.z, t.w);
          if constexpr (SXL) {
            if (ok) sx[u] = FMT == 0 ? ((const float*)sxs)[l16 * KB + kb]
                                     : __int_as_float((int)sxs[l16 * KB + kb]);
          } else {
            const uint32_t so = ok ? (uint32_t)((l16 * KB + kb) * SBX) : kOOB;
            if constexpr (FMT == 0) {
              sx[u] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rxs, so, 0, 0));
            } else {
              const int b = (int)__builtin_amdgcn_raw_buffer_load_b8(rxs, so, 0, 0);
              sx[u] = __int_as_float(ok ? b : 127);
            }
          }
        } else if (kb < KB && mvalid) {
          const int64_t k0 = (int64_t)kb * 128 + kx0, k1 = (int64_t)kb * 128 + kx1;
          if (k0 < K) xa[u] = *(const uint4*)(xq + (int64_t)l16 * K + k0);
          if (k1 < K) xb[u] = *(const uint4*)(xq + (int64_t)l16 * K + k1);
          if constexpr (SXL) {
            sx[u] = FMT == 0 ? ((const float*)sxs)[l16 * KB + kb]
                             : __int_as_float((int)sxs[l16 * KB + kb]);
          } else if (!B32) {
            sx[u] = load_scale<FMT>(xs, (int64_t)l16 * KB + kb);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int kb = kb0 + u * kDecodeWaves;
      if (kb >= KB) break;
      v8i bx;
      float sa;
      if constexpr (FUSED) {
        const uint4* v = xv[u];
        float f[32];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[8 * i + 0] = bf16_lo(v[i].x); f[8 * i + 1] = bf16_hi(v[i].x);
          f[8 * i + 2] = bf16_lo(v[i].y); f[8 * i + 3] = bf16_hi(v[i].y);
          f[8 * i + 4] = bf16_lo(v[i].z); f[8 * i + 5] = bf16_hi(v[i].z);
          f[8 * i + 6] = bf16_lo(v[i].w); f[8 * i + 7] = bf16_hi(v[i].w);
        }
        float s = 0.0f;
        int e = 0;
        if (xstat) {
          // static scheme: the one calibrated per-tensor scale
          if (FMT == 0) s = *(const float*)xstat;
          else e = (int)*(const uint8_t*)xstat - 127;
        } else {
          float amax = 0.0f;
#pragma unroll
          for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(f[i]));
          amax = fmaxf(amax, __shfl_xor(amax, 16));
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          if (FMT == 0) s = act_scale_f32(amax);
          else e = ue8m0_exp(amax);
        }
        if (FMT == 0 && (xstat || !(s >= kMinNormal))) {
          // a subnormal scale (1 / s can overflow and the residual of the
          // reciprocal form can round) or a static one (x / s is not bounded
          // by 448 and may overflow): divide directly
#pragma unroll
          for (int i = 0; i < 8; ++i)
            bx[i] = (int)act_encode4<FMT>(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3], s, e);
        } else {
          const RcpDiv dv = rcp_div(FMT == 0 ? s : 1.0f);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            bx[i] = (int)act_encode4_rcp<FMT>(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3],
                                              dv, e);
        }
        sa = FMT == 0 ? s : __int_as_float(e + 127);
      } else {
        sa = sx[u < XD ? u : 0];
        bx = join(xa[u < XD ? u : 0], xb[u < XD ? u : 0]);
      }
      if constexpr (W4) {
        acc = mfma_step_w4<FMT>(acc, join(wa[u], make_uint4(0, 0, 0, 0)), bx, sa, sw4[u]);
      } else if constexpr (B32) {
        const v8i a = join(wa[u], wb[u]);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          v8i ag;
#pragma unroll
          for (int i = 0; i < 8; ++i) ag[i] = g4 == g ? a[i] : 0;
          acc = mfma_step<0>(acc, ag, bx, sx4[u][g], sw32[u][g]);   // fp32 promotion
        }
      } else {
        acc = mfma_step<FMT>(acc, join(wa[u], wb[u]), bx, sa, swb[u]);
      }
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  v4f sum = red[0][lane];
#pragma unroll
  for (int w = 1; w < kDecodeWaves; ++w) sum += red[w][lane];
  // lane holds n = n0 + 4 g4 + {0..3} for token m = l16
  const int64_t n = n0 + 4 * g4;
  if (mvalid && n < N) store_out4(y, N, l16, n, sum, bias);
}

// ------------------------------------------------------------------------
// Persistent decode kernel (4 <= M <= 16, FP8 weights in 128 x 128 blocks,
// X quantized beforehand).  Same 16-row tiles, lane layout and per-block
// arithmetic as gemm_decode_kernel, but the grid is the workgroups that fit
// on the device at once and each walks the tiles t = blockIdx.x,
// + gridDim.x, ...: the whole M x K of X codes (and the activation scales)
// is copied to LDS once per workgroup and serves all its tiles.  In
// gemm_decode_kernel each lane loads its X fragment per block from L2, a
// second stream as large as the weights' at M = 16 that held that kernel to
// about 3.3 TB/s on weight-bound shapes (4.5 TB/s at M = 1).  X rows are
// padded by 16 bytes so that the 16 token rows of a fragment read fall in
// distinct LDS banks.
// The K blocks of a tile are dealt to the 16 waves (wave w takes w + 16 j),
// DEPTH per chunk; every chunk's loads are issued before the previous chunk
// is multiplied, across tile boundaries, so a chunk stays in flight through
// the MFMAs, the LDS reduction of the waves' partial tiles and the store.
// Chunk slots past a tile's blocks load nothing (out-of-range buffer offsets
// read zeros) and are multiplied like the others: every chunk issues the
// same loads and consumes all of them.
// ------------------------------------------------------------------------
constexpr int kPersXsBytes = 4096;   // activation scales (M x KB)
constexpr int kPersXlBytes = 163840 - 2 * kDecodeWaves * 64 * 16 - kPersXsBytes;   // X codes

template <int FMT, int DEPTH, bool FUSED = false>
__global__ __launch_bounds__(64 * kDecodeWaves) void gemm_decode_pers_kernel(
    const uint8_t* __restrict__ xq, const void* __restrict__ xs, const uint8_t* __restrict__ wq,
    const void* __restrict__ wsc, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int M, int64_t N, int64_t K, int ntiles, const uint16_t* __restrict__ x, int64_t ldx,
    const void* __restrict__ xstat) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ v4f red[2][kDecodeWaves][64];
  __shared__ __attribute__((aligned(16))) uint8_t sxs[kPersXsBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sxl[kPersXlBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const bool mvalid = l16 < M;
  const int KB = (int)((K + 127) / 128);
  const int64_t NB = (N + 127) / 128;
  constexpr int SB = FMT == 0 ? 4 : 1;
  const int64_t KP = K + 16;                                // X row pitch in LDS
  const int nbw = (KB + kDecodeWaves - 1) / kDecodeWaves;   // blocks per wave and tile
  const int C = (nbw + DEPTH - 1) / DEPTH;                  // chunks per tile

  // two chunks' registers (index S = 0, 1, always a constant): the lane's
  // 32 W bytes of a block (K [32 g4, 32 g4 + 32), the K assignment of
  // gemm_decode_kernel, so both kernels form the same sums) and the wave's
  // weight-block scale per slot
  uint4 wa[2][DEPTH], wb[2][DEPTH];
  float sw[2][DEPTH];
  auto issue = [&](auto sc, int t, int c) __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value;
    const bool tin = t < ntiles;
    const int64_t n0 = (int64_t)t * 16;
    const int64_t rows = tin ? min((int64_t)16, N - n0) : 0;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(wq + (tin ? n0 * K : 0), rows * K);
    const int64_t nblk = n0 >> 7;
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int kb = wave + kDecodeWaves * (c * DEPTH + u);
      const int64_t k = (int64_t)kb * 128 + g4 * 32;
      const bool kin = kb < KB;
      const uint32_t ow = (uint32_t)(l16 * K + k);
      u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, kin && k < K ? ow : kOOB, 0, 2);   // nt
      wa[S][u] = make_uint4(v.x, v.y, v.z, v.w);
      v = __builtin_amdgcn_raw_buffer_load_b128(rw, kin && k + 16 < K ? ow + 16 : kOOB, 0, 2);
      wb[S][u] = make_uint4(v.x, v.y, v.z, v.w);
      // the wave's weight-block scale: one uniform address, a scalar load
      // (clamped in range; slots past the blocks multiply zeros)
      sw[S][u] = load_scale<FMT>(wsc, min(nblk * KB + kb, NB * KB - 1));
    }
  };

  int t0 = blockIdx.x, c0 = 0;       // the launcher sizes the grid <= ntiles

  // FUSED: every lane's bf16 loads of all its groups (at most XB batches of
  // XU: M K <= 40960 is at most 336 groups) go out before the first weight
  // chunk, unconditionally through a buffer resource over the M rows of ldx
  // values (out-of-range offsets read zeros; the launcher keeps that span in
  // the 32-bit range): with no branch between the loads the compiler counts
  // them exactly, so encoding a batch waits for its own loads alone (loads
  // complete in issue order), not for the weight chunk behind them
  constexpr int QW = 4 * kDecodeWaves;     // quarter-waves per workgroup
  constexpr int XU = 4;                    // groups (loads) per lane and batch
  constexpr int XB = 2;                    // batches
  uint4 xv[FUSED ? XB * XU : 1];
  if constexpr (FUSED) {
    const __amdgpu_buffer_rsrc_t rxv = make_rsrc(x, (int64_t)M * ldx * 2);
    const int ql = threadIdx.x & 15;
#pragma unroll
    for (int b = 0; b < XB * XU; ++b) {
      const int gi = (int)(threadIdx.x >> 4) + b * QW;
      const int m = gi / KB, g = gi - m * KB;
      const int64_t k0 = (int64_t)g * 128 + ql * 8;
      const uint32_t off =
          (gi < M * KB && k0 < K) ? (uint32_t)(((int64_t)m * ldx + k0) * 2) : kOOB;
      const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rxv, off, 0, 0);
      xv[b] = make_uint4(t.x, t.y, t.z, t.w);
    }
    __builtin_amdgcn_sched_barrier(0);     // ahead of the weight chunk
  }
  issue(std::integral_constant<int, 0>{}, t0, c0);   // in flight during the copy below

  // activation scales (M x KB) and codes (M x K), once per workgroup
  if constexpr (FUSED) {
    // FUSED: quantized here from the bf16 rows x (row stride ldx) with the
    // activation codec, to the codes and scales fp8_quant_act writes: one
    // 1 x 128 group per quarter-wave, 8 values per lane, the group amax
    // gathered over the quarter-wave's 16 lanes; xstat: the static scheme's
    // calibrated scale.  (Every workgroup repeats this M x K quantization, so
    // the launcher keeps it to small M: at 16 x 4096 the repeated encoding
    // costs more vector-ALU time than the quantization launch it saves.)
    // Each lane has XU groups' loads in flight before encoding any of them.
    const int ql = threadIdx.x & 15;
    const int ngroups = M * KB;
#pragma unroll
    for (int bt = 0; bt < XB; ++bt) {
      const int gi0 = (int)(threadIdx.x >> 4) + bt * XU * QW;
      const uint4* v = xv + bt * XU;
#pragma unroll
      for (int u = 0; u < XU; ++u) {
        const int gi = gi0 + u * QW;
        if (gi >= ngroups) break;            // uniform per quarter-wave
        const int m = gi / KB, g = gi - m * KB;
        const int64_t k0 = (int64_t)g * 128 + ql * 8;
        const float f[8] = {bf16_lo(v[u].x), bf16_hi(v[u].x), bf16_lo(v[u].y), bf16_hi(v[u].y),
                            bf16_lo(v[u].z), bf16_hi(v[u].z), bf16_lo(v[u].w), bf16_hi(v[u].w)};
        float sc = 0.0f;
        int e = 0;
        if (xstat) {
          if (FMT == 0) sc = *(const float*)xstat;
          else e = (int)*(const uint8_t*)xstat - 127;
        } else {
          float amax = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
          if (FMT == 0) sc = act_scale_f32(amax);
          else e = ue8m0_exp(amax);
        }
        uint2 codes;
        if (FMT == 0 && (xstat || !(sc >= kMinNormal))) {
          // a subnormal or static scale: divide directly (as the other fused paths)
          codes.x = act_encode4<FMT>(f[0], f[1], f[2], f[3], sc, e);
          codes.y = act_encode4<FMT>(f[4], f[5], f[6], f[7], sc, e);
        } else {
          const RcpDiv dv = rcp_div(FMT == 0 ? sc : 1.0f);
          codes.x = act_encode4_rcp<FMT>(f[0], f[1], f[2], f[3], dv, e);
          codes.y = act_encode4_rcp<FMT>(f[4], f[5], f[6], f[7], dv, e);
        }
        if (k0 < K) *(uint2*)(sxl + m * KP + k0) = codes;
        if (ql == 0) {
          if (FMT == 0) ((float*)sxs)[gi] = sc;
          else sxs[gi] = (uint8_t)(e + 127);
        }
      }
    }
  } else {
    const int nbytes = M * KB * SB;  // launcher: <= kPersXsBytes
    for (int i = threadIdx.x * 4; i < nbytes; i += 64 * kDecodeWaves * 4) {
      if (i + 4 <= nbytes) {
        *(uint32_t*)(sxs + i) = *(const uint32_t*)((const uint8_t*)xs + i);
      } else {
        for (int b = i; b < nbytes; ++b) sxs[b] = ((const uint8_t*)xs)[b];
      }
    }
    const int k16 = (int)(K / 16);
    const int nch = M * k16;         // launcher: M * KP <= kPersXlBytes
    for (int i = threadIdx.x; i < nch; i += 64 * kDecodeWaves) {
      const int m = i / k16, c = i - m * k16;
      *(uint4*)(sxl + m * KP + c * 16) = *(const uint4*)(xq + (int64_t)m * K + c * 16);
    }
  }
  __syncthreads();

  auto compute = [&](auto sc, int c, v4f& acc) __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value;
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int kb = wave + kDecodeWaves * (c * DEPTH + u);
      const int64_t k = (int64_t)kb * 128 + g4 * 32;
      uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
      const uint8_t* p = sxl + l16 * KP + k;
      if (mvalid && k < K) a = *(const uint4*)p;
      if (mvalid && k + 16 < K) b = *(const uint4*)(p + 16);
      float sa = FMT == 0 ? 0.0f : __int_as_float(127);
      if (mvalid && kb < KB)
        sa = FMT == 0 ? ((const float*)sxs)[l16 * KB + kb] : __int_as_float((int)sxs[l16 * KB + kb]);
      acc = mfma_step<FMT>(acc, join(wa[S][u], wb[S][u]), join(a, b), sa, sw[S][u]);
    }
  };
  // the waves' partial tiles summed through LDS (two buffers: a wave may
  // write the next tile's partial while wave 0 still reads this one)
  int par = 0;
  auto finish = [&](int t, v4f& acc) __attribute__((always_inline)) {
    red[par][wave][lane] = acc;
    acc = v4f{0.f, 0.f, 0.f, 0.f};
    wait_lgkmcnt0();                 // this wave's LDS write is done
    __builtin_amdgcn_s_barrier();    // no wait for the chunk in flight
    asm volatile("" ::: "memory");
    if (wave == 0) {
      v4f sum = red[par][0][lane];
#pragma unroll
      for (int w = 1; w < kDecodeWaves; ++w) sum += red[par][w][lane];
      const int64_t n = (int64_t)t * 16 + 4 * g4;
      if (mvalid && n < N) store_out4(y, N, l16, n, sum, bias);
    }
    par ^= 1;
  };

  // Chunk q of this workgroup: tile blockIdx.x + (q / C) gridDim.x, chunk
  // q % C of it.  The loop runs an even number of chunks (one all-zero chunk
  // past the end when needed) and tests only at its bottom, so the set
  // issued last in an iteration is always multiplied in the next: no path
  // back to the loop head carries unconsumed loads, which would make the
  // compiler wait for them before reusing their registers.
  const int nT = (ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int Q = nT * C;
  const int QP = (Q + 1) & ~1;
  auto advance = [&](int& t, int& c) __attribute__((always_inline)) {
    if (++c == C) { c = 0; t += gridDim.x; }
  };
  int t1 = t0, c1 = c0;              // chunk q + 1
  advance(t1, c1);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < QP; q += 2) {
    issue(std::integral_constant<int, 1>{}, t1, c1);   // past the last tile: no loads
    compute(std::integral_constant<int, 0>{}, c0, acc);
    if (q < Q && c0 == C - 1) finish(t0, acc);
    int t2 = t1, c2 = c1;
    advance(t2, c2);
    issue(std::integral_constant<int, 0>{}, t2, c2);
    compute(std::integral_constant<int, 1>{}, c1, acc);
    if (q + 1 < Q && c1 == C - 1) finish(t1, acc);
    t0 = t2;
    c0 = c2;
    t1 = t2;
    c1 = c2;
    advance(t1, c1);
  }
#endif
}

// ------------------------------------------------------------------------
// (32, 32) weight blocks with 1 x 32 activation groups (the fine-grained FP8
// guide, section 九, names weight_block_size=(32, 32) among the non-default
// blocks its tests cover).  A 128-wide K block then holds four
// scale groups and, with fp32 scales, each group's partial product needs a
// promotion of its own, so a K block runs as four 16x16x32 FP8 MFMAs per
// output tile: acc += (s_a[m, g] s_w[n / 32, g]) P_g.  (The 16x16x128
// scaled form applies one power of two per row and 32-wide K group and
// cannot carry fp32 scales.)  UE8M0 scales are exactly such powers of two:
// they run one scaled 16x16x128 MFMA per tile and K block, each group's
// pair of scale bytes passed as its operands (1.8-2.9x over the fp32 form
// on the same shapes).  Tile 128 (m) x 128 (n), four waves of 64 x 64, two LDS
// stages laid out as in the large-M kernel: the 8-byte fragment a lane
// takes for group g is half (u & 1) of logical chunk u >> 1, u = 4 g + g4,
// and the chunk swizzle keeps those reads free of bank conflicts.
// ------------------------------------------------------------------------
//
// GROUPED: the MoE expert GEMM over contiguous row segments with (32, 32)
// expert weight blocks, on the same tile table as the large-M kernel (one
// expert class, 128-row M tiles).
template <int FMT, bool SA, bool GROUPED = false>
__global__ __launch_bounds__(256, 2) void gemm_b32_kernel(
    const uint8_t* __restrict__ xq, const void* __restrict__ xs, const uint8_t* __restrict__ wq,
    const void* __restrict__ wsc, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int64_t M, int64_t N, int64_t K, const int32_t* __restrict__ seg, int E) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = 128, BN = 128, WAVES = 4;
  constexpr int MI = 4, NI = 4;                      // 64 x 64 per wave
  constexpr int XBYTES = BM * kRowBytes;
  constexpr int STAGE = (BM + BN) * kRowBytes;
  constexpr int SB = FMT == 0 ? 4 : 1;
  constexpr int J = BM * 8 / (64 * WAVES);           // DMA loads per lane per operand
  // Activation scales are staged through LDS in chunks of 32 bytes per row
  // (SCH K blocks: 2 of fp32, 8 of UE8M0 scales), one request per row and
  // chunk instead of one per row and group.  UE8M0 rows (K/32 bytes) are
  // dword-aligned only when K is a multiple of 128; the launcher picks the
  // per-group loads (SA false) otherwise.  fp32 always stages.
  constexpr bool SCL = FMT == 0 || SA;
  constexpr int SCH = 32 / (4 * SB);                 // K blocks per chunk
  constexpr int SBUF = BM * 32;                      // bytes per chunk buffer
  constexpr int SJ = BM * 8 / (64 * WAVES);          // chunk DMA loads per lane
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE + (SCL ? 2 * SBUF : 0)];
  uint8_t* const sbuf = lds + 2 * STAGE;
  static_assert(!GROUPED || 2 * STAGE >= 1025 * 4, "tile table fits the stage buffers");
  Tile tl;
  // the grouped tile table lives in the stage buffers until the tile is known
  if (GROUPED) tl = grouped_tile<BM, BN, 64 * WAVES>(seg, E, N, (int*)lds, 0);
  else tl = dense_tile<BM, BN>(M, N, 1);
  if (!tl.valid) return;
  if (GROUPED) __syncthreads();            // every lookup done before the first DMA
  const int KB = (int)((K + 127) / 128);
  const int GS = (int)((K + 31) / 32);               // scale groups per row
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int64_t mrows = min((int64_t)BM, (GROUPED ? tl.mlim : M) - tl.m0);
  const int64_t nrows = min((int64_t)BN, N - tl.n0);
  const int64_t NBS = (N + 31) / 32;
  // this tile's expert: weights (E, N, K), scales (E, NBS, GS)
  const uint8_t* wbase = wq + (int64_t)tl.expert * N * K;
  const uint8_t* wsb = (const uint8_t*)wsc + (int64_t)tl.expert * NBS * GS * SB;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xq + tl.m0 * K, mrows * K);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wbase + tl.n0 * K, nrows * K);
  const __amdgpu_buffer_rsrc_t rsa =
      make_rsrc((const uint8_t*)xs + tl.m0 * GS * SB, mrows * GS * SB);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(wsb, NBS * GS * SB);
  auto dma_src = [&](int q, int64_t rows, uint32_t kbyte) -> uint32_t {
    const int row = q >> 3, c = (q & 7) ^ ((row >> 1) & 7);
    const uint32_t kc = kbyte + c * 16;
    return (row < rows && kc < (uint32_t)K) ? (uint32_t)(row * K) + kc : kOOB;
  };
  uint32_t saoff[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int r = wm * 64 + i * 16 + l16;
    saoff[i] = r < mrows ? (uint32_t)(r * GS * SB) : kOOB;
  }
  const int64_t nb0 = (tl.n0 + wn * 64) >> 5;        // the wave's two weight blocks
  float sa_reg[SCL ? 1 : 2][MI][4];
  float sw_reg[2][2][4];
  // UE8M0: the raw scale bytes of this lane's group 4 kb + g4 (see step)
  int sa_raw[FMT == 1 && !SCL ? 2 : 1][MI];
  int sw_raw[FMT == 1 ? 2 : 1][2];

  auto issue = [&](int kb, int buf) {
    uint8_t* sx = lds + buf * STAGE;
    uint8_t* sw = sx + XBYTES;
    const uint32_t kbyte = (uint32_t)kb * 128;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int q = (j * WAVES + wave) * 64 + lane;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, BSFP8_LDS(sx + (j * WAVES + wave) * 1024), 16,
                                               dma_src(q, mrows, kbyte), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, BSFP8_LDS(sw + (j * WAVES + wave) * 1024), 16,
                                               dma_src(q, nrows, kbyte), 0, 0, 0);
    }
    if constexpr (SCL) {
      // at a chunk's first K block: 32 bytes of every row (lane q: row q / 8,
      // dword q % 8); bytes past the row's last group are never used
      if (kb % SCH == 0) {
        uint8_t* dst = sbuf + ((kb / SCH) & 1) * SBUF;
#pragma unroll
        for (int j = 0; j < SJ; ++j) {
          const int q = (j * WAVES + wave) * 64 + lane;
          const int row = q >> 3;
          const uint32_t off = row < mrows ? (uint32_t)(row * GS * SB + kb * 4 * SB + (q & 7) * 4) : kOOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, BSFP8_LDS(dst + (j * WAVES + wave) * 256), 4,
                                                   off, 0, 0, 0);
        }
      }
    }
    if constexpr (FMT == 1) {
      const int gi = kb * 4 + g4;
      if constexpr (!SCL) {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const uint32_t off = (saoff[i] == kOOB || gi >= GS) ? kOOB : saoff[i] + gi;
          sa_raw[buf][i] = (int)__builtin_amdgcn_raw_buffer_load_b8(rsa, off, 0, 0);
        }
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int64_t nbs = nb0 + b;
        const uint32_t off = (nbs < NBS && gi < GS) ? (uint32_t)(nbs * GS + gi) : kOOB;
        sw_raw[buf][b] = (int)__builtin_amdgcn_raw_buffer_load_b8(rsw, off, 0, 0);
      }
    } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int gi = kb * 4 + g;
      if constexpr (!SCL) {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const uint32_t off = (saoff[i] == kOOB || gi >= GS) ? kOOB : saoff[i] + gi * SB;
          sa_reg[buf][i][g] = FMT == 0
              ? __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsa, off, 0, 0))
              : e8m0_f32(__builtin_amdgcn_raw_buffer_load_b8(rsa, off, 0, 0));
        }
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int64_t nbs = nb0 + b;
        const uint32_t off = (nbs < NBS && gi < GS) ? (uint32_t)((nbs * GS + gi) * SB) : kOOB;
        sw_reg[buf][b][g] = FMT == 0
            ? __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsw, off, 0, 0))
            : e8m0_f32(__builtin_amdgcn_raw_buffer_load_b8(rsw, off, 0, 0));
      }
    }
    }
  };

  v4f acc[NI][MI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto step = [&](auto buf_c, int kb_next) {
    constexpr int buf = decltype(buf_c)::value;
    const uint8_t* sx = lds + buf * STAGE + (wm * 64 + l16) * kRowBytes;
    const uint8_t* swl = lds + buf * STAGE + XBYTES + (wn * 64 + l16) * kRowBytes;
    issue(kb_next, buf ^ 1);
    if constexpr (FMT == 1) {
      // UE8M0: one scaled 16x16x128 MFMA per tile and K block.  Its per-lane
      // scale operands follow the operand's K order, not the lane's own
      // bytes: lane (l16, g4) holds K [16 g4, 16 g4 + 16) and
      // [64 + 16 g4, 80 + 16 g4) of row l16 (the fragment layout of the
      // 128-block kernel), while its scale byte serves row l16's K group
      // [32 g4, 32 g4 + 32) -- two other lanes' bytes (checked on the GPU,
      // every lane and byte of both operands).  So lane g4 passes group
      // 4 kb + g4: the row's activation scale, the subtile's weight-block
      // scale.  Groups past K take 2^0 (their codes are zeros).
      const int kb = kb_next - 1;
      const bool gin = kb * 4 + g4 < GS;
      int sxb[MI], swb[2];
#pragma unroll
      for (int j = 0; j < MI; ++j) {
        if constexpr (SCL) {
          const uint8_t* sc = sbuf + ((kb / SCH) & 1) * SBUF + (kb % SCH) * 4;
          sxb[j] = gin ? (int)read_byte(sc, (wm * 64 + j * 16 + l16) * 32 + g4) : 127;
        } else {
          sxb[j] = gin ? sa_raw[buf][j] & 0xff : 127;
        }
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) swb[b] = gin ? sw_raw[buf][b] & 0xff : 127;
      const int ch0 = (g4 ^ (l16 >> 1)) << 4;
      const int ch1 = ((g4 + 4) ^ (l16 >> 1)) << 4;
      v8i bx[MI];
#pragma unroll
      for (int j = 0; j < MI; ++j) bx[j] = read_frag(sx + j * 16 * kRowBytes, ch0, ch1);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const v8i aw = read_frag(swl + i * 16 * kRowBytes, ch0, ch1);
#pragma unroll
        for (int j = 0; j < MI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw, bx[j], acc[i][j], 0, 0, 0,
                                                                        swb[i >> 1], 0, sxb[j]);
      }
      return;
    }
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // this block's token scales (4 groups per row) from the chunk buffer;
    // groups past K take 0 so no other row's scale meets a zero product
    float sa[MI][4];
    if constexpr (SCL) {
      const int kb = kb_next - 1;
      const uint8_t* sc = sbuf + ((kb / SCH) & 1) * SBUF + (kb % SCH) * 4 * SB;
#pragma unroll
      for (int j = 0; j < MI; ++j) {
        const int o = (wm * 64 + j * 16 + l16) * 32;
        if constexpr (FMT == 0) {
          const float4 v = read_scale4(sc, o);
          sa[j][0] = v.x; sa[j][1] = v.y; sa[j][2] = v.z; sa[j][3] = v.w;
        } else {
          const uint32_t v = read_u32(sc, o);
#pragma unroll
          for (int g = 0; g < 4; ++g) sa[j][g] = e8m0_f32((v >> (8 * g)) & 0xff);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (kb * 4 + g >= GS) sa[j][g] = 0.0f;
      }
    } else {
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) sa[j][g] = sa_reg[buf][j][g];
    }
    // fragments of group g: rows start at multiples of 16, so the row
    // swizzle is the lane's (l16 >> 1)
    long bx[2][MI], aw[2][NI];
    auto rd = [&](int g, int s) {
      const int u = 4 * g + g4;
      const int off = (((u >> 1) ^ (l16 >> 1)) << 4) + ((u & 1) << 3);
#pragma unroll
      for (int j = 0; j < MI; ++j) bx[s][j] = read_u64(sx + j * 16 * kRowBytes, off);
#pragma unroll
      for (int i = 0; i < NI; ++i) aw[s][i] = read_u64(swl + i * 16 * kRowBytes, off);
    };
    rd(0, 0);
    static_for<4>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g + 1 < 4) rd(g + 1, (g + 1) & 1);
      float sc[2][MI];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < MI; ++j) sc[b][j] = sa[j][g] * sw_reg[buf][b][g];
      // the group's 16 products first, then their promotions: long runs of
      // independent MFMAs and of FMAs, which the two waves of a SIMD overlap
      // (with the next group's fragments read ahead: same bits, 1.15-1.3x
      // over one product promoted after each MFMA)
      v4f t[NI][MI];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < MI; ++j)
          t[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(aw[g & 1][i], bx[g & 1][j], zero, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < MI; ++j) {
          const float s = sc[i >> 1][j];
          acc[i][j][0] = fmaf(t[i][j][0], s, acc[i][j][0]);
          acc[i][j][1] = fmaf(t[i][j][1], s, acc[i][j][1]);
          acc[i][j][2] = fmaf(t[i][j][2], s, acc[i][j][2]);
          acc[i][j][3] = fmaf(t[i][j][3], s, acc[i][j][3]);
        }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  issue(0, 0);
  for (int kb0 = 0;; kb0 += 2) {
    bool last = false;
    static_for<2>([&](auto sc) {
      constexpr int st = decltype(sc)::value;
      if (last) return;
      const int kb = kb0 + st;
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      step(std::integral_constant<int, st>{}, kb + 1);
      last = kb + 1 >= KB;
    });
    if (last) break;
  }
  wait_vmcnt<0>();

  // bf16 epilogue through the first stage buffer: lane holds n = 16 i + 4 g4
  // + {0..3} of its wave's columns for token m_j; the tile is written row-
  // major with 16-byte chunks swizzled by row, then stored whole chunks at a
  // time, 16 lanes to a 256-byte row
  constexpr int CPR = BN / 8;
  __syncthreads();                           // every fragment read of the last stage done
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int col = wn * 64 + i * 16 + 4 * g4;
    const int64_t n = tl.n0 + col;
#pragma unroll
    for (int j = 0; j < MI; ++j) {
      const int row = wm * 64 + j * 16 + l16;
      v4f v = acc[i][j];
      if (bias && n < N) {
        const uint2 b = *(const uint2*)(bias + n);
        v[0] += bf16_lo(b.x); v[1] += bf16_hi(b.x);
        v[2] += bf16_lo(b.y); v[3] += bf16_hi(b.y);
      }
      uint2 o;
      o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
      o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
      const int c = col >> 3;
      *(uint2*)(lds + row * (BN * 2) + ((c ^ (row & (CPR - 1))) << 4) + ((col >> 2) & 1) * 8) = o;
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < BM * CPR / (64 * WAVES); ++p) {
    const int L = p * 64 * WAVES + (int)threadIdx.x;
    const int row = L / CPR, c = L % CPR;
    const int64_t m = tl.m0 + row, n = tl.n0 + c * 8;
    if (row < mrows && n < N)
      *(uint4*)(y + m * N + n) = *(const uint4*)(lds + row * (BN * 2) + ((c ^ (row & (CPR - 1))) << 4));
  }
#endif
}

#define BSFP8_B32(FMT, SA, G)                                                                  \
  template __global__ void gemm_b32_kernel<FMT, SA, G>(                                        \
      const uint8_t* __restrict__, const void* __restrict__, const uint8_t* __restrict__,      \
      const void* __restrict__, const uint16_t* __restrict__, uint16_t* __restrict__, int64_t, \
      int64_t, int64_t, const int32_t* __restrict__, int);
BSFP8_B32(0, false, false)
BSFP8_B32(1, false, false)
BSFP8_B32(1, true, false)
BSFP8_B32(0, false, true)
BSFP8_B32(1, false, true)
BSFP8_B32(1, true, true)
#undef BSFP8_B32

// Explicit instantiations of every tile configuration the dispatcher below
// can launch (the host pass does not always emit launch stubs for kernel
// templates that are only instantiated implicitly).
#define BSFP8_INST(FMT, WMN, WNN, WM, WN, G, W4, SW, SA)                                      \
  BSFP8_INST2(FMT, WMN, WNN, WM, WN, G, W4, SW, SA, false)
#define BSFP8_INST2(FMT, WMN, WNN, WM, WN, G, W4, SW, SA, SW4)                                \
  BSFP8_INST3(FMT, WMN, WNN, WM, WN, G, W4, SW, SA, SW4, false)
#define BSFP8_INST3(FMT, WMN, WNN, WM, WN, G, W4, SW, SA, SW4, XQ)                            \
  template __global__ void gemm_lds_kernel<FMT, WMN, WNN, WM, WN, G, W4, SW, SA, SW4, XQ>(   \
      const uint8_t* __restrict__, const void* __restrict__, const uint8_t* __restrict__,     \
      const void* __restrict__, const uint16_t* __restrict__, uint16_t* __restrict__, int64_t, \
      int64_t, int64_t, const int32_t* __restrict__, int, int, float* __restrict__, int,      \
      uint8_t* __restrict__, void* __restrict__, const uint16_t* __restrict__, int64_t);
#define BSFP8_INST_ALL(FMT)                                 \
  BSFP8_INST(FMT, 4, 2, 64, 128, false, false, false, false) \
  BSFP8_INST(FMT, 2, 4, 64, 64, false, false, false, false)  \
  BSFP8_INST(FMT, 2, 4, 64, 64, false, true, false, false)   \
  BSFP8_INST(FMT, 4, 2, 64, 128, false, true, false, false)  \
  BSFP8_INST(FMT, 1, 4, 64, 64, true, false, false, false)   \
  BSFP8_INST(FMT, 4, 2, 64, 128, true, false, false, false)  \
  BSFP8_INST(FMT, 1, 4, 64, 64, true, false, true, false)    \
  BSFP8_INST(FMT, 4, 2, 64, 128, true, false, true, false)
// UE8M0 tiles with staged (dword-aligned) activation scales
#define BSFP8_INST_UE8M0_STAGED                          \
  BSFP8_INST(1, 4, 2, 64, 128, false, false, false, true) \
  BSFP8_INST(1, 2, 4, 64, 64, false, false, false, true)  \
  BSFP8_INST(1, 2, 4, 64, 64, false, true, false, true)   \
  BSFP8_INST(1, 4, 2, 64, 128, false, true, false, true)  \
  BSFP8_INST(1, 4, 2, 64, 128, true, false, false, true)
BSFP8_INST_ALL(0)
BSFP8_INST_ALL(1)
BSFP8_INST_UE8M0_STAGED
// MXFP4 tiles with staged weight scales (K a multiple of 128; the 256 x 256
// tile with fp32 activation scales keeps the per-subtile loads: staged, the
// compiler spills it heavily)
BSFP8_INST2(0, 2, 4, 64, 64, false, true, false, false, true)
BSFP8_INST2(1, 4, 2, 64, 128, false, true, false, false, true)
BSFP8_INST2(1, 2, 4, 64, 64, false, true, false, false, true)
BSFP8_INST2(1, 4, 2, 64, 128, false, true, false, true, true)
BSFP8_INST2(1, 2, 4, 64, 64, false, true, false, true, true)
// MoE experts with MXFP4 weights: the two grouped tile classes, with and
// without staged weight scales (K a multiple of 128 or not)
#define BSFP8_INST_W4G(FMT)                                       \
  BSFP8_INST2(FMT, 4, 2, 64, 128, true, true, false, false, false) \
  BSFP8_INST2(FMT, 1, 4, 64, 64, true, true, false, false, false)  \
  BSFP8_INST2(FMT, 1, 4, 64, 64, true, true, false, false, true)
BSFP8_INST2(0, 2, 4, 64, 64, true, true, false, false, true)
BSFP8_INST_W4G(0)
BSFP8_INST_W4G(1)
BSFP8_INST2(1, 4, 2, 64, 128, true, true, false, false, true)
BSFP8_INST2(1, 4, 2, 64, 128, true, true, false, true, true)
#undef BSFP8_INST_W4G
// fp8_linear's fused large-M form: bf16 X quantized inside the 128 x 256 tile
BSFP8_INST3(0, 2, 4, 64, 64, false, false, false, false, false, true)
BSFP8_INST3(1, 2, 4, 64, 64, false, false, false, false, false, true)
#undef BSFP8_INST3
#undef BSFP8_INST_UE8M0_STAGED
#undef BSFP8_INST2
#undef BSFP8_INST_ALL
#undef BSFP8_INST

// ------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------
constexpr int64_t kDecodeMaxM = 16;
constexpr int64_t kDecodeFusedMaxNK = int64_t(1) << 24;
constexpr int64_t kDecodeFusedMaxK = 6144;
// fused act quant in the large-M GEMM: every 256-wide N tile re-encodes
// its M x K activations, about seven VALU operations per value, against the
// separate launch it saves.  Measured (fp32 and UE8M0 scales): 1.1-1.2x
// faster while M K ceil(N / 256) <= 2^21 (e.g. M = 32 at 4096 -> 4096 or
// 7168 -> 1536), break-even near 2^22, 0.55-0.9x beyond
constexpr int64_t kLinearXqMaxWork = int64_t(1) << 21;

// Large-M tile configurations (WAVES_M x WAVES_N waves, wave tile WM x WN,
// two LDS stages): BM = WM WAVES_M, BN = WN WAVES_N.
//   small: 128 x 256, 8 waves of 64 x 64 (two per SIMD)
//   short: 64 x 256, 4 waves of 64 x 64, two workgroups per CU (MoE
//          segments of at most 128 rows)
//   big:   256 x 256, 8 waves of 64 x 128 (two per SIMD); per flop a third
//          fewer operand bytes through L2 and the texture path and a quarter
//          fewer LDS fragment reads than the small tile, so it runs about
//          1.5x faster per CU once every CU has a tile of its own.
// Two stages wait for vmcnt(0) before each K block, which does not depend
// on the completion order of the LDS-DMA loads and the scale loads.
template <int FMT, int WMN, int WNN, int WM, int WN, bool GROUPED, bool W4 = false,
          bool SW = false, bool SA = false, bool SW4 = false, bool XQ = false>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t st, int splits, int kbps, int gsel = 0) {
  constexpr int BM = WMN * WM, BN = WNN * WN;
  const int64_t NT = (a.N + BN - 1) / BN;
  int64_t tiles;
  if (GROUPED) {
    // upper bound on the class's M tiles: every expert adds <= 1 partial
    // tile; more than kSmallSegment rows each bounds the count of big ones
    const int64_t full = (a.M + BM - 1) / BM;
    const int64_t parts = gsel == 1 ? std::min<int64_t>(a.E, a.M / (kSmallSegment + 1) + 1)
                                    : (int64_t)a.E;
    tiles = (gsel == 2 ? (int64_t)a.E * ((kSmallSegment + BM - 1) / BM) : full + parts) * NT;
  } else {
    tiles = (a.M + BM - 1) / BM * NT * splits;
  }
  tiles = (tiles + 7) / 8 * 8;                   // whole rounds over the 8 XCDs
  float* part = splits > 1 ? (float*)a.workspace : nullptr;
  hipLaunchKernelGGL((gemm_lds_kernel<FMT, WMN, WNN, WM, WN, GROUPED, W4, SW, SA, SW4, XQ>),
                     dim3((unsigned)tiles), dim3(64 * WMN * WNN), 0, st, a.xq, a.xs, a.wq, a.ws,
                     GROUPED ? nullptr : a.bias, a.y, a.M, a.N, a.K, a.seg, a.E, gsel, part,
                     kbps, a.hq, a.hs, XQ ? a.x_bf16 : nullptr, XQ ? a.ldx : (int64_t)0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || part == nullptr) return e;
  const int64_t MN = a.M * a.N;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256), 0,
                     st, part, splits, MN, a.N, a.bias, a.y);
  return hipGetLastError();
}

// Tile and K-split choice for a dense launch, from a cost model of one
// round of workgroups over the 256 CUs: rounds x K blocks per split x the
// measured time of one K block of one tile (2.15 us for 128 x 256 tiles,
// 2.8 us for 256 x 256 tiles with fp32 scales; UE8M0 runs both about 1.3x
// faster, which leaves the choice unchanged), plus, when K is split, one
// reduction launch and the fp32 partial sums written and read back at
// about 5 TB/s.  A grid of few tiles leaves CUs idle that smaller tiles or
// K splits fill; splits pay for their partial sums.
struct Plan {
  int big;      // 256 x 256 tiles, else 128 x 256
  int splits;   // K splits (1: no split, bf16 written directly)
  int kbps;     // K blocks per split
};

Plan plan_dense(int64_t M, int64_t N, int64_t K, bool allow_big = true) {
  constexpr int64_t kCUs = 256;                 // MI355X compute units
  const double t_blk[2] = {2.15, 2.8};
  const int64_t KB = (K + 127) / 128;
  Plan best{0, 1, (int)KB};
  double best_t = 1e300;
  for (int big = 0; big < (allow_big ? 2 : 1); ++big) {
    const int64_t BM = big ? 256 : 128;
    const int64_t tiles = (M + BM - 1) / BM * ((N + 255) / 256);
    for (int64_t S = 1; S <= 32; S *= 2) {
      if (S > 1 && KB < 2 * S) break;           // at least two K blocks per split
      const int64_t kbps = (KB + S - 1) / S;
      const int64_t real = (KB + kbps - 1) / kbps;
      const int64_t rounds = (tiles * real + kCUs - 1) / kCUs;
      double t = (double)rounds * (double)kbps * t_blk[big];
      if (real > 1) t += 3.0 + (double)real * (double)M * (double)N * 8.0 / 5e6;
      if (t < best_t) {
        best_t = t;
        best = Plan{big, (int)real, (int)kbps};
      }
    }
  }
  return best;
}

// UE8M0 activation scales can be staged in dword chunks: every row and every
// K split starts on a multiple of 4 scale bytes
inline bool ue8m0_aligned(const GemmArgs& a, int splits, int kbps) {
  const int64_t KB = (a.K + 127) / 128;
  return a.fmt == 1 && KB % 4 == 0 && (splits == 1 || kbps % 4 == 0);
}

template <int FMT, bool GROUPED, bool SW = false>
hipError_t launch_lds(const GemmArgs& a, hipStream_t st) {
  constexpr bool U = FMT == 1;   // staged UE8M0 scales exist for FMT 1 only
  if constexpr (SW) {
    // gate/up tiles with the SiLU-mul requant epilogue: the same two expert
    // classes and tile shapes as the plain grouped GEMM
    const int kb = (int)((a.K + 127) / 128);
    hipError_t e = launch_cfg<FMT, 4, 2, 64, 128, true, false, true>(a, st, 1, kb, 1);
    if (e != hipSuccess) return e;
    return launch_cfg<FMT, 1, 4, 64, 64, true, false, true>(a, st, 1, kb, 2);
  } else if constexpr (GROUPED) {
    // experts with many rows on 256 x 256 tiles, the short segments (most
    // of them under skewed routing) on 64 x 256 tiles of four waves (two
    // workgroups per CU), which pad a 42-row median segment to 64 rather
    // than 128: two launches over disjoint experts, each with its own
    // device-built tile table
    const int kb = (int)((a.K + 127) / 128);
    if (a.w4) {
      // MXFP4 experts: the dense FP8 x MXFP4 tiles over the same two expert
      // classes; weight scales staged through LDS when K is a multiple of
      // 128 (for the big tile with UE8M0 scales only: with fp32 activation
      // scales the staged big tile spills)
      const bool sw4 = a.K % 128 == 0;
      hipError_t e;
      if constexpr (FMT == 1) {
        if (sw4)
          e = ue8m0_aligned(a, 1, kb)
                  ? launch_cfg<FMT, 4, 2, 64, 128, true, true, false, true, true>(a, st, 1, kb, 1)
                  : launch_cfg<FMT, 4, 2, 64, 128, true, true, false, false, true>(a, st, 1, kb, 1);
        else
          e = launch_cfg<FMT, 4, 2, 64, 128, true, true>(a, st, 1, kb, 1);
      } else {
        // fp32 activation scales: the large experts on 128 x 256 tiles, whose
        // staged weight scales fit (the 256 x 256 tile loads a scale byte per
        // lane, subtile and K block: 2x slower on the MoE gate/up shape)
        e = sw4 ? launch_cfg<FMT, 2, 4, 64, 64, true, true, false, false, true>(a, st, 1, kb, 1)
                : launch_cfg<FMT, 4, 2, 64, 128, true, true>(a, st, 1, kb, 1);
      }
      if (e != hipSuccess) return e;
      return sw4 ? launch_cfg<FMT, 1, 4, 64, 64, true, true, false, false, true>(a, st, 1, kb, 2)
                 : launch_cfg<FMT, 1, 4, 64, 64, true, true>(a, st, 1, kb, 2);
    }
    const hipError_t e = ue8m0_aligned(a, 1, kb)
                             ? launch_cfg<FMT, 4, 2, 64, 128, true, false, false, U>(a, st, 1, kb, 1)
                             : launch_cfg<FMT, 4, 2, 64, 128, true>(a, st, 1, kb, 1);
    if (e != hipSuccess) return e;
    return launch_cfg<FMT, 1, 4, 64, 64, true>(a, st, 1, kb, 2);
  } else {
    const Plan p = plan_dense(a.M, a.N, a.K);
    if (a.x_bf16) {
      // fp8_linear's fused form (linear_xq chose it: the plan's small tile),
      // the same tile and K splits as fp8_block_gemm, so the same sums
      return launch_cfg<FMT, 2, 4, 64, 64, false, false, false, false, false, true>(a, st, p.splits,
                                                                                  p.kbps);
    }
    const bool sa = ue8m0_aligned(a, p.splits, p.kbps);
    if (a.w4) {
      if (a.K % 128 == 0 && (FMT == 1 || !p.big)) {   // staged MXFP4 weight scales
        if constexpr (FMT == 1) {
          if (p.big)
            return sa ? launch_cfg<FMT, 4, 2, 64, 128, false, true, false, U, true>(a, st, p.splits,
                                                                                    p.kbps)
                      : launch_cfg<FMT, 4, 2, 64, 128, false, true, false, false, true>(a, st, p.splits,
                                                                                    p.kbps);
        }
        return sa ? launch_cfg<FMT, 2, 4, 64, 64, false, true, false, U, true>(a, st, p.splits, p.kbps)
                  : launch_cfg<FMT, 2, 4, 64, 64, false, true, false, false, true>(a, st, p.splits,
                                                                                 p.kbps);
      }
      if (p.big)
        return sa ? launch_cfg<FMT, 4, 2, 64, 128, false, true, false, U>(a, st, p.splits, p.kbps)
                  : launch_cfg<FMT, 4, 2, 64, 128, false, true>(a, st, p.splits, p.kbps);
      return sa ? launch_cfg<FMT, 2, 4, 64, 64, false, true, false, U>(a, st, p.splits, p.kbps)
                : launch_cfg<FMT, 2, 4, 64, 64, false, true>(a, st, p.splits, p.kbps);
    }
    if (p.big)
      return sa ? launch_cfg<FMT, 4, 2, 64, 128, false, false, false, U>(a, st, p.splits, p.kbps)
                : launch_cfg<FMT, 4, 2, 64, 128, false>(a, st, p.splits, p.kbps);
    return sa ? launch_cfg<FMT, 2, 4, 64, 64, false, false, false, U>(a, st, p.splits, p.kbps)
              : launch_cfg<FMT, 2, 4, 64, 64, false>(a, st, p.splits, p.kbps);
  }
}

}  // namespace detail
using namespace detail;

size_t fp8_fp4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= kDecodeMaxM || N <= 0 || K <= 0) return 0;
  const Plan p = plan_dense(M, N, K);
  return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= kDecodeMaxM || N <= 0 || K <= 0) return 0;
  const Plan p = plan_dense(M, N, K);
  return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
}

// The persistent decode kernel where it measured faster than
// gemm_decode_kernel: X codes and scales that fit its LDS, and several tiles
// per resident workgroup (counted for 256 CUs) or long rows; below 4 token
// rows (no X reuse worth its copy) only with at least two blocks per wave
// and tile.  1.1-1.4x at M = 4..16 on 4096 x 28672, 7168 x 18432,
// 1536 x 24576, 14336 x 4096; 1.03-1.1x at M = 1..3 on the long-row and
// many-tile shapes; slower on one tile of short rows per workgroup.
// (The fp32 activation scales, M KB 4 bytes, fit whenever the codes do.)
bool decode_pers(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || M > kDecodeMaxM || N <= 0 || K <= 0) return false;
  const int64_t KB = (K + 127) / 128;
  if (M * (K + 16) > kPersXlBytes || M * KB * 4 > kPersXsBytes) return false;
  const int64_t ntiles = (N + 15) / 16;
  const int64_t nbw = (KB + kDecodeWaves - 1) / kDecodeWaves;
  if (!(2 * ntiles >= 3 * 256 || KB >= 48)) return false;
  return M >= 4 || nbw >= 2;
}

// fp8_linear's one-launch decode forms: gemm_decode_kernel quantizing per
// block (every workgroup re-encodes X, so only while N K is small), or the
// persistent kernel quantizing X once per workgroup while M K is small
// enough that this prologue costs less than a quantization launch
// (measured: faster up to 4 x 7168 and 2 x 18432, slower at 4 x 14336 and
// 16 x 4096)
constexpr int64_t kPersFusedMaxMK = 40960;
bool linear_fused(int64_t M, int64_t N, int64_t K) {
  if (M > 0 && M * K <= kPersFusedMaxMK && decode_pers(M, N, K)) return true;
  return M > 0 && M <= kDecodeMaxM && K <= kDecodeFusedMaxK && N * K <= kDecodeFusedMaxNK;
}

// fp8_linear quantizes the activations inside the large-M GEMM (128 x 256
// tiles, the plan's choice) instead of staging them with a separate launch
bool linear_xq(int64_t M, int64_t N, int64_t K) {
  if (M <= kDecodeMaxM || N <= 0 || K <= 0) return false;
  if (M * K * ((N + 255) / 256) > kLinearXqMaxWork) return false;
  return !plan_dense(M, N, K).big;
}

size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int blk) {
  if (M <= 0) return 0;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  if (blk == 32) return up((size_t)M * K) + up((size_t)M * ((K + 31) / 32) * 4);
  if (linear_fused(M, N, K)) return 0;   // quantization inside the decode kernel
  if (linear_xq(M, N, K)) return gemm_workspace_bytes(M, N, K);   // inside the large-M GEMM
  const int64_t G = (K + 127) / 128;
  return up((size_t)M * K) + up((size_t)M * G * 4) + gemm_workspace_bytes(M, N, K);
}

size_t grouped_workspace_bytes(int64_t, int64_t, int64_t, int) { return 0; }

int gemm_kind(int64_t M, int64_t N, int64_t K, int* splits) {
  if (splits) *splits = 1;
  if (M <= 0 || N <= 0 || K <= 0) return BSFP8_GEMM_NONE;
  if (M <= kDecodeMaxM) return BSFP8_GEMM_DECODE;
  const Plan p = plan_dense(M, N, K);
  if (splits) *splits = p.splits;
  return p.big ? BSFP8_GEMM_TILE_256x256 : BSFP8_GEMM_TILE_128x256;
}

// compute units of the current device, queried once per device
int cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev] = cus;
  }
  return cache[dev];
}

template <int FMT, int DEPTH, bool FUSED>
hipError_t launch_pers(const GemmArgs& a, hipStream_t st, int ntiles, int res) {
  const int grid = ntiles < res ? ntiles : res;
  hipLaunchKernelGGL((gemm_decode_pers_kernel<FMT, DEPTH, FUSED>), dim3((unsigned)grid),
                     dim3(64 * kDecodeWaves), 0, st, a.xq, a.xs, a.wq, a.ws, a.bias, a.y, (int)a.M,
                     a.N, a.K, ntiles, FUSED ? a.x_bf16 : nullptr, FUSED ? a.ldx : (int64_t)0,
                     FUSED ? a.xstat : nullptr);
  return hipGetLastError();
}

// chunk depth from the blocks each wave takes per tile: the depth (2 or 3:
// 128 VGPRs at 16 waves) that pads the fewest slots
template <int FMT, bool FUSED>
hipError_t launch_pers_depth(const GemmArgs& a, hipStream_t st) {
  const int64_t KB = (a.K + 127) / 128;
  const int ntiles = (int)((a.N + 15) / 16);
  const int res = cu_count();        // its LDS holds one workgroup per CU
  if (res <= 0) return hipErrorInvalidDevice;
  const int nbw = (int)((KB + kDecodeWaves - 1) / kDecodeWaves);
  const int d = nbw <= 3 ? nbw : ((nbw + 2) / 3 * 3 - nbw <= (nbw + 1) / 2 * 2 - nbw ? 3 : 2);
  switch (d) {
    case 1: return launch_pers<FMT, 1, FUSED>(a, st, ntiles, res);
    case 2: return launch_pers<FMT, 2, FUSED>(a, st, ntiles, res);
    default: return launch_pers<FMT, 3, FUSED>(a, st, ntiles, res);
  }
}

template <int FMT>
hipError_t launch_decode(const GemmArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.N + 15) / 16));
  const dim3 block(64 * kDecodeWaves);
  // staged activation scales when the M x KB scales fit the LDS slot and
  // several token rows share the staging (at M = 1 its prologue costs more
  // than the one scale row's loads it saves)
  const bool sxl = a.M >= 4 && a.M * ((a.K + 127) / 128) * (a.fmt == 0 ? 4 : 1) <= kDecodeXsBytes;
  const bool pers = decode_pers(a.M, a.N, a.K);
  if (a.x_bf16 && pers && a.M * a.K <= kPersFusedMaxMK && a.M * a.ldx * 2 <= 0x7fffffffLL) {
    return launch_pers_depth<FMT, true>(a, st);
  } else if (a.x_bf16 && a.M >= 8 && a.M * a.ldx * 2 <= 0x7fffffffLL) {
    // from 8 tokens the branch-free loads (XB; the activations through a
    // buffer resource over M ldx bf16 values, so that span must fit its
    // 32-bit range): 1.12x at 16 x 4096 x 4096; below 8 tokens they measured
    // 1-4% slower and the loads stay behind their branches
    hipLaunchKernelGGL((gemm_decode_kernel<FMT, true>), grid, block, 0, st, nullptr, nullptr,
                       a.x_bf16, a.ldx, a.wq, a.ws, a.bias, a.y, (int)a.M, a.N, a.K, a.xstat);
  } else if (a.x_bf16) {
    hipLaunchKernelGGL((gemm_decode_kernel<FMT, true, false, false, false, false, false>), grid,
                       block, 0, st, nullptr, nullptr, a.x_bf16, a.ldx, a.wq, a.ws, a.bias, a.y,
                       (int)a.M, a.N, a.K, a.xstat);
  } else if (a.blk == 32) {
    // (32, 32) blocks: the M x K/32 activation scales (M >= 4) and the tile's
    // row of weight-block scales from LDS
    const int64_t gbytes = (a.K + 31) / 32 * (a.fmt == 0 ? 4 : 1);
    const bool sx32 = a.M >= 4 && a.M * gbytes <= kDecodeXsBytes;
    const bool sw32 = a.M >= 4 && gbytes <= kDecodeXsBytes;   // at M = 1 the copy costs more
#define BSFP8_DEC32(SX, SW)                                                                     \
  hipLaunchKernelGGL((gemm_decode_kernel<FMT, false, false, true, SX, SW>), grid, block, 0, st, \
                     a.xq, a.xs, nullptr, (int64_t)0, a.wq, a.ws, a.bias, a.y, (int)a.M, a.N, a.K, \
                     nullptr)
    if (sx32 && sw32) BSFP8_DEC32(true, true);
    else if (sw32) BSFP8_DEC32(false, true);
    else BSFP8_DEC32(false, false);
#undef BSFP8_DEC32
  } else if (a.w4) {
    // staged MXFP4 weight scales when 16 rows of them fit and rows are dword-aligned
    const bool swl = a.K % 128 == 0 && 16 * (a.K / 32) <= kDecodeXsBytes;
#define BSFP8_DEC4(SX, SW)                                                                      \
  hipLaunchKernelGGL((gemm_decode_kernel<FMT, false, true, false, SX, SW>), grid, block, 0, st, \
                     a.xq, a.xs, nullptr, (int64_t)0, a.wq, a.ws, a.bias, a.y, (int)a.M, a.N, a.K, \
                     nullptr)
    if (sxl && swl) BSFP8_DEC4(true, true);
    else if (sxl) BSFP8_DEC4(true, false);
    else if (swl) BSFP8_DEC4(false, true);
    else BSFP8_DEC4(false, false);
#undef BSFP8_DEC4
  } else if (pers) {
    return launch_pers_depth<FMT, false>(a, st);
  } else {
    if (sxl)
      hipLaunchKernelGGL((gemm_decode_kernel<FMT, false, false, false, true>), grid, block, 0, st,
                         a.xq, a.xs, nullptr, (int64_t)0, a.wq, a.ws, a.bias, a.y, (int)a.M, a.N,
                         a.K, nullptr);
    else if (a.M >= 8)
      hipLaunchKernelGGL((gemm_decode_kernel<FMT, false>), grid, block, 0, st, a.xq, a.xs, nullptr,
                         (int64_t)0, a.wq, a.ws, a.bias, a.y, (int)a.M, a.N, a.K, nullptr);
    else
      hipLaunchKernelGGL((gemm_decode_kernel<FMT, false, false, false, false, false, false>), grid,
                         block, 0, st, a.xq, a.xs, nullptr, (int64_t)0, a.wq, a.ws, a.bias, a.y,
                         (int)a.M, a.N, a.K, nullptr);
  }
  return hipGetLastError();
}

template <bool G>
hipError_t launch_b32(const GemmArgs& a, hipStream_t st) {
  const int64_t NT = (a.N + 127) / 128;
  // grouped: every expert adds at most one partial M tile
  int64_t tiles = G ? ((a.M + 127) / 128 + a.E) * NT : (a.M + 127) / 128 * NT;
  tiles = (tiles + 7) / 8 * 8;                   // whole rounds over the 8 XCDs
  const uint16_t* bias = G ? nullptr : a.bias;
#define BSFP8_B32L(FMT, SA)                                                                       \
  hipLaunchKernelGGL((gemm_b32_kernel<FMT, SA, G>), dim3((unsigned)tiles), dim3(256), 0, st, a.xq, \
                     a.xs, a.wq, a.ws, bias, a.y, a.M, a.N, a.K, a.seg, a.E)
  if (a.fmt == 0) BSFP8_B32L(0, false);
  else if (a.K % 128 == 0) BSFP8_B32L(1, true);   // UE8M0 rows of K/32 bytes dword-aligned: staged
  else BSFP8_B32L(1, false);
#undef BSFP8_B32L
  return hipGetLastError();
}

hipError_t launch_block_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.blk == 32 && a.M > kDecodeMaxM) return launch_b32<false>(a, st);
  if (a.M <= kDecodeMaxM) return a.fmt == 0 ? launch_decode<0>(a, st) : launch_decode<1>(a, st);
  return a.fmt == 0 ? launch_lds<0, false>(a, st) : launch_lds<1, false>(a, st);
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.blk == 32) return launch_b32<true>(a, st);
  return a.fmt == 0 ? launch_lds<0, true>(a, st) : launch_lds<1, true>(a, st);
}

hipError_t launch_grouped_silu_mul_quant(const GemmArgs& a, hipStream_t st) {
  return a.fmt == 0 ? launch_lds<0, true, true>(a, st) : launch_lds<1, true, true>(a, st);
}

}  // namespace bsfp8
