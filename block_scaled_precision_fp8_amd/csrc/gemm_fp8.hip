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
//   gemm_lds_kernel     large M: workgroup tile BM x BN, operands staged in
//                       LDS (double-buffered, XOR-swizzled 16-byte chunks),
//                       XCD-aware tile order.  Also serves the MoE grouped
//                       GEMM through a device-built tile table.
//   gemm_stream_kernel  small M (<= 128): weight-streaming split-K kernel,
//                       W fragments loaded straight into registers.
//   splitk_reduce_kernel  fp32 partials -> bf16 (+ bias).
#include "bsfp8_internal.h"

namespace bsfp8 {
namespace {

constexpr int kRowBytes = 128;   // one K block of FP8 codes

__device__ __forceinline__ v8i join(uint4 a, uint4 b) {
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

template <int FMT>
__device__ __forceinline__ float load_scale(const void* p, int64_t idx) {
  if (FMT == 0) return ((const float*)p)[idx];
  return __int_as_float(((const uint8_t*)p)[idx]);   // carries the byte
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
  bool valid;
};

template <int BM, int BN>
__device__ __forceinline__ Tile dense_tile(int64_t M, int64_t N) {
  const int MT = (int)((M + BM - 1) / BM), NT = (int)((N + BN - 1) / BN);
  const int T = MT * NT;
  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so
  // bid -> (xcd, slot) and consecutive logical tiles go to one XCD.
  const int bid = blockIdx.x;
  const int per_xcd = (int)(gridDim.x / 8);
  int t = (bid & 7) * per_xcd + (bid >> 3);
  Tile tl;
  tl.valid = t < T;
  tl.expert = 0;
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
template <int BM, int BN, int THREADS>
__device__ __forceinline__ Tile grouped_tile(const int32_t* __restrict__ seg, int E, int64_t N,
                                             int* s_pref) {
  const int NT = (int)((N + BN - 1) / BN);
  // per-expert M-tile counts, then an inclusive scan (Hillis-Steele).
  for (int e = threadIdx.x; e < E; e += THREADS) {
    const int rows = seg[e + 1] - seg[e];
    s_pref[e + 1] = (rows + BM - 1) / BM;
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
  const int t = blockIdx.x;
  const int total = s_pref[E] * NT;
  tl.valid = t < total;
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

template <int FMT, int BM, int BN, int WAVES_M, int WAVES_N, bool GROUPED>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void gemm_lds_kernel(
    const uint8_t* __restrict__ xq, const void* __restrict__ xs, const uint8_t* __restrict__ wq,
    const void* __restrict__ wsc, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int64_t M, int64_t N, int64_t K, const int32_t* __restrict__ seg, int E) {
  constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int MI = WM / 16, NI = WN / 16;
  static_assert(128 % WN == 0 || WN % 128 == 0, "wave N range inside one weight block");
  static_assert(WN <= 128, "wave N range inside one weight block");
  constexpr int XCH = BM * 8 / THREADS;     // 16-byte chunks per thread per stage
  constexpr int WCH = BN * 8 / THREADS;
  constexpr int STAGE = (BM + BN) * kRowBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];
  __shared__ int s_pref[GROUPED ? 1025 : 1];

  Tile tl;
  if (GROUPED) tl = grouped_tile<BM, BN, THREADS>(seg, E, N, s_pref);
  else tl = dense_tile<BM, BN>(M, N);
  if (!tl.valid) return;

  const int64_t KB = (K + 127) / 128;
  const int64_t NB = (N + 127) / 128;
  const uint8_t* wbase = wq + (int64_t)tl.expert * N * K;
  const uint8_t* wsb = (const uint8_t*)wsc + (int64_t)tl.expert * NB * KB * (FMT == 0 ? 4 : 1);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int l16 = lane & 15, g4 = lane >> 4;

  // ---- global -> register staging of one K block
  uint4 xr[XCH], wr[WCH];
  auto gload = [&](int64_t kb) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + THREADS * i;
      const int row = c >> 3, ch = c & 7;
      const int64_t m = tl.m0 + row;
      const int64_t k = kb * 128 + ch * 16;
      xr[i] = make_uint4(0, 0, 0, 0);
      if (m < tl.mlim && k < K) xr[i] = *(const uint4*)(xq + m * K + k);
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = tid + THREADS * i;
      const int row = c >> 3, ch = c & 7;
      const int64_t n = tl.n0 + row;
      const int64_t k = kb * 128 + ch * 16;
      wr[i] = make_uint4(0, 0, 0, 0);
      if (n < N && k < K) wr[i] = *(const uint4*)(wbase + n * K + k);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* sx = lds + buf * STAGE;
    uint8_t* sw = sx + BM * kRowBytes;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int c = tid + THREADS * i;
      const int row = c >> 3, ch = c & 7;
      *(uint4*)(sx + row * kRowBytes + ((ch ^ (row & 7)) << 4)) = xr[i];
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = tid + THREADS * i;
      const int row = c >> 3, ch = c & 7;
      *(uint4*)(sw + row * kRowBytes + ((ch ^ (row & 7)) << 4)) = wr[i];
    }
  };
  // fragment read: 16 rows x 128 codes, lane (l16, g4) gets row l16, bytes
  // [32 g4, 32 g4 + 32) -- the same K split for both operands.
  auto frag = [&](const uint8_t* base, int row) -> v8i {
    const uint8_t* r = base + row * kRowBytes;
    const uint4 a = *(const uint4*)(r + (((2 * g4) ^ (row & 7)) << 4));
    const uint4 b = *(const uint4*)(r + (((2 * g4 + 1) ^ (row & 7)) << 4));
    return join(a, b);
  };

  v4f acc[NI][MI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // per-lane token rows for the scales and the epilogue
  int64_t mrow[MI];
#pragma unroll
  for (int j = 0; j < MI; ++j) mrow[j] = tl.m0 + wm * WM + j * 16 + l16;
  const int64_t nwave = tl.n0 + wn * WN;
  const int64_t nblk = nwave >> 7;

  gload(0);
  sstore(0);
  __syncthreads();

  for (int64_t kb = 0; kb < KB; ++kb) {
    const int buf = (int)(kb & 1);
    if (kb + 1 < KB) gload(kb + 1);
    float sa[MI];
#pragma unroll
    for (int j = 0; j < MI; ++j)
      sa[j] = (mrow[j] < tl.mlim) ? load_scale<FMT>(xs, mrow[j] * KB + kb)
                                  : (FMT == 0 ? 0.f : __int_as_float(127));
    const float sw = (nwave < N) ? load_scale<FMT>(wsb, nblk * KB + kb)
                                 : (FMT == 0 ? 0.f : __int_as_float(127));
    const uint8_t* sx = lds + buf * STAGE;
    const uint8_t* swl = sx + BM * kRowBytes;
    v8i bx[MI];
#pragma unroll
    for (int j = 0; j < MI; ++j) bx[j] = frag(sx, wm * WM + j * 16 + l16);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const v8i aw = frag(swl, wn * WN + i * 16 + l16);
#pragma unroll
      for (int j = 0; j < MI; ++j) acc[i][j] = mfma_step<FMT>(acc[i][j], aw, bx[j], sa[j], sw);
    }
    if (kb + 1 < KB) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds n = nwave + 16 i + 4 g4 + {0..3}, m = mrow[j]
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int64_t n = nwave + i * 16 + 4 * g4;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < MI; ++j)
      if (mrow[j] < tl.mlim) store_out4(y, N, mrow[j], n, acc[i][j], bias);
  }
}

// ------------------------------------------------------------------------
// Small-M weight-streaming kernel: each wave owns 16 weight rows and walks
// the K blocks [kb0, kb1) of its split; W fragments go straight from HBM to
// registers (each weight byte is used by exactly one wave), X fragments and
// scales come from L2.  MT = number of 16-token column tiles.
// ------------------------------------------------------------------------
constexpr int kStreamWaves = 4;
constexpr int kStreamUnroll = 4;

template <int FMT, int MT>
__global__ __launch_bounds__(64 * kStreamWaves) void gemm_stream_kernel(
    const uint8_t* __restrict__ xq, const void* __restrict__ xs, const uint8_t* __restrict__ wq,
    const void* __restrict__ wsc, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    float* __restrict__ part, int M, int64_t N, int64_t K, int kb_per_split) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int64_t n0 = ((int64_t)blockIdx.x * kStreamWaves + wave) * 16;
  if (n0 >= N) return;
  const int64_t KB = (K + 127) / 128;
  const int64_t kb0 = (int64_t)blockIdx.y * kb_per_split;
  const int64_t kb1 = min(KB, kb0 + kb_per_split);
  const int64_t nrow = n0 + l16;
  const bool nvalid = nrow < N;
  const int64_t nblk = n0 >> 7;

  v4f acc[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int64_t kb = kb0; kb < kb1; kb += kStreamUnroll) {
    uint4 wa[kStreamUnroll], wb[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t k = (kb + u) * 128 + g4 * 32;
      wa[u] = make_uint4(0, 0, 0, 0);
      wb[u] = make_uint4(0, 0, 0, 0);
      if (kb + u < kb1 && nvalid) {
        if (k < K) wa[u] = ld_stream16(wq + nrow * K + k);
        if (k + 16 < K) wb[u] = ld_stream16(wq + nrow * K + k + 16);
      }
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      if (kb + u >= kb1) break;
      const int64_t k = (kb + u) * 128 + g4 * 32;
      const float sw = load_scale<FMT>(wsc, nblk * KB + kb + u);
      const v8i aw = join(wa[u], wb[u]);
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int m = j * 16 + l16;
        uint4 xa = make_uint4(0, 0, 0, 0), xb = make_uint4(0, 0, 0, 0);
        float sa = (FMT == 0) ? 0.f : __int_as_float(127);
        if (m < M) {
          if (k < K) xa = *(const uint4*)(xq + (int64_t)m * K + k);
          if (k + 16 < K) xb = *(const uint4*)(xq + (int64_t)m * K + k + 16);
          sa = load_scale<FMT>(xs, (int64_t)m * KB + kb + u);
        }
        acc[j] = mfma_step<FMT>(acc[j], aw, join(xa, xb), sa, sw);
      }
    }
  }

  // lane holds n = n0 + 4 g4 + {0..3} for token m = 16 j + l16
  const int64_t n = n0 + 4 * g4;
  if (n >= N) return;
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int m = j * 16 + l16;
    if (m >= M) continue;
    if (part == nullptr) {
      store_out4(y, N, m, n, acc[j], bias);
    } else {
      float* p = part + ((int64_t)blockIdx.y * M + m) * N + n;
      *(float4*)p = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
    }
  }
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
// host side
// ------------------------------------------------------------------------
constexpr int kBM = 128, kBN = 256, kWavesM = 2, kWavesN = 2;
constexpr int64_t kStreamMaxM = 128;

int stream_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t KB = (K + 127) / 128;
  const int64_t wg_n = (N + 16 * kStreamWaves - 1) / (16 * kStreamWaves);
  int64_t want = (2048 + wg_n - 1) / wg_n;            // ~8 workgroups per CU
  int64_t max_by_depth = KB / 4;                      // >= 4 K blocks per split
  int64_t s = want < max_by_depth ? want : max_by_depth;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  (void)M;
  return (int)s;
}

template <int FMT>
hipError_t launch_stream(const GemmArgs& a, hipStream_t st) {
  const int splits = stream_splits(a.M, a.N, a.K);
  const int64_t KB = (a.K + 127) / 128;
  const int kbps = (int)((KB + splits - 1) / splits);
  const int real_splits = (int)((KB + kbps - 1) / kbps);
  float* part = real_splits > 1 ? (float*)a.workspace : nullptr;
  dim3 grid((unsigned)((a.N + 16 * kStreamWaves - 1) / (16 * kStreamWaves)), real_splits);
  const int M = (int)a.M;
#define BSFP8_STREAM(MT)                                                                     \
  hipLaunchKernelGGL((gemm_stream_kernel<FMT, MT>), grid, dim3(64 * kStreamWaves), 0, st,   \
                     a.xq, a.xs, a.wq, a.ws, a.bias, a.y, part, M, a.N, a.K, kbps)
  if (M <= 16) BSFP8_STREAM(1);
  else if (M <= 32) BSFP8_STREAM(2);
  else if (M <= 64) BSFP8_STREAM(4);
  else BSFP8_STREAM(8);
#undef BSFP8_STREAM
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || part == nullptr) return e;
  const int64_t MN = a.M * a.N;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((MN / 4 + 255) / 256)), dim3(256), 0,
                     st, part, real_splits, MN, a.N, a.bias, a.y);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_lds(const GemmArgs& a, hipStream_t st) {
  const int64_t MT = (a.M + kBM - 1) / kBM, NT = (a.N + kBN - 1) / kBN;
  int64_t tiles = MT * NT;
  tiles = (tiles + 7) / 8 * 8;   // whole rounds over the 8 XCDs
  hipLaunchKernelGGL((gemm_lds_kernel<FMT, kBM, kBN, kWavesM, kWavesN, false>),
                     dim3((unsigned)tiles), dim3(64 * kWavesM * kWavesN), 0, st, a.xq, a.xs, a.wq,
                     a.ws, a.bias, a.y, a.M, a.N, a.K, nullptr, 0);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || M > kStreamMaxM) return 0;
  const int splits = stream_splits(M, N, K);
  const int64_t KB = (K + 127) / 128;
  const int kbps = (int)((KB + splits - 1) / splits);
  const int real = (int)((KB + kbps - 1) / kbps);
  return real > 1 ? (size_t)real * M * N * sizeof(float) : 0;
}

size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0) return 0;
  const int64_t G = (K + 127) / 128;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  return up((size_t)M * K) + up((size_t)M * G * 4) + gemm_workspace_bytes(M, N, K);
}

size_t grouped_workspace_bytes(int64_t, int64_t, int64_t, int) { return 0; }

hipError_t launch_block_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M <= kStreamMaxM) return a.fmt == 0 ? launch_stream<0>(a, st) : launch_stream<1>(a, st);
  return a.fmt == 0 ? launch_lds<0>(a, st) : launch_lds<1>(a, st);
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t st) {
  // upper bound on tiles: every expert adds at most one partial M tile
  const int64_t NT = (a.N + kBN - 1) / kBN;
  const int64_t tiles = ((a.M + kBM - 1) / kBM + a.E) * NT;
  if (a.fmt == 0)
    hipLaunchKernelGGL((gemm_lds_kernel<0, kBM, kBN, kWavesM, kWavesN, true>), dim3((unsigned)tiles),
                       dim3(64 * kWavesM * kWavesN), 0, st, a.xq, a.xs, a.wq, a.ws, nullptr, a.y,
                       a.M, a.N, a.K, a.seg, a.E);
  else
    hipLaunchKernelGGL((gemm_lds_kernel<1, kBM, kBN, kWavesM, kWavesN, true>), dim3((unsigned)tiles),
                       dim3(64 * kWavesM * kWavesN), 0, st, a.xq, a.xs, a.wq, a.ws, nullptr, a.y,
                       a.M, a.N, a.K, a.seg, a.E);
  return hipGetLastError();
}

}  // namespace bsfp8
