// Hardware ceilings that bound the block-scaled GEMM kernels on one MI355X,
// measured with three small kernels (no library code):
//   1. vector-memory load throughput per CU, from an L2-resident 2 MB window
//      and from a 512 MB window in HBM, with LDS-DMA loads (16 bytes per
//      lane, as the GEMM kernels stage their operands) and with loads into
//      VGPRs (with and without a copy into LDS);
//   2. LDS read throughput per CU with 16-byte reads;
//   3. the scaled FP8 MFMA (16x16x128) alone, and followed by the fp32
//      promotion of its 16x16 result (acc += t * c, four FMAs per lane), at
//      one and two waves per SIMD;
//   4. the floor of a decode-shaped launch: 256 workgroups of 1024 lanes
//      reading 0-117 MB once (each lane 16-byte loads, four in flight),
//      back to back, the per-launch time and the rate.
// Build and run:
//   hipcc -O3 -std=c++17 --offload-arch=gfx950 -Xclang -target-feature \
//     -Xclang -packed-fp32-ops -o /tmp/bench_hw bench_hw.hip && /tmp/bench_hw
// Every load stays inside its buffer; every loop has a fixed trip count.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
#include <algorithm>

#define CHECK(x)                                                                \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);     \
      return 1;                                                                 \
    }                                                                           \
  } while (0)

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
#define LDSP(p) ((__attribute__((address_space(3))) void*)(p))
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// 1. loads: workgroup b reads chunk ((97 b + i) mod chunks) of the window at
// iteration i, THREADS x 16 bytes per chunk
template <int THREADS, int DEPTH>
__global__ __launch_bounds__(THREADS) void load_dma(const uint8_t* src, uint32_t window, int iters,
                                                    uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[DEPTH * THREADS * 16];
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src, window);
  const uint32_t chunk = THREADS * 16, nchunks = window / chunk;
  const int wave = threadIdx.x >> 6;
  for (int i = 0; i < iters; ++i) {
    const uint32_t c = (blockIdx.x * 97u + (uint32_t)i) % nchunks;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDSP(lds + (i % DEPTH) * chunk + wave * 1024), 16,
                                             c * chunk + threadIdx.x * 16, 0, 0, 0);
    if (i >= DEPTH - 1) wait_vmcnt<DEPTH - 1>();
  }
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0 && lds[3] == 0xAB && lds[1] == 0xCD) sink[blockIdx.x] = 1;
}

template <int THREADS, int DEPTH, bool TO_LDS>
__global__ __launch_bounds__(THREADS) void load_vgpr(const uint8_t* src, uint32_t window, int iters,
                                                     uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[TO_LDS ? DEPTH * THREADS * 16 : 16];
  const uint32_t chunk = THREADS * 16, nchunks = window / chunk;
  uint4 acc = make_uint4(0, 0, 0, 0), v[DEPTH];
  for (int i = 0; i < iters; i += DEPTH) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const uint32_t c = (blockIdx.x * 97u + (uint32_t)(i + u)) % nchunks;
      v[u] = *(const uint4*)(src + c * chunk + threadIdx.x * 16);
    }
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      if constexpr (TO_LDS) {
        *(uint4*)(lds + u * chunk + threadIdx.x * 16) = v[u];
      } else {
        acc.x ^= v[u].x; acc.y ^= v[u].y; acc.z ^= v[u].z; acc.w ^= v[u].w;
      }
    }
  }
  if constexpr (TO_LDS) {
    __syncthreads();
    if (threadIdx.x == 0 && lds[5] == 0xAB && lds[9] == 0xCD) sink[blockIdx.x] = 3;
  } else if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x12345678u) {
    sink[blockIdx.x] = 2;
  }
}

// 2. LDS reads: eight 16-byte reads per lane and iteration, contiguous per wave
template <int THREADS>
__global__ __launch_bounds__(THREADS) void lds_read(int iters, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[65536];
  for (int i = threadIdx.x * 16; i < 65536; i += THREADS * 16) *(uint4*)(lds + i) = make_uint4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  uint4 acc = make_uint4(0, 0, 0, 0);
  int base = ((threadIdx.x >> 6) * 1024 + (threadIdx.x & 63) * 16) & 65535;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint4 v = *(const uint4*)(lds + ((base + u * 8192) & 65535));
      acc.x ^= v.x; acc.y += v.y; acc.z ^= v.z; acc.w += v.w;
    }
    base = (base + 4096 + 16 * (i & 1)) & 65535;
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[blockIdx.x] = 4;
}

// 3. MFMA: PROMOTE = false accumulates in the MFMA; true writes a zero-based
// 16x16 result and adds it times c into the accumulator with four FMAs.
// Sixteen independent accumulators; distinct scale operands keep the MFMAs
// distinct, and the operands change every iteration.
template <bool PROMOTE>
__global__ __launch_bounds__(512) void mfma_loop(int iters, float c, uint32_t* sink) {
  v8i a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (int)(threadIdx.x * 0x01010101u + i);
    b[i] = (int)(threadIdx.x * 0x02020202u + 3 * i);
  }
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v4f acc[16];
  for (int j = 0; j < 16; ++j) acc[j] = zero;
  for (int it = 0; it < iters; ++it) {
    a[0] += 1;
    b[1] ^= it;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (PROMOTE) {
        const v4f t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0,
                                                                      127 - (j & 3), 0, 127 - (j >> 2));
        acc[j][0] = fmaf(t[0], c, acc[j][0]);
        acc[j][1] = fmaf(t[1], c, acc[j][1]);
        acc[j][2] = fmaf(t[2], c, acc[j][2]);
        acc[j][3] = fmaf(t[3], c, acc[j][3]);
      } else {
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], 0, 0, 0, 127, 0, 127);
      }
    }
  }
  float s = 0.f;
  for (int j = 0; j < 16; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (s == 1234.5f) sink[blockIdx.x] = 5;
}

// 4. one pass over `bytes` (a multiple of 16 x 1024 x 256): workgroup b
// reads its contiguous share, 16 bytes per lane per load, four in flight
template <int T>
__global__ __launch_bounds__(T) void stream_once(const uint4* __restrict__ src, int64_t n16,
                                                 uint32_t* sink) {
  const int64_t per = n16 / gridDim.x;
  const uint4* p = src + (int64_t)blockIdx.x * per;
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int64_t i = threadIdx.x; i < per; i += 4 * T) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i + u * T < per ? p[i + u * T] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) { acc.x ^= v[u].x; acc.y ^= v[u].y; acc.z ^= v[u].z; acc.w ^= v[u].w; }
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x2468ace0u) sink[blockIdx.x] = 6;
}

template <typename F>
static float time_ms(F launch, int reps) {
  hipEvent_t a, b;
  (void)hipEventCreate(&a);
  (void)hipEventCreate(&b);
  launch();
  (void)hipDeviceSynchronize();
  (void)hipEventRecord(a);
  for (int i = 0; i < reps; ++i) launch();
  (void)hipEventRecord(b);
  (void)hipEventSynchronize(b);
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, a, b);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return ms / reps;
}

int main() {
  int cus = 0, clk_khz = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  CHECK(hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeClockRate, 0));
  const double ghz = 2.1;   // the clock these kernels ran at under load (per-CU byte rates below)
  printf("CUs %d, rated clock %.2f GHz; per-CU rates are bytes per cycle at %.1f GHz\n", cus,
         clk_khz / 1e6, ghz);
  const size_t big = (size_t)1 << 30;
  uint8_t* src;
  uint32_t* sink;
  CHECK(hipMalloc(&src, big));
  CHECK(hipMalloc(&sink, 1 << 20));
  CHECK(hipMemset(src, 1, big));
  CHECK(hipMemset(sink, 0, 1 << 20));
  CHECK(hipDeviceSynchronize());

  printf("# 1. vector-memory loads: window | workgroups per CU | kind | us | TB/s | B/cycle/CU\n");
  for (uint32_t window : {2u << 20, 512u << 20}) {
    const int iters = window == (2u << 20) ? 2048 : 256;
    for (int per_cu : {1, 2}) {
      const int grid = cus * per_cu;
      auto report = [&](const char* name, int threads, float ms) {
        const double bytes = (double)grid * iters * threads * 16;
        printf("%4u MB | %d | %-28s | %8.1f | %6.2f | %6.1f\n", window >> 20, per_cu, name, ms * 1e3,
               bytes / (ms * 1e-3) / 1e12, bytes / (ms * 1e-3) / cus / (ghz * 1e9));
      };
      report("LDS-DMA, 512 lanes, 4 deep", 512, time_ms([&] {
        hipLaunchKernelGGL((load_dma<512, 4>), dim3(grid), dim3(512), 0, 0, src, window, iters, sink);
      }, 5));
      report("LDS-DMA, 256 lanes, 8 deep", 256, time_ms([&] {
        hipLaunchKernelGGL((load_dma<256, 8>), dim3(grid), dim3(256), 0, 0, src, window, iters, sink);
      }, 5));
      report("VGPR, 512 lanes, 8 deep", 512, time_ms([&] {
        hipLaunchKernelGGL((load_vgpr<512, 8, false>), dim3(grid), dim3(512), 0, 0, src, window, iters, sink);
      }, 5));
      report("VGPR + LDS copy, 512 lanes", 512, time_ms([&] {
        hipLaunchKernelGGL((load_vgpr<512, 4, true>), dim3(grid), dim3(512), 0, 0, src, window, iters, sink);
      }, 5));
      CHECK(hipGetLastError());
    }
  }

  printf("# 2. LDS reads (16 bytes per lane): lanes per CU | us | B/cycle/CU\n");
  for (int threads : {512, 1024}) {
    const int iters = 4096;
    const float ms = time_ms([&] {
      if (threads == 512) hipLaunchKernelGGL((lds_read<512>), dim3(cus), dim3(512), 0, 0, iters, sink);
      else hipLaunchKernelGGL((lds_read<1024>), dim3(cus), dim3(1024), 0, 0, iters, sink);
    }, 5);
    const double bytes = (double)threads * iters * 8 * 16;
    printf("%4d | %8.1f | %6.1f\n", threads, ms * 1e3, bytes / (ms * 1e-3) / (ghz * 1e9));
  }
  CHECK(hipGetLastError());

  printf("# 3. scaled FP8 MFMA 16x16x128: kind | waves per SIMD | us | TFLOP/s (dense peak 5000)\n");
  const int iters = 20000;
  for (int promote = 0; promote < 2; ++promote) {
    for (int threads : {256, 512}) {
      const float ms = time_ms([&] {
        if (promote) hipLaunchKernelGGL((mfma_loop<true>), dim3(cus), dim3(threads), 0, 0, iters, 0.5f, sink);
        else hipLaunchKernelGGL((mfma_loop<false>), dim3(cus), dim3(threads), 0, 0, iters, 0.5f, sink);
      }, 3);
      const double fl = (double)cus * (threads / 64) * iters * 16 * 65536.0;
      printf("%-34s | %d | %8.1f | %7.1f\n", promote ? "MFMA + fp32 promotion (4 FMAs)" : "MFMA accumulating",
             threads / 256, ms * 1e3, fl / (ms * 1e-3) / 1e12);
    }
  }
  CHECK(hipGetLastError());

  printf("# 4. decode-shaped launches (256 workgroups), back to back over rotating buffers: lanes per workgroup | MB | us per launch | TB/s\n");
  for (int lanes : {1024, 256}) {
    for (int mb : {0, 17, 25, 60, 117}) {
      const int64_t bytes = (int64_t)mb << 20;
      const int64_t n16 = bytes / 16 / (1024 * 256) * (1024 * 256);
      const int copies = mb ? (int)std::min<int64_t>(8, (int64_t)(big / std::max<int64_t>(bytes, 1))) : 1;
      int it = 0;
      const float ms = time_ms([&] {
        const uint4* p = (const uint4*)(src + (size_t)(it++ % copies) * (size_t)bytes);
        if (lanes == 1024) hipLaunchKernelGGL(stream_once<1024>, dim3(256), dim3(1024), 0, 0, p, n16, sink);
        else hipLaunchKernelGGL(stream_once<256>, dim3(256), dim3(256), 0, 0, p, n16, sink);
      }, 40);
      printf("%4d | %4d | %7.2f | %6.2f\n", lanes, mb, ms * 1e3, n16 * 16.0 / (ms * 1e-3) / 1e12);
    }
  }
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  printf("bench_hw done\n");
  return 0;
}
