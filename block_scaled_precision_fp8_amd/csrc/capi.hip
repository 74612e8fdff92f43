// C-ABI of libbsfp8.so (declared in include/bsfp8.h).
//
// Every entry point validates its arguments on the host first (no HIP call
// before that), so every error return is reachable without a GPU.  Then it
// checks, once per device, that the current device is a gfx950, checks that
// the stream belongs to the current device, and enqueues the kernels.
#include <atomic>
#include <cstring>

#include "bsfp8.h"
#include "bsfp8_internal.h"

using namespace bsfp8;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool fits_i32(int64_t v) { return v >= 0 && v <= 0x7fffffffLL; }
bool valid_fmt(int32_t f) { return f == BSFP8_SCALE_FLOAT || f == BSFP8_SCALE_UE8M0; }

// Block sizes: the pages allow any positive pair ([FG-FP8] §四); 128 x 128
// and 32 x 32 (with 1 x 32 act groups, §九) are provided, other positive
// sizes return ENOTSUP.
int32_t check_blocks(int32_t bn, int32_t bk) {
  if (bn <= 0 || bk <= 0) return BSFP8_EINVAL;
  if (!((bn == 128 && bk == 128) || (bn == 32 && bk == 32))) return BSFP8_ENOTSUP;
  return BSFP8_OK;
}

int32_t hip_status(hipError_t e) {
  if (e == hipSuccess) return BSFP8_OK;
  return e == hipErrorNotSupported ? BSFP8_ENOTSUP : BSFP8_EHIP;
}

// shared checks of the FP8 GEMM operand set
// 32-bit in-tile byte offsets of the GEMM kernels (256 rows x K)
constexpr int64_t kMaxGemmK = int64_t(1) << 22;

int32_t check_gemm(const void* xq, const void* xs, const void* wq, const void* ws,
                   const void* bias, const void* y, int64_t M, int64_t N, int64_t K,
                   int32_t bn, int32_t bk, int32_t fmt) {
  if (M < 0 || N < 0 || K < 0) return BSFP8_EINVAL;
  if (!fits_i32(M) || !fits_i32(N) || !fits_i32(K)) return BSFP8_EINVAL;
  if (K % 16 != 0 || N % 8 != 0) return BSFP8_EINVAL;
  if (K > kMaxGemmK) return BSFP8_ENOTSUP;
  if (!valid_fmt(fmt)) return BSFP8_EINVAL;
  int32_t r = check_blocks(bn, bk);
  if (r != BSFP8_OK) return r;
  if (M == 0) return BSFP8_OK;
  if (N == 0 || K == 0) return BSFP8_EINVAL;
  if (!xq || !xs || !wq || !ws || !y) return BSFP8_EINVAL;
  if (!al16(xq) || !al16(wq) || !al16(y) || (bias && !al16(bias))) return BSFP8_EINVAL;
  if (!al16(xs) || !al16(ws)) return BSFP8_EINVAL;
  return BSFP8_OK;
}


}  // namespace

namespace bsfp8 {

int32_t check_device(void* stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BSFP8_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return BSFP8_ENOTSUP;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BSFP8_EHIP;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return BSFP8_ENOTSUP;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return BSFP8_EHIP;
    if (sdev != dev) return BSFP8_ENOTSUP;
  }
  return BSFP8_OK;
}

// ---- fp8_linear: host-only argument checks, then the launches

// *need: the workspace bytes the call takes
int32_t linear_checks(const void* x, int64_t ldx, const void* wq, const void* w_scale_inv,
                      const void* bias, const void* y, int64_t M, int64_t N, int64_t K,
                      int32_t block_n, int32_t block_k, int32_t act_scheme, int32_t scale_fmt,
                      const void* act_scale, size_t* need) {
  *need = 0;
  if (act_scheme != BSFP8_ACT_DYNAMIC && act_scheme != BSFP8_ACT_STATIC) return BSFP8_EINVAL;
  // the staged activations stand in for xq / x_scale in the operand checks
  static const uint8_t dummy[16] __attribute__((aligned(16))) = {0};
  int32_t r = check_gemm(x, dummy, wq, w_scale_inv, bias, y, M, N, K, block_n, block_k,
                         scale_fmt);
  if (r != BSFP8_OK) return r;
  const bool stat = act_scheme == BSFP8_ACT_STATIC;
  if (stat && block_k != 128) return BSFP8_ENOTSUP;   // as fp8_quant_act
  if (M == 0) return BSFP8_OK;
  if (stat && (!act_scale || (scale_fmt == BSFP8_SCALE_FLOAT && ((uintptr_t)act_scale & 3u))))
    return BSFP8_EINVAL;
  if (ldx < K || ldx % 8 != 0) return BSFP8_EINVAL;
  const int blk = block_k;                  // 128, or 32 for (32, 32) blocks
  if (!fits_i32(M * ((K + blk - 1) / blk))) return BSFP8_EINVAL;
  *need = linear_workspace_bytes(M, N, K, blk);
  return BSFP8_OK;
}

// after the checks and the device check: quantization (fused into the
// decode kernel, or staged in the workspace), then the GEMM
int32_t linear_launch(const void* x, int64_t ldx, const void* wq, const void* w_scale_inv,
                      const void* bias, void* y, int64_t M, int64_t N, int64_t K, int32_t blk,
                      int32_t act_scheme, int32_t scale_fmt, const void* act_scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const bool stat = act_scheme == BSFP8_ACT_STATIC;
  hipStream_t st = (hipStream_t)stream;
  GemmArgs a{};
  a.wq = (const uint8_t*)wq; a.ws = w_scale_inv;
  a.bias = (const uint16_t*)bias; a.y = (uint16_t*)y; a.M = M; a.N = N; a.K = K;
  a.fmt = scale_fmt;
  a.blk = blk;
  if (blk == 128 && linear_fused(M, N, K)) {
    // one launch: the decode kernel quantizes the activations itself
    a.x_bf16 = (const uint16_t*)x; a.ldx = ldx;
    a.xstat = stat ? act_scale : nullptr;
    return hip_status(launch_block_gemm(a, st));
  }
  if (blk == 128 && linear_xq(M, N, K)) {
    // the large-M GEMM quantizes the activations in its K loop (xs: the
    // static scale or null); the workspace holds only the K splits' partials
    a.x_bf16 = (const uint16_t*)x; a.ldx = ldx;
    a.xs = stat ? act_scale : nullptr;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    return hip_status(launch_block_gemm(a, st));
  }
  // workspace: [xq M*K][x_scale M*G*4][gemm workspace], 256-byte aligned parts
  const int64_t G = (K + blk - 1) / blk;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  uint8_t* ws = (uint8_t*)workspace;
  uint8_t* xq = ws;
  void* xs = ws + up((size_t)M * K);
  void* gw = ws + up((size_t)M * K) + up((size_t)M * G * 4);
  hipError_t e = launch_quant_act((const uint16_t*)x, M, K, ldx, scale_fmt, xq, xs, st,
                                  stat ? act_scale : nullptr, blk);
  if (e != hipSuccess) return BSFP8_EHIP;
  a.xq = xq; a.xs = xs; a.workspace = gw;
  a.workspace_bytes = workspace_bytes - (size_t)((uint8_t*)gw - ws);
  return hip_status(launch_block_gemm(a, st));
}

}  // namespace bsfp8

extern "C" {

int32_t bsfp8_version(void) { return 100; }

const char* bsfp8_status_string(int32_t s) {
  switch (s) {
    case BSFP8_OK: return "ok";
    case BSFP8_EINVAL: return "invalid argument";
    case BSFP8_ENOTSUP: return "not supported (option, block size or device)";
    case BSFP8_ENOSPC: return "workspace too small";
    case BSFP8_EHIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

size_t bsfp8_workspace_size(int32_t op, int64_t M, int64_t N, int64_t K, int32_t E) {
  if (M < 0 || N < 0 || K < 0 || E < 0) return (size_t)-1;
  switch (op) {
    case BSFP8_OP_BLOCK_GEMM: return gemm_workspace_bytes(M, N, K);
    case BSFP8_OP_LINEAR: return linear_workspace_bytes(M, N, K);
    case BSFP8_OP_GROUPED_GEMM: return grouped_workspace_bytes(M, N, K, E);
    case BSFP8_OP_FP4_QUANT: return fp4_quant_workspace_bytes(M, K);
    case BSFP8_OP_FP4_GEMM: return fp4_gemm_workspace_bytes(M, N, K);
    case BSFP8_OP_FP8_FP4_GEMM: return fp8_fp4_workspace_bytes(M, N, K);
    case BSFP8_OP_LINEAR_B32: return linear_workspace_bytes(M, N, K, 32);
    default: return (size_t)-1;
  }
}

int32_t bsfp8_gemm_kernel(int64_t M, int64_t N, int64_t K, int32_t* splits) {
  if (M < 0 || N < 0 || K < 0) return -1;
  int s = 1;
  const int kind = gemm_kind(M, N, K, &s);
  if (splits) *splits = s;
  return kind;
}

int32_t fp8_quant_act(const void* x, int64_t M, int64_t K, int64_t ldx, int32_t group_k,
                      int32_t act_scheme, int32_t scale_fmt, void* xq, void* x_scale,
                      void* stream) {
  if (M < 0 || K < 0 || !fits_i32(M) || !fits_i32(K)) return BSFP8_EINVAL;
  if (K % 16 != 0 || ldx < K || ldx % 8 != 0) return BSFP8_EINVAL;
  if (act_scheme != BSFP8_ACT_DYNAMIC && act_scheme != BSFP8_ACT_STATIC) return BSFP8_EINVAL;
  if (!valid_fmt(scale_fmt)) return BSFP8_EINVAL;
  if (group_k <= 0) return BSFP8_EINVAL;
  if (group_k != 128 && group_k != 32) return BSFP8_ENOTSUP;
  if (act_scheme == BSFP8_ACT_STATIC && group_k != 128) return BSFP8_ENOTSUP;
  if (M == 0) return BSFP8_OK;
  if (K == 0) return BSFP8_EINVAL;
  if (!x || !xq || !x_scale) return BSFP8_EINVAL;
  if (!al16(x) || !al16(xq) || !al16(x_scale)) return BSFP8_EINVAL;
  if (!fits_i32(M * ((K + group_k - 1) / group_k))) return BSFP8_EINVAL;
  int32_t r = check_device(stream);
  if (r != BSFP8_OK) return r;
  // STATIC: the calibrated scale sits in x_scale[0] on entry; every group's
  // entry (x_scale[0] included) is set to that same value
  return hip_status(launch_quant_act((const uint16_t*)x, M, K, ldx, scale_fmt, (uint8_t*)xq,
                                     x_scale, (hipStream_t)stream,
                                     act_scheme == BSFP8_ACT_STATIC ? x_scale : nullptr,
                                     group_k));
}

int32_t fp8_dequant_weight(const void* wq, int64_t N, int64_t K, int32_t block_n,
                           int32_t block_k, int32_t scale_fmt, const void* w_scale_inv, void* w,
                           void* stream) {
  if (N < 0 || K < 0 || !fits_i32(N) || !fits_i32(K)) return BSFP8_EINVAL;
  if (K % 16 != 0) return BSFP8_EINVAL;
  if (!valid_fmt(scale_fmt)) return BSFP8_EINVAL;
  int32_t r = check_blocks(block_n, block_k);
  if (r != BSFP8_OK) return r;
  if (N == 0 || K == 0) return BSFP8_OK;
  if (!wq || !w_scale_inv || !w) return BSFP8_EINVAL;
  if (!al16(wq) || !al16(w) || ((uintptr_t)w_scale_inv & 3u)) return BSFP8_EINVAL;
  r = check_device(stream);
  if (r != BSFP8_OK) return r;
  return hip_status(launch_dequant_weight((const uint8_t*)wq, N, K, scale_fmt, w_scale_inv,
                                          (uint16_t*)w, (hipStream_t)stream, block_n));
}

int32_t fp8_scale_to_ue8m0(const float* scale, int64_t n, void* out, void* stream) {
  if (n < 0) return BSFP8_EINVAL;
  if (n == 0) return BSFP8_OK;
  if (!scale || !out || ((uintptr_t)scale & 3u)) return BSFP8_EINVAL;
  int32_t r = check_device(stream);
  if (r != BSFP8_OK) return r;
  return hip_status(launch_pow2_to_ue8m0(scale, n, (uint8_t*)out, (hipStream_t)stream));
}

int32_t mxfp4_quant_weight(const void* w, int64_t N, int64_t K, int64_t ldw, void* wq4,
                           void* w_scale, void* stream) {
  if (N < 0 || K < 0 || !fits_i32(N) || !fits_i32(K)) return BSFP8_EINVAL;
  if (K % 32 != 0 || ldw < K || ldw % 8 != 0) return BSFP8_EINVAL;
  if (N == 0 || K == 0) return BSFP8_OK;
  if (!w || !wq4 || !w_scale) return BSFP8_EINVAL;
  if (!al16(w) || !al16(wq4)) return BSFP8_EINVAL;
  int32_t r = check_device(stream);
  if (r != BSFP8_OK) return r;
  return hip_status(launch_mxfp4_quant_weight((const uint16_t*)w, N, K, ldw, (uint8_t*)wq4,
                                              (uint8_t*)w_scale, (hipStream_t)stream));
}

int32_t fp8_fp4_gemm(const void* xq, const void* x_scale, const void* wq4, const void* w_scale,
                     const void* bias, void* y, int64_t M, int64_t N, int64_t K,
                     int32_t scale_fmt, void* workspace, size_t workspace_bytes, void* stream) {
  int32_t r = check_gemm(xq, x_scale, wq4, w_scale, bias, y, M, N, K, 128, 128, scale_fmt);
  if (r != BSFP8_OK) return r;
  if (K % 32 != 0) return BSFP8_EINVAL;
  if (M == 0) return BSFP8_OK;
  const size_t need = fp8_fp4_workspace_bytes(M, N, K);
  if (workspace_bytes < need) return BSFP8_ENOSPC;
  if (need && (!workspace || !al16(workspace))) return BSFP8_EINVAL;
  if (!fits_i32(M * ((K + 127) / 128))) return BSFP8_EINVAL;
  r = check_device(stream);
  if (r != BSFP8_OK) return r;
  GemmArgs a{};
  a.xq = (const uint8_t*)xq; a.xs = x_scale; a.wq = (const uint8_t*)wq4; a.ws = w_scale;
  a.bias = (const uint16_t*)bias; a.y = (uint16_t*)y; a.M = M; a.N = N; a.K = K;
  a.fmt = scale_fmt; a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.w4 = true;
  return hip_status(launch_block_gemm(a, (hipStream_t)stream));
}

int32_t fp8_quant_weight(const void* w, int64_t N, int64_t K, int64_t ldw, int32_t block_n,
                         int32_t block_k, int32_t scale_fmt, void* wq, void* w_scale_inv,
                         void* stream) {
  if (N < 0 || K < 0 || !fits_i32(N) || !fits_i32(K)) return BSFP8_EINVAL;
  if (K % 16 != 0 || ldw < K || ldw % 8 != 0) return BSFP8_EINVAL;
  if (!valid_fmt(scale_fmt)) return BSFP8_EINVAL;
  int32_t r = check_blocks(block_n, block_k);
  if (r != BSFP8_OK) return r;
  if (N == 0) return BSFP8_OK;
  if (K == 0) return BSFP8_EINVAL;
  if (!w || !wq || !w_scale_inv) return BSFP8_EINVAL;
  if (!al16(w) || !al16(wq) || !al16(w_scale_inv)) return BSFP8_EINVAL;
  if ((N + 127) / 128 > 65535) return BSFP8_EINVAL;
  r = check_device(stream);
  if (r != BSFP8_OK) return r;
  return hip_status(launch_quant_weight((const uint16_t*)w, N, K, ldw, scale_fmt, (uint8_t*)wq,
                                        w_scale_inv, (hipStream_t)stream, block_n));
}

int32_t fp8_block_gemm(const void* xq, const void* x_scale, const void* wq,
                       const void* w_scale_inv, const void* bias, void* y, int64_t M, int64_t N,
                       int64_t K, int32_t block_n, int32_t block_k, int32_t scale_fmt,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int32_t r = check_gemm(xq, x_scale, wq, w_scale_inv, bias, y, M, N, K, block_n, block_k,
                         scale_fmt);
  if (r != BSFP8_OK || M == 0) return r;
  // (32, 32) blocks run without workspace
  const size_t need = block_n == 32 ? 0 : gemm_workspace_bytes(M, N, K);
  if (workspace_bytes < need) return BSFP8_ENOSPC;
  if (need && (!workspace || !al16(workspace))) return BSFP8_EINVAL;
  if (block_n == 32 && !fits_i32((M + 127) / 128 * ((N + 127) / 128) + 8)) return BSFP8_EINVAL;
  r = check_device(stream);
  if (r != BSFP8_OK) return r;
  GemmArgs a{};
  a.xq = (const uint8_t*)xq; a.xs = x_scale; a.wq = (const uint8_t*)wq; a.ws = w_scale_inv;
  a.bias = (const uint16_t*)bias; a.y = (uint16_t*)y; a.M = M; a.N = N; a.K = K;
  a.fmt = scale_fmt; a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.blk = block_n;
  return hip_status(launch_block_gemm(a, (hipStream_t)stream));
}

int32_t fp8_linear(const void* x, int64_t ldx, const void* wq, const void* w_scale_inv,
                   const void* bias, void* y, int64_t M, int64_t N, int64_t K, int32_t block_n,
                   int32_t block_k, int32_t act_scheme, int32_t scale_fmt,
                   const void* act_scale, void* workspace, size_t workspace_bytes,
                   void* stream) {
  size_t need = 0;
  int32_t r = linear_checks(x, ldx, wq, w_scale_inv, bias, y, M, N, K, block_n, block_k,
                            act_scheme, scale_fmt, act_scale, &need);
  if (r != BSFP8_OK || M == 0) return r;
  if (workspace_bytes < need) return BSFP8_ENOSPC;
  if (need && (!workspace || !al16(workspace))) return BSFP8_EINVAL;
  r = check_device(stream);
  if (r != BSFP8_OK) return r;
  return linear_launch(x, ldx, wq, w_scale_inv, bias, y, M, N, K, block_k, act_scheme,
                       scale_fmt, act_scale, workspace, workspace_bytes, stream);
}

int32_t fp8_grouped_gemm(const void* xq, const void* x_scale, const void* wq,
                         const void* w_scale_inv, const int32_t* seg_offsets, int32_t E, void* y,
                         int64_t T, int64_t N, int64_t K, int32_t block_n, int32_t block_k,
                         int32_t scale_fmt, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (E < 1 || E > 1024) return BSFP8_EINVAL;
  int32_t r = check_gemm(xq, x_scale, wq, w_scale_inv, nullptr, y, T, N, K, block_n, block_k,
                         scale_fmt);
  if (r != BSFP8_OK) return r;
  if (T == 0) return BSFP8_OK;
  if (!seg_offsets || ((uintptr_t)seg_offsets & 3u)) return BSFP8_EINVAL;
  const size_t need = grouped_workspace_bytes(T, N, K, E);
  if (workspace_bytes < need) return BSFP8_ENOSPC;
  if (need && (!workspace || !al16(workspace))) return BSFP8_EINVAL;
  const int64_t NT = block_n == 32 ? (N + 127) / 128 : (N + 255) / 256;
  if (!fits_i32(((T + 127) / 128 + E) * NT)) return BSFP8_EINVAL;
  if (!fits_i32(T * ((K + block_k - 1) / block_k))) return BSFP8_EINVAL;
  r = check_device(stream);
  if (r != BSFP8_OK) return r;
  GemmArgs a{};
  a.xq = (const uint8_t*)xq; a.xs = x_scale; a.wq = (const uint8_t*)wq; a.ws = w_scale_inv;
  a.bias = nullptr; a.y = (uint16_t*)y; a.M = T; a.N = N; a.K = K; a.fmt = scale_fmt;
  a.seg = seg_offsets; a.E = E; a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.blk = block_n;
  return hip_status(launch_grouped_gemm(a, (hipStream_t)stream));
}

int32_t fp8_fp4_grouped_gemm(const void* xq, const void* x_scale, const void* wq4,
                             const void* w_scale, const int32_t* seg_offsets, int32_t E, void* y,
                             int64_t T, int64_t N, int64_t K, int32_t scale_fmt, void* stream) {
  if (E < 1 || E > 1024) return BSFP8_EINVAL;
  int32_t r = check_gemm(xq, x_scale, wq4, w_scale, nullptr, y, T, N, K, 128, 128, scale_fmt);
  if (r != BSFP8_OK) return r;
  if (K % 32 != 0) return BSFP8_EINVAL;
  if (T == 0) return BSFP8_OK;
  if (!seg_offsets || ((uintptr_t)seg_offsets & 3u)) return BSFP8_EINVAL;
  const int64_t NT = (N + 255) / 256;
  if (!fits_i32(((T + 127) / 128 + E) * NT)) return BSFP8_EINVAL;
  if (!fits_i32(T * ((K + 127) / 128))) return BSFP8_EINVAL;
  r = check_device(stream);
  if (r != BSFP8_OK) return r;
  GemmArgs a{};
  a.xq = (const uint8_t*)xq; a.xs = x_scale; a.wq = (const uint8_t*)wq4; a.ws = w_scale;
  a.bias = nullptr; a.y = (uint16_t*)y; a.M = T; a.N = N; a.K = K; a.fmt = scale_fmt;
  a.seg = seg_offsets; a.E = E; a.w4 = true;
  return hip_status(launch_grouped_gemm(a, (hipStream_t)stream));
}

int32_t fp8_grouped_gemm_silu_mul_quant(const void* xq, const void* x_scale, const void* wq,
                                        const void* w_scale_inv, const int32_t* seg_offsets,
                                        int32_t E, void* hq, void* h_scale, void* h_bf16,
                                        int64_t T, int64_t I, int64_t K, int32_t scale_fmt,
                                        void* stream) {
  if (E < 1 || E > 1024) return BSFP8_EINVAL;
  if (I <= 0 || I % 128 != 0 || !fits_i32(2 * I)) return BSFP8_EINVAL;
  int32_t r = check_gemm(xq, x_scale, wq, w_scale_inv, nullptr, hq, T, 2 * I, K, 128, 128,
                         scale_fmt);
  if (r != BSFP8_OK) return r;
  if (T == 0) return BSFP8_OK;
  if (!seg_offsets || ((uintptr_t)seg_offsets & 3u)) return BSFP8_EINVAL;
  if (!h_scale || ((uintptr_t)h_scale & 3u)) return BSFP8_EINVAL;
  if (h_bf16 && !al16(h_bf16)) return BSFP8_EINVAL;
  if (!fits_i32(((T + 127) / 128 + E) * (I / 128))) return BSFP8_EINVAL;
  // a gate/up tile addresses rows of both halves of one expert's weight
  // through one buffer resource with 32-bit byte offsets
  if (2 * I * K > 0x7fffffffLL) return BSFP8_ENOTSUP;
  r = check_device(stream);
  if (r != BSFP8_OK) return r;
  GemmArgs a{};
  a.xq = (const uint8_t*)xq; a.xs = x_scale; a.wq = (const uint8_t*)wq; a.ws = w_scale_inv;
  a.bias = nullptr; a.y = (uint16_t*)h_bf16; a.M = T; a.N = 2 * I; a.K = K; a.fmt = scale_fmt;
  a.seg = seg_offsets; a.E = E;
  a.hq = (uint8_t*)hq; a.hs = h_scale;
  return hip_status(launch_grouped_silu_mul_quant(a, (hipStream_t)stream));
}

int32_t fp4_quant(const void* x, int64_t R, int64_t K, int32_t dynamic_tscale, void* q4,
                  void* gscale, float* tscale, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (R < 0 || K < 0 || !fits_i32(R) || !fits_i32(K)) return BSFP8_EINVAL;
  if (K % 32 != 0) return BSFP8_EINVAL;
  if (dynamic_tscale != 0 && dynamic_tscale != 1) return BSFP8_EINVAL;
  if (R == 0) return BSFP8_OK;
  if (K == 0) return BSFP8_EINVAL;
  if (!x || !q4 || !gscale || !tscale) return BSFP8_EINVAL;
  if (!al16(x) || !al16(q4) || !al16(gscale) || ((uintptr_t)tscale & 3u)) return BSFP8_EINVAL;
  const size_t need = fp4_quant_workspace_bytes(R, K);
  if (workspace_bytes < need) return BSFP8_ENOSPC;
  if (need && (!workspace || !al16(workspace))) return BSFP8_EINVAL;
  int32_t r = check_device(stream);
  if (r != BSFP8_OK) return r;
  return hip_status(launch_fp4_quant((const uint16_t*)x, R, K, dynamic_tscale, (uint8_t*)q4,
                                     (uint8_t*)gscale, tscale, workspace, (hipStream_t)stream));
}

int32_t fp4_group_gemm(const void* xq4, const void* x_gscale, const float* x_tscale,
                       const void* wq4, const void* w_gscale, const float* w_tscale, void* y,
                       int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (M < 0 || N < 0 || K < 0 || !fits_i32(M) || !fits_i32(N) || !fits_i32(K))
    return BSFP8_EINVAL;
  if (K % 32 != 0 || N % 8 != 0) return BSFP8_EINVAL;
  // the kernels address a tile's rows (up to 256 of K/2 bytes) with 32-bit
  // offsets from one base: the same K bound as the FP8 GEMMs
  if (K > kMaxGemmK) return BSFP8_ENOTSUP;
  if (M == 0) return BSFP8_OK;
  if (N == 0 || K == 0) return BSFP8_EINVAL;
  if (!xq4 || !x_gscale || !x_tscale || !wq4 || !w_gscale || !w_tscale || !y)
    return BSFP8_EINVAL;
  if (!al16(xq4) || !al16(x_gscale) || !al16(wq4) || !al16(w_gscale) || !al16(y))
    return BSFP8_EINVAL;
  if (((uintptr_t)x_tscale & 3u) || ((uintptr_t)w_tscale & 3u)) return BSFP8_EINVAL;
  const size_t need = fp4_gemm_workspace_bytes(M, N, K);
  if (workspace_bytes < need) return BSFP8_ENOSPC;
  if (need && (!workspace || !al16(workspace))) return BSFP8_EINVAL;
  int32_t r = check_device(stream);
  if (r != BSFP8_OK) return r;
  return hip_status(launch_fp4_gemm((const uint8_t*)xq4, (const uint8_t*)x_gscale, x_tscale,
                                    (const uint8_t*)wq4, (const uint8_t*)w_gscale, w_tscale,
                                    (uint16_t*)y, M, N, K, workspace, workspace_bytes,
                                    (hipStream_t)stream));
}

}  // extern "C"
