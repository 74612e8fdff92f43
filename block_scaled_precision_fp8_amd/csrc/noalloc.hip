// fp8_linear_noalloc: fp8_linear for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Its workspace is the file-scope device array below
// instead of a caller buffer; everything else is fp8_linear's own code path
// (capi.hip: linear_checks, linear_launch), so results are identical.
//
// The array exists once per device and is held until the process ends
// (zero-initialised at load; afterwards it keeps whatever the last call on
// that device left).  fp8_linear needs nothing in its workspace to start at
// zero: every byte a call reads back was written earlier in the same call.
// Calls that overlap on one device share the array and race: serialise them
// (one stream, or events between streams).
#include <atomic>

#include "bsfp8.h"
#include "bsfp8_internal.h"

using namespace bsfp8;

// In host code `scratch` names a host-side stand-in, not device memory: the
// device address comes from hipGetSymbolAddress below, and only that
// address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[BSFP8_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
constexpr size_t kScratchBytes = BSFP8_NOALLOC_SCRATCH_BYTES;
std::atomic<void*> g_scratch[kMaxDevices];   // device address of `scratch`, per device

// The current device's copy of the array, looked up once per device (with
// that device current) and cached.
int32_t scratch_ptr(void** p) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BSFP8_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return BSFP8_ENOTSUP;
  void* q = g_scratch[dev].load(std::memory_order_acquire);
  if (q == nullptr) {
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
      return BSFP8_EHIP;
    g_scratch[dev].store(q, std::memory_order_release);
  }
  *p = q;
  return BSFP8_OK;
}

}  // namespace

extern "C" {

int32_t fp8_linear_noalloc(const void* x, int64_t ldx, const void* wq, const void* w_scale_inv,
                           const void* bias, void* y, int64_t M, int64_t N, int64_t K,
                           int32_t block_n, int32_t block_k, int32_t act_scheme,
                           int32_t scale_fmt, const void* act_scale, void* stream) {
  size_t need = 0;
  int32_t r = linear_checks(x, ldx, wq, w_scale_inv, bias, y, M, N, K, block_n, block_k,
                            act_scheme, scale_fmt, act_scale, &need);
  if (r != BSFP8_OK || M == 0) return r;
  if (need > kScratchBytes) return BSFP8_ENOSPC;   // beyond the array: use fp8_linear
  r = check_device(stream);
  if (r != BSFP8_OK) return r;
  void* ws = nullptr;
  r = scratch_ptr(&ws);
  if (r != BSFP8_OK) return r;
  return linear_launch(x, ldx, wq, w_scale_inv, bias, y, M, N, K, block_k, act_scheme,
                       scale_fmt, act_scale, ws, kScratchBytes, stream);
}

}  // extern "C"
