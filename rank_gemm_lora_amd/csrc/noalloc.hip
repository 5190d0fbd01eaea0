// lora_linear_fwd without a workspace argument, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). The call runs exactly lora_linear_fwd's
// kernels; the scratch they need (the rank-wide intermediate, K-split partial
// sums, the few-token path's partial sums) lives in one file-scope device array
// that every GPU holds, at its own address, until the process ends.
//
// The array's name in host code is only a host-side stand-in: its device address
// is looked up once per device with hipGetSymbolAddress (that device current) and
// kept per device; only that address is ever passed to a kernel.
#include <hip/hip_runtime.h>

#include <atomic>

#include "lora_mi355x.h"

namespace {

__device__ __align__(256) char scratch[LORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // device address of `scratch` per device (null until looked up)

// The device address of this device's copy of `scratch` (looked up on its first use).
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LORA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LORA_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return LORA_ERR_HIP;
    g_scratch[dev].store(p, std::memory_order_release);  // (a concurrent first call stores the same value)
  }
  *out = p;
  return LORA_OK;
}

}  // namespace

extern "C" int lora_linear_fwd_noalloc(const void* x, int64_t T, int64_t K, int64_t ldx, const void* W, int64_t N,
                                       const void* bias, const void* A, const void* B, int32_t rank,
                                       int32_t adapter_dtype, double alpha, double strength, double request_scale,
                                       void* y, int64_t ldy, int32_t act_dtype, int32_t quality, void* stream) {
  const int32_t r = rank;
  const size_t need =
      lora_linear_workspace_size(T, K, N, &r, (A != nullptr || B != nullptr) ? 1 : 0, adapter_dtype, quality);
  if (need > static_cast<size_t>(LORA_NOALLOC_SCRATCH_BYTES)) return LORA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (T > 0) {
    const int st = scratch_address(&ws);
    if (st != LORA_OK) return st;
  }
  return lora_linear_fwd(x, T, K, ldx, W, N, bias, A, B, rank, adapter_dtype, alpha, strength, request_scale, y, ldy,
                         act_dtype, quality, ws, ws != nullptr ? static_cast<size_t>(LORA_NOALLOC_SCRATCH_BYTES) : 0,
                         stream);
}
