// Device probe: the sustained rate of the matrix cores and the shader clock under
// that load. Two waves per SIMD each issue back-to-back v_mfma_f32_16x16x32_bf16
// on eight independent accumulators (no memory traffic in the loop), so the
// matrix pipe of each SIMD is never starved; lane 0 of each workgroup records the shader
// cycles (s_memtime) and the 100 MHz real-time ticks (s_memrealtime) the loop
// took. The rate this reaches is the ceiling a GEMM on the same device and
// clock can approach, and cycles over real time is the clock it ran at.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "lora_mi355x.h"

namespace lora {
namespace {

__global__ __launch_bounds__(512) void mfma_probe_kernel(int64_t iters, float* __restrict__ sink,
                                                         uint64_t* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  // operands that differ per lane and per wave (values in [1, 2): no denormals, no overflow)
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1.0f + 0.0078125f * static_cast<float>((lane * 8 + e) & 127));
    b[e] = static_cast<__bf16>(1.0f + 0.00390625f * static_cast<float>((threadIdx.x + 3 * e) & 255));
  }
  // eight independent accumulators, each MFMA in place: the loop is written as asm so that the
  // register allocator cannot merge or rotate the chains (which serializes them on their latency)
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{static_cast<float>(j), 0.f, 0.f, 0.f};
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u)  // 64 MFMAs per trip: the loop's own instructions are noise
#pragma unroll
      for (int j = 0; j < 8; ++j)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[j]) : "v"(a), "v"(b));
  }
  // (the compiler does not know the asm wrote the accumulators with an MFMA: wait out its latency
  // before they are read)
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;  // keeps the loop
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace
}  // namespace lora

extern "C" int lora_mfma_probe(int64_t iters, int32_t blocks, float* sink, uint64_t* clocks, void* stream) {
  if (iters < 1 || blocks < 1) return LORA_ERR_SHAPE;
  if (sink == nullptr || clocks == nullptr) return LORA_ERR_NULL_PTR;
  if (reinterpret_cast<uintptr_t>(sink) % 4 != 0 || reinterpret_cast<uintptr_t>(clocks) % 8 != 0)
    return LORA_ERR_ALIGN;
  hipLaunchKernelGGL(lora::mfma_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(512), 0,
                     static_cast<hipStream_t>(stream), iters, sink, clocks);
  return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}
