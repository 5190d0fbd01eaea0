// Dense payloads applied in place (FastVideo lora_patch page):
//   .diff / .diff_b  (DenseLoRAPatch.apply_to):      dst = RN_dst(RN_f32(dst + RN_f32(src * s32)))
//   .set_weight      (DenseLoRAPatch.replacement_for): dst = RN_dst(RN_f32(src * s32))
// with s32 = RN_f32(strength). The page sums in fp32 because a bf16 sum would
// quantize away a delta three orders of magnitude below the weight; the caller
// casts back once. Multiply and add stay separate operations (compiled with
// -ffp-contract=off and the pragma below).
//
// HBM-bound streaming: each thread handles 8 consecutive elements per step
// (16-byte loads/stores for bf16; two for fp32) in a grid-stride loop sized to
// a few waves per CU. The scalar tail covers n % 8.
#include "common.hpp"
#include "launch.hpp"

#pragma clang fp contract(off)

namespace lora {
namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<bf16_bits>(const bf16_bits* p, float (&v)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8]);

template <>
__device__ __forceinline__ void store8<bf16_bits>(bf16_bits* p, const float (&v)[8]) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = static_cast<uint32_t>(f32_to_bf16_rne(v[2 * i])) |
           (static_cast<uint32_t>(f32_to_bf16_rne(v[2 * i + 1])) << 16);
  *reinterpret_cast<u32x4*>(p) = w;
}

template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&v)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

__device__ __forceinline__ float to_f32(bf16_bits h) { return bf16_to_f32(h); }
__device__ __forceinline__ float to_f32(float f) { return f; }
__device__ __forceinline__ void store1(bf16_bits* p, float v) { *p = f32_to_bf16_rne(v); }
__device__ __forceinline__ void store1(float* p, float v) { *p = v; }

__device__ __forceinline__ float patch_value(float dst, float src, float s32, bool add) {
  const float prod = src * s32;  // RN_f32
  return add ? dst + prod : prod;  // RN_f32
}

template <typename TD, typename TS>
__global__ __launch_bounds__(256) void dense_patch_kernel(TD* __restrict__ dst, const TS* __restrict__ src,
                                                          int64_t n, float s32, int add, int vec) {
  const int64_t nvec = vec ? n / 8 : 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    float d[8], s[8];
    load8(src + v * 8, s);
    if (add) load8(dst + v * 8, d);
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = patch_value(add ? d[i] : 0.f, s[i], s32, add != 0);
    store8(dst + v * 8, d);
  }
  // scalar tail (all of it when the pointers are not 16-byte aligned)
  for (int64_t i = nvec * 8 + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    store1(dst + i, patch_value(add ? to_f32(dst[i]) : 0.f, to_f32(src[i]), s32, add != 0));
}

template <typename TD, typename TS>
hipError_t launch_patch_t(void* dst, const void* src, int64_t n, float s32, int add, hipStream_t s) {
  const int vec = (reinterpret_cast<uintptr_t>(dst) % 16 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0) ? 1 : 0;
  const int64_t nvec = vec ? n / 8 : n;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 256 * 8) blocks = 256 * 8;  // 8 blocks of 4 waves per CU, grid-stride beyond
  hipLaunchKernelGGL((dense_patch_kernel<TD, TS>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<TD*>(dst), static_cast<const TS*>(src), n, s32, add, vec);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_patch(void* dst, Elt dst_t, const void* src, Elt src_t, int64_t n, float s32, int mode,
                              hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int add = mode == 0 ? 1 : 0;
  if (dst_t == Elt::BF16 && src_t == Elt::BF16) return launch_patch_t<bf16_bits, bf16_bits>(dst, src, n, s32, add, s);
  if (dst_t == Elt::BF16) return launch_patch_t<bf16_bits, float>(dst, src, n, s32, add, s);
  if (src_t == Elt::BF16) return launch_patch_t<float, bf16_bits>(dst, src, n, s32, add, s);
  return launch_patch_t<float, float>(dst, src, n, s32, add, s);
}

}  // namespace lora
