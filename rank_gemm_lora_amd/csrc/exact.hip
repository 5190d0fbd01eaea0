// Exact tier: the separate-pass chain, reproduced bit for bit.
//
// SGLang PR #43501, Modifications (quality="exact"): the chain of the dynamic
// LoRA path -- base GEMM with bias, x.A^T, then .B^T, one multiply pass per
// scale (alpha/rank, strength, request scale), then the add -- is kept as is,
// except that multiplications by a unit scale are skipped (x * 1.0 is exact).
// The GEMMs of that chain are defined here as: products summed in fp64 with k
// ascending from +0.0 (each product of bf16/fp32 values is exact in fp64), then
// one rounding to fp32. Every other step is an fp32 operation followed by a
// rounding to the tensor's dtype. This file is compiled with -ffp-contract=off;
// nothing below may be fused into an FMA except the exact-product fp64 sums.
//
// Kernels
//   exact_t_kernel      t[m, t_col + q] = RN_adt(G(x, A_g))        per group
//   exact_out_kernel    base, d, scale passes and the add, per output element
// Both are LDS-tiled fp64 dot products: 64 x 64 outputs per 256-thread block,
// 4 x 4 per thread, k staged 16 at a time.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

#pragma clang fp contract(off)

namespace lora {
namespace {

constexpr int TM = 64, TN = 64, KC = 16;

// Element loaders: value of row `row`, column k of a row-major operand, widened
// exactly to double (0 outside the valid range).
struct LoadBf16 {
  const bf16_bits* p; int64_t ld; int64_t rows; int64_t cols;
  __device__ double operator()(int64_t row, int64_t k) const {
    return (row < rows && k < cols) ? static_cast<double>(bf16_to_f32(p[row * ld + k])) : 0.0;
  }
};
struct LoadF32 {
  const float* p; int64_t ld; int64_t rows; int64_t cols;
  __device__ double operator()(int64_t row, int64_t k) const {
    return (row < rows && k < cols) ? static_cast<double>(p[row * ld + k]) : 0.0;
  }
};
// Rows [lo, lo + inner.rows) of an operand addressed by an outer row index
// (the LoRA B of a group, indexed by output column).
template <class Inner>
struct RowShift {
  Inner inner; int64_t lo;
  __device__ double operator()(int64_t row, int64_t k) const {
    return row >= lo ? inner(row - lo, k) : 0.0;
  }
};
// 4-bit weight element: RN_bf16( RN_f32( codebook[code] * absmax[block] ) ).
struct LoadNf4 {
  const uint8_t* codes; const float* absmax; const float* codebook; int64_t rows; int64_t K;
  __device__ double operator()(int64_t row, int64_t k) const {
    if (row >= rows || k >= K) return 0.0;
    const uint8_t byte = codes[row * (K / 2) + k / 2];
    const int code = (k & 1) ? (byte >> 4) : (byte & 0xf);
    const float prod = codebook[code] * absmax[(row * K + k) / 64];
    return static_cast<double>(bf16_to_f32(f32_to_bf16_rne(prod)));
  }
};

// acc[i][j] = sum over k in [0, K) ascending of P(m0 + ty + 16 i, k) * Q(n0 + tx + 16 j, k),
// starting from +0.0 and rounding once per add (fp64).
template <class LP, class LQ>
__device__ __forceinline__ void dot_tile(double (&acc)[4][4], const LP& P, const LQ& Q, int64_t m0, int64_t n0,
                                         int64_t K, double (*ps)[TM + 1], double (*qs)[TN + 1]) {
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  for (int64_t k0 = 0; k0 < K; k0 += KC) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int e = it * 256 + threadIdx.x;
      const int row = e / KC, kk = e % KC;
      ps[kk][row] = P(m0 + row, k0 + kk);
      qs[kk][row] = Q(n0 + row, k0 + kk);
    }
    __syncthreads();
    const int kn = static_cast<int>(min<int64_t>(KC, K - k0));
    for (int kk = 0; kk < kn; ++kk) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = ps[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = qs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = acc[i][j] + a[i] * b[j];
    }
  }
}

__device__ __forceinline__ float rn_dt(float v, bool bf16) {
  return bf16 ? bf16_to_f32(f32_to_bf16_rne(v)) : v;
}

// ----------------------------------------------------------------- t = RN_adt(G(x, A_g))
template <typename TX, typename TL>
__global__ __launch_bounds__(256) void exact_t_kernel(LinearProblem p) {
  __shared__ double ps[KC][TM + 1];
  __shared__ double qs[KC][TN + 1];
  const GroupDev& g = p.g[blockIdx.z];
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * TM, q0 = static_cast<int64_t>(blockIdx.y) * TN;
  if (q0 >= g.rank) return;  // uniform over the block
  typedef typename std::conditional<sizeof(TX) == 2, LoadBf16, LoadF32>::type LX;
  typedef typename std::conditional<sizeof(TL) == 2, LoadBf16, LoadF32>::type LA;
  const LX P{static_cast<const TX*>(p.x), p.ldx, p.T, p.K};
  const LA Q{static_cast<const TL*>(g.A), p.K, g.rank, p.K};
  double acc[4][4];
  dot_tile(acc, P, Q, m0, q0, p.K, ps, qs);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  TL* t = static_cast<TL*>(p.work);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty + 16 * i;
    if (m >= p.T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t q = q0 + tx + 16 * j;
      if (q >= g.rank) continue;
      const float v = static_cast<float>(acc[i][j]);  // RN_f32
      if constexpr (sizeof(TL) == 2) t[m * p.ldt + g.t_col + q] = f32_to_bf16_rne(v);
      else t[m * p.ldt + g.t_col + q] = v;
    }
  }
}

// ----------------------------------------------------------------- y
template <typename TA, typename TL, bool NF4>
__global__ __launch_bounds__(256) void exact_out_kernel(LinearProblem p) {
  __shared__ double ps[KC][TM + 1];
  __shared__ double qs[KC][TN + 1];
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * TM, n0 = static_cast<int64_t>(blockIdx.y) * TN;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  constexpr bool act_bf16 = sizeof(TA) == 2, ad_bf16 = sizeof(TL) == 2;
  typedef typename std::conditional<act_bf16, LoadBf16, LoadF32>::type LX;
  typedef typename std::conditional<ad_bf16, LoadBf16, LoadF32>::type LT;
  const LX X{static_cast<const TA*>(p.x), p.ldx, p.T, p.K};

  double acc[4][4];
  if constexpr (NF4) {
    const LoadNf4 Wl{p.codes, p.absmax, p.codebook, p.N, p.K};
    dot_tile(acc, X, Wl, m0, n0, p.K, ps, qs);
  } else {
    const LX Wl{static_cast<const TA*>(p.W), p.K, p.N, p.K};
    dot_tile(acc, X, Wl, m0, n0, p.K, ps, qs);
  }

  // E2: base = RN_dt( RN_f32( G + b ) )
  const TA* bias = static_cast<const TA*>(p.bias);
  float out[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + tx + 16 * j;
    float bv = 0.f;
    const bool has_b = bias != nullptr && n < p.N;
    if (has_b) bv = act_bf16 ? bf16_to_f32(reinterpret_cast<const bf16_bits*>(bias)[n])
                             : reinterpret_cast<const float*>(bias)[n];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gv = static_cast<float>(acc[i][j]);
      out[i][j] = rn_dt(has_b ? gv + bv : gv, act_bf16);
    }
  }

  // E3-E5 per group whose columns meet this tile
  for (int gi = 0; gi < p.n_groups; ++gi) {
    const GroupDev& g = p.g[gi];
    if (g.col_off >= n0 + TN || g.col_off + g.n_cols <= n0) continue;
    const LT T{static_cast<const TL*>(p.work) + g.t_col, p.ldt, p.T, g.rank};
    // B rows indexed by output column: row n of this operand is B_g[n - col_off].
    const RowShift<LT> Bq{LT{static_cast<const TL*>(g.B), g.rank, g.n_cols, g.rank}, g.col_off};
    double dacc[4][4];
    dot_tile(dacc, T, Bq, m0, n0, g.rank, ps, qs);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx + 16 * j;
      if (n < g.col_off || n >= g.col_off + g.n_cols) continue;
      float cb = 0.f;
      if (g.Bb != nullptr)
        cb = ad_bf16 ? bf16_to_f32(static_cast<const bf16_bits*>(g.Bb)[n - g.col_off])
                     : static_cast<const float*>(g.Bb)[n - g.col_off];
      // the legacy lora_B bias: its own passes over strength and request scale (not alpha / rank),
      // added after the adapter's delta
      float e = cb;
#pragma unroll
      for (int f = 1; f < 3; ++f) {
        if (g.f[f] != 1.0f) e = rn_dt(e * g.f[f], ad_bf16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float d = rn_dt(static_cast<float>(dacc[i][j]), ad_bf16);     // E3
#pragma unroll
        for (int f = 0; f < 3; ++f) {                                 // E4
          if (g.f[f] != 1.0f) d = rn_dt(d * g.f[f], ad_bf16);
        }
        out[i][j] = rn_dt(out[i][j] + d, act_bf16);                   // E5
        if (g.Bb != nullptr) out[i][j] = rn_dt(out[i][j] + e, act_bf16);
      }
    }
  }

  TA* y = static_cast<TA*>(p.y);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty + 16 * i;
    if (m >= p.T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx + 16 * j;
      if (n >= p.N) continue;
      if constexpr (act_bf16) y[m * p.ldy + n] = f32_to_bf16_rne(out[i][j]);
      else y[m * p.ldy + n] = out[i][j];
    }
  }
}

template <typename TA, typename TL, bool NF4>
hipError_t launch_exact_t(const LinearProblem& p, hipStream_t s) {
  if (p.n_groups > 0) {
    int max_rank = 0;
    for (int i = 0; i < p.n_groups; ++i) max_rank = max_rank > p.g[i].rank ? max_rank : p.g[i].rank;
    const dim3 grid(static_cast<unsigned>((p.T + TM - 1) / TM), static_cast<unsigned>((max_rank + TN - 1) / TN),
                    static_cast<unsigned>(p.n_groups));
    hipLaunchKernelGGL((exact_t_kernel<TA, TL>), grid, dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(static_cast<unsigned>((p.T + TM - 1) / TM), static_cast<unsigned>((p.N + TN - 1) / TN));
  hipLaunchKernelGGL((exact_out_kernel<TA, TL, NF4>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// Exact merge: W[n,k] <- RN_w(RN_f32(W + d)), d = RN_f32(G . s) (no multiply when s == 1),
// G = RN_f32(sum over q ascending of B[n,q] . A[q,k] in fp64 from +0.0). One thread per element.
template <typename TW, typename TL>
__global__ __launch_bounds__(256) void exact_merge_kernel(TW* W, int64_t N, int64_t K, const TL* A, const TL* B,
                                                          int rank, float s32) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= N * K) return;
  const int64_t n = i / K, k = i - n * K;
  auto ld = [](const auto& v) -> float {
    if constexpr (sizeof(v) == 2) return bf16_to_f32(v);
    else return v;
  };
  double acc = 0.0;
  for (int q = 0; q < rank; ++q)
    acc = acc + static_cast<double>(ld(B[n * rank + q])) * static_cast<double>(ld(A[static_cast<int64_t>(q) * K + k]));
  const float g = static_cast<float>(acc);
  const float d = s32 == 1.0f ? g : g * s32;
  const float v = ld(W[i]) + d;
  if constexpr (sizeof(TW) == 2) W[i] = f32_to_bf16_rne(v);
  else W[i] = v;
}

}  // namespace

hipError_t launch_exact_merge(void* W, Elt wdt, int64_t N, int64_t K, const void* A, const void* B, int rank,
                              Elt adt, float s32, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((N * K + 255) / 256));
  if (wdt == Elt::BF16 && adt == Elt::BF16)
    hipLaunchKernelGGL((exact_merge_kernel<bf16_bits, bf16_bits>), grid, dim3(256), 0, st, static_cast<bf16_bits*>(W),
                       N, K, static_cast<const bf16_bits*>(A), static_cast<const bf16_bits*>(B), rank, s32);
  else if (wdt == Elt::BF16)
    hipLaunchKernelGGL((exact_merge_kernel<bf16_bits, float>), grid, dim3(256), 0, st, static_cast<bf16_bits*>(W),
                       N, K, static_cast<const float*>(A), static_cast<const float*>(B), rank, s32);
  else if (adt == Elt::BF16)
    hipLaunchKernelGGL((exact_merge_kernel<float, bf16_bits>), grid, dim3(256), 0, st, static_cast<float*>(W),
                       N, K, static_cast<const bf16_bits*>(A), static_cast<const bf16_bits*>(B), rank, s32);
  else
    hipLaunchKernelGGL((exact_merge_kernel<float, float>), grid, dim3(256), 0, st, static_cast<float*>(W),
                       N, K, static_cast<const float*>(A), static_cast<const float*>(B), rank, s32);
  return hipGetLastError();
}

hipError_t launch_exact(const LinearProblem& p, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const bool act_bf16 = p.act == Elt::BF16, ad_bf16 = p.adapter == Elt::BF16;
  if (p.nf4) return ad_bf16 ? launch_exact_t<bf16_bits, bf16_bits, true>(p, s)
                            : launch_exact_t<bf16_bits, float, true>(p, s);
  if (act_bf16 && ad_bf16) return launch_exact_t<bf16_bits, bf16_bits, false>(p, s);
  if (act_bf16) return launch_exact_t<bf16_bits, float, false>(p, s);
  return launch_exact_t<float, float, false>(p, s);
}

}  // namespace lora
