// Internal interface of the backward kernels (backward.hip) for the C-ABI host code.
#pragma once

#include "launch.hpp"

namespace lora {

// dst[c][r] = src[r][c] (r < R, c < C), zero elsewhere in dst [Cpad, Rpad] (row stride Rpad).
hipError_t transpose_pad(const uint16_t* src, int64_t ld, int64_t R, int64_t C, uint16_t* dst, int64_t Rpad,
                         int64_t Cpad, hipStream_t s);

// dst[0 .. n) = 0.0f by a kernel (a memset node in a captured HIP graph is avoided).
hipError_t zero_fill(float* dst, int64_t n, hipStream_t s);

// Token contractions (tn_kernel): kTnI rows of P per workgroup, kTnJ columns of Q per slice,
// kTnT tokens per step.
constexpr int kTnI = 256, kTnJ = 64, kTnT = 64;

// Token chunks of a contraction over T tokens with `tiles` workgroups per chunk.
inline void tn_plan(int64_t T, int64_t tiles, int* S, int64_t* tchunk) {
  if (T <= 0 || tiles <= 0) {  // nothing to contract
    *S = 1;
    *tchunk = kTnT;
    return;
  }
  int64_t s = 512 / tiles;
  const int64_t smax = (T + 255) / 256;
  s = s < 1 ? 1 : (s > smax ? smax : s);
  s = s > 64 ? 64 : s;
  int64_t c = (T + s - 1) / s;
  c = (c + kTnT - 1) / kTnT * kTnT;
  *tchunk = c;
  *S = static_cast<int>((T + c - 1) / c);
}

// fp32 partial sums of one contraction: P [T, M] against Q [T, J] (+ a column of ones).
inline size_t tn_partial_bytes(int64_t T, int64_t M, int J, bool ones) {
  const int jslices = (J + kTnJ - 1) / kTnJ;
  const int Jt = J + (ones ? 16 : 0);
  int S;
  int64_t c;
  tn_plan(T, ((M + kTnI - 1) / kTnI) * jslices, &S, &c);
  return static_cast<size_t>(S) * static_cast<size_t>(M) * static_cast<size_t>(Jt) * 4;
}

// Token padding of the transposed rank-wide operand Qt [J, tpad] (zeros past T).
inline int64_t tn_tpad(int64_t T) { return (T + 63) / 64 * 64; }

// out = P^T Q summed over tokens (token chunks added in order), Q given as Qt [J, tpad].
// transpose: out[j][i] (row stride ldo), else out[i][j]; columns j >= jvalid are not
// written. ones: also the column sums of P into col_out[i] (when col_out is not null).
hipError_t tn_contract(const uint16_t* P, int64_t ldp, int64_t M, const uint16_t* Qt, int64_t tpad, int J, int64_t T,
                       bool ones, float* part, float* out, int64_t ldo, int jvalid, bool transpose, float* col_out,
                       hipStream_t s);

}  // namespace lora
