// Internal interface of the backward kernels (backward.hip) for the C-ABI host code.
#pragma once

#include "launch.hpp"

namespace lora {

// dst[c][r] = src[r][c] (r < R, c < C), zero elsewhere in dst [Cpad, Rpad] (row stride Rpad).
hipError_t transpose_pad(const uint16_t* src, int64_t ld, int64_t R, int64_t C, uint16_t* dst, int64_t Rpad,
                         int64_t Cpad, hipStream_t s);

// Token chunks of a contraction over T tokens with `tiles` workgroups per chunk.
void tn_plan(int64_t T, int64_t tiles, int* S, int64_t* tchunk);
// fp32 partial sums of one contraction: P [T, M] against Q [T, J] (+ a column of ones).
size_t tn_partial_bytes(int64_t T, int64_t M, int J, bool ones);

// Token padding of the transposed rank-wide operand Qt [J, tpad] (zeros past T).
inline int64_t tn_tpad(int64_t T) { return (T + 63) / 64 * 64; }

// out = P^T Q summed over tokens (token chunks added in order), Q given as Qt [J, tpad].
// transpose: out[j][i] (row stride ldo), else out[i][j]; columns j >= jvalid are not
// written. ones: also the column sums of P into col_out[i] (when col_out is not null).
hipError_t tn_contract(const uint16_t* P, int64_t ldp, int64_t M, const uint16_t* Qt, int64_t tpad, int J, int64_t T,
                       bool ones, float* part, float* out, int64_t ldo, int jvalid, bool transpose, float* col_out,
                       hipStream_t s);

}  // namespace lora
