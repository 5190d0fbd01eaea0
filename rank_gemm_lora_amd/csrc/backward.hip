// Backward of the LoRA linear, lossless tier, bf16 (Unsloth fast-LoRA chapter,
// sections 2 and 4: the gradients have a closed form, computed directly, the
// frozen base weight needed only for dX):
//
//   u~ = RN_bf16(s . dy.B)                   rank-wide producer over dy and B^T
//   dx = RN_bf16(dy.W + u~.A)                the fused forward GEMM over W^T and A^T
//   t~ = RN_bf16(s . x.A^T)                  the forward's rank-wide producer
//   dA = u~^T . x,  dB = dy^T . t~,  db = sum_t dy      token contractions (fp32)
//
// The first two reuse the forward kernels unchanged: with W^T [K, N], B^T
// [r_pad, N] and A^T [K, r_pad] (transposed copies in the workspace, ranks
// zero-padded to a multiple of 64) dx is the forward layer of the input dy.
// The token contractions (both operands token-major) run on
// v_mfma_f32_16x16x32_bf16 after each 64-token slice of both operands is staged
// transposed in LDS; token chunks write fp32 partial sums that a second kernel
// adds in chunk order. db is the contraction with a column of ones.
#include "backward.hpp"

#include "common.hpp"

namespace lora {
namespace {

// ---------------------------------------------------------------------------
// dst[c][r] = src[r][c] for r < R, c < C, zero elsewhere in dst [Cpad, Rpad] (row stride Rpad).
// 64 x 64 tiles through LDS: coalesced reads of src rows and writes of dst rows.
__global__ __launch_bounds__(256) void transpose_pad_kernel(const bf16_bits* __restrict__ src, int64_t lds_,
                                                            int64_t R, int64_t C, bf16_bits* __restrict__ dst,
                                                            int64_t Rpad, int64_t Cpad) {
  __shared__ bf16_bits tile[64][66];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 64, c0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? src[r * lds_ + c] : static_cast<bf16_bits>(0);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < Cpad && r < Rpad) dst[c * Rpad + r] = tile[tx][i];
  }
}

// The same transpose with 16-byte accesses: a thread reads one 8-element piece of a source row
// (8 threads per 64-element tile row, 32 rows per pass) and writes one 8-element piece of a
// destination row, gathered from 8 rows of the tile in LDS (rows padded to 72 elements so that
// 16-byte stores of consecutive rows stay aligned). Needs C, ld and Rpad multiples of 8 and
// 16-byte aligned src and dst. Measured on MI355X: B^T of 8960 x 64 2.6 against 5.3 us, W^T of
// 8960 x 1536 11.6 against 18.7 us; the same bytes.
__global__ __launch_bounds__(256) void transpose_pad16_kernel(const bf16_bits* __restrict__ src, int64_t lds_,
                                                              int64_t R, int64_t C, bf16_bits* __restrict__ dst,
                                                              int64_t Rpad, int64_t Cpad) {
  __shared__ __attribute__((aligned(16))) bf16_bits tile[64][72];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 64, c0 = static_cast<int64_t>(blockIdx.y) * 64;
  const int pc = threadIdx.x & 7, rr = threadIdx.x >> 3;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = rr + 32 * h;
    const int64_t r = r0 + i, c = c0 + pc * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < R && c < C) v = *reinterpret_cast<const u32x4*>(src + r * lds_ + c);
    *reinterpret_cast<u32x4*>(&tile[i][pc * 8]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = rr + 32 * h;  // destination row c0 + j, elements r0 + 8 pc .. + 7
    const int64_t c = c0 + j, r = r0 + pc * 8;
    if (c < Cpad && r < Rpad) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = static_cast<uint32_t>(tile[pc * 8 + 2 * e][j]) |
               (static_cast<uint32_t>(tile[pc * 8 + 2 * e + 1][j]) << 16);
      *reinterpret_cast<u32x4*>(dst + c * Rpad + r) = o;
    }
  }
}

hipError_t transpose_pad_impl(const bf16_bits* src, int64_t ld, int64_t R, int64_t C, bf16_bits* dst, int64_t Rpad,
                              int64_t Cpad, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((Rpad + 63) / 64), static_cast<unsigned>((Cpad + 63) / 64));
  const bool wide = C % 8 == 0 && ld % 8 == 0 && Rpad % 8 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(dst) % 16 == 0;
  if (wide) hipLaunchKernelGGL(transpose_pad16_kernel, grid, dim3(256), 0, s, src, ld, R, C, dst, Rpad, Cpad);
  else hipLaunchKernelGGL(transpose_pad_kernel, grid, dim3(256), 0, s, src, ld, R, C, dst, Rpad, Cpad);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Token contraction: part[z][i][j] = sum over tokens t of chunk z of P[t][i] . Q[t][j],
// P [T, M] (row stride ldp, M % 8 == 0) token-major, Q given transposed as Qt [J, Tpad]
// (token-contiguous rows, zero past T), bf16; i < M, j in the grid's 64-column slice of J;
// with ONES, one more 16-column block whose column 0 is 1 (the column sums of P, written at
// column J).
// Workgroup: 256 values of i (4 waves of 64) x 64 values of j, tokens in 64-token steps. Each
// thread loads an 8-token x 8-column block of P (eight 16-byte loads, 512 contiguous bytes per
// half wave and token), transposes it in registers and writes 8 row pieces of P^T to LDS; the Q
// slice (64 j x 64 tokens) is staged in LDS once for the 4 waves. Two LDS buffers, the next
// step's loads in flight during the current step's MFMAs.

// A staged slice in LDS: row = i (or j), 64 tokens = 128 bytes = 8 pieces of 16 bytes, the piece
// index XOR-swizzled by bits 0-2 and 3-5 of the row: 8 lanes that write 8 rows 8 apart, or read 8
// consecutive rows, touch 8 different bank groups.
__device__ __forceinline__ int tsw(int row, int piece) { return row * 8 + (piece ^ ((row ^ (row >> 3)) & 7)); }

template <bool ONES>
__global__ __launch_bounds__(256, 2) void tn_kernel(const bf16_bits* __restrict__ P, int64_t ldp, int64_t M,
                                                    const bf16_bits* __restrict__ Qt, int64_t tpad, int J, int64_t T,
                                                    int64_t tchunk, float* __restrict__ part, int Jt) {
  constexpr int kPBytes = kTnI * kTnT * 2, kQBytes = kTnJ * kTnT * 2;
  __shared__ __attribute__((aligned(256))) char buf[2][kPBytes + kQBytes];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kTnI;
  const int z = blockIdx.y;
  const int j0 = blockIdx.z * kTnJ;
  const int jn = min(kTnJ, J - j0);         // columns of Q in this slice (a multiple of 16)
  const int nj = jn / 16;
  const bool ones = ONES && blockIdx.z == 0;  // the column-of-ones block rides with the first slice
  const int64_t t_lo = z * tchunk, t_hi = min<int64_t>(T, t_lo + tchunk);
  const int nsteps = static_cast<int>((t_hi - t_lo + kTnT - 1) / kTnT);

  // this thread's P block: columns i0 + 8 c .. + 7, tokens 8 g .. 8 g + 7 of the step
  const int c = threadIdx.x & 31, g = threadIdx.x >> 5;
  const bool pcol = i0 + 8 * c < M;
  const bf16_bits* prow = P + i0 + 8 * c;
  // this thread's two Q pieces: rows j0 + (k >> 3), tokens 8 (k & 7) .. + 7, k = tid, tid + 256
  u32x4 pv[8], qv[2];
  auto load = [&](int step) {
    const int64_t t = t_lo + static_cast<int64_t>(step) * kTnT + 8 * g;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[e] = u32x4{0u, 0u, 0u, 0u};
      if (pcol && t + e < t_hi) pv[e] = *reinterpret_cast<const u32x4*>(prow + (t + e) * ldp);
    }
    const int64_t ts = t_lo + static_cast<int64_t>(step) * kTnT;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = threadIdx.x + 256 * h, jr = k >> 3;
      qv[h] = u32x4{0u, 0u, 0u, 0u};
      if (jr < jn) qv[h] = *reinterpret_cast<const u32x4*>(Qt + static_cast<int64_t>(j0 + jr) * tpad + ts + 8 * (k & 7));
    }
  };
  auto stage = [&](int b) {
    char* pb = buf[b];
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) {  // row 8 c + ii of P^T: tokens 8 g .. 8 g + 7
      u32x4 o;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t lo = pv[2 * m][ii >> 1], hi = pv[2 * m + 1][ii >> 1];
        o[m] = (ii & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      *reinterpret_cast<u32x4*>(pb + tsw(8 * c + ii, g) * 16) = o;
    }
    char* qb = pb + kPBytes;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = threadIdx.x + 256 * h;
      *reinterpret_cast<u32x4*>(qb + tsw(k >> 3, k & 7) * 16) = qv[h];
    }
  };

  f32x4 acc[4][kTnJ / 16], acc1[4];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    acc1[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jb = 0; jb < kTnJ / 16; ++jb) acc[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // the ones operand: column 0 of the block is 1 for every token, the other columns 0
  const bf16_bits one = 0x3f80;
  const uint32_t ow = r == 0 ? (static_cast<uint32_t>(one) | (static_cast<uint32_t>(one) << 16)) : 0u;
  const bf16x8 ones_frag = __builtin_bit_cast(bf16x8, u32x4{ow, ow, ow, ow});

  if (nsteps > 0) {
    load(0);
    stage(0);
  }
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const int b = step & 1;
    if (step + 1 < nsteps) load(step + 1);
    const char* pb = buf[b];
    const char* qb = pb + kPBytes;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {  // 32-token halves of the step
      bf16x8 af[4], bq[kTnJ / 16];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
        af[ib] = *reinterpret_cast<const bf16x8*>(pb + tsw(wave * 64 + ib * 16 + r, 4 * kk + q) * 16);
#pragma unroll
      for (int jb = 0; jb < kTnJ / 16; ++jb)
        if (jb < nj) bq[jb] = *reinterpret_cast<const bf16x8*>(qb + tsw(jb * 16 + r, 4 * kk + q) * 16);
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
#pragma unroll
        for (int jb = 0; jb < kTnJ / 16; ++jb)
          if (jb < nj) acc[ib][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ib], bq[jb], acc[ib][jb], 0, 0, 0);
        if (ones) acc1[ib] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ib], ones_frag, acc1[ib], 0, 0, 0);
      }
    }
    if (step + 1 < nsteps) stage(b ^ 1);  // (buffer b ^ 1 was last read before the previous barrier)
    __syncthreads();
  }
  // lane (r, q) of block (ib, jb) holds D[i = 64 wave + 16 ib + 4 q + e][j = 16 jb + r]
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = i0 + wave * 64 + ib * 16 + 4 * q + e;
      if (i >= M) continue;
      float* row = part + (static_cast<int64_t>(z) * M + i) * Jt;
#pragma unroll
      for (int jb = 0; jb < kTnJ / 16; ++jb)
        if (jb < nj) row[j0 + jb * 16 + r] = acc[ib][jb][e];
      if (ones && r == 0) row[J] = acc1[ib][e];
    }
  }
}

// out = sum over z (in order) of part[z]: dA^T layout (TRANSPOSE: out[j][i], j < jvalid) or
// dB layout (out[i][j], j < jvalid) plus, with a column of ones, its sums to col_out[i].
__global__ __launch_bounds__(256) void tn_reduce_kernel(const float* __restrict__ part, int S, int64_t M, int Jt,
                                                        int jvalid, bool transpose, float* __restrict__ out,
                                                        int64_t ldo, int ones_col, float* __restrict__ col_out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= M * Jt) return;
  const int64_t i = idx / Jt;
  const int j = static_cast<int>(idx - i * Jt);
  const bool is_ones = ones_col >= 0 && j == ones_col;
  if (!is_ones && j >= jvalid) return;
  if (is_ones && col_out == nullptr) return;
  // chunks added in order; eight loads issued before their adds
  const float* pz = part + i * Jt + j;
  const int64_t zs = M * Jt;
  float v = 0.f;
  int z = 0;
  for (; z + 8 <= S; z += 8) {
    float t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = pz[(z + k) * zs];
#pragma unroll
    for (int k = 0; k < 8; ++k) v += t[k];
  }
  for (; z < S; ++z) v += pz[z * zs];
  if (is_ones) col_out[i] = v;
  else if (transpose) out[static_cast<int64_t>(j) * ldo + i] = v;
  else out[i * ldo + j] = v;
}

__global__ __launch_bounds__(256) void zero_fill_kernel(float* __restrict__ dst, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = 0.f;
}

}  // namespace

hipError_t zero_fill(float* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(zero_fill_kernel, dim3(static_cast<unsigned>(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s,
                     dst, n);
  return hipGetLastError();
}

hipError_t transpose_pad(const uint16_t* src, int64_t ld, int64_t R, int64_t C, uint16_t* dst, int64_t Rpad,
                         int64_t Cpad, hipStream_t s) {
  return transpose_pad_impl(src, ld, R, C, dst, Rpad, Cpad, s);
}

// Token chunks of a contraction over T tokens with `tiles` workgroups per chunk: at most 512
// workgroups (two per compute unit, all resident at once), chunks a multiple of 64 tokens and
// of at least 256 tokens, at most 64 chunks.
hipError_t tn_contract(const bf16_bits* P, int64_t ldp, int64_t M, const bf16_bits* Qt, int64_t tpad, int J,
                       int64_t T, bool ones, float* part, float* out, int64_t ldo, int jvalid, bool transpose,
                       float* col_out, hipStream_t s) {
  const int jslices = (J + kTnJ - 1) / kTnJ;
  const int Jt = J + (ones ? 16 : 0);
  int S;
  int64_t tchunk;
  const int64_t itiles = (M + kTnI - 1) / kTnI;
  tn_plan(T, itiles * jslices, &S, &tchunk);
  const dim3 grid(static_cast<unsigned>(itiles), static_cast<unsigned>(S), static_cast<unsigned>(jslices));
  if (ones) hipLaunchKernelGGL(tn_kernel<true>, grid, dim3(256), 0, s, P, ldp, M, Qt, tpad, J, T, tchunk, part, Jt);
  else hipLaunchKernelGGL(tn_kernel<false>, grid, dim3(256), 0, s, P, ldp, M, Qt, tpad, J, T, tchunk, part, Jt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = M * Jt;
  hipLaunchKernelGGL(tn_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, part, S, M, Jt,
                     jvalid, transpose, out, ldo, ones ? J : -1, col_out);
  return hipGetLastError();
}

}  // namespace lora
