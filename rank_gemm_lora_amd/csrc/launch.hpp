// Internal interface between the C-ABI host code (api.cpp) and the kernel
// launchers (*.hip). Not part of the public header.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace lora {

constexpr int kMaxGroups = 8;
constexpr int kRankPad = 64;  // rank columns of the t~ workspace are padded to this

enum class Elt : int { F32 = 0, BF16 = 1 };

inline int64_t rank_pad(int64_t r) { return (r + kRankPad - 1) / kRankPad * kRankPad; }
inline int esize(Elt e) { return e == Elt::F32 ? 4 : 2; }

// One adapter group as the kernels see it.
struct GroupDev {
  const void* A;     // [rank, K] adapter dtype
  const void* B;     // [n_cols, rank] adapter dtype
  int64_t col_off;   // first output column of the group
  int64_t n_cols;
  int32_t rank;
  int32_t t_col;     // first column of this group's block in the t workspace
  int32_t r_pad;     // padded rank (multiple of kRankPad)
  float scale;       // lossless: combined scale rounded to fp32
  float f[3];        // exact tier: alpha/rank, strength, request_scale, each rounded to fp32
  // Lossless tier, fp32 adapter on bf16 activations: bf16 split copies in the
  // workspace. A2 [2 r_pad, K]: row 2q = hi(A[q]), row 2q + 1 = lo(A[q]);
  // B2 [n_cols, 3 r_pad]: hi(B) | lo(B) | hi(B), each block r_pad wide
  // (hi(v) = RN_bf16(v), lo(v) = RN_bf16(v - hi(v)); padding zero).
  void* A2;
  void* B2;
};

// Lossless 4-bit weight with at least this many tokens: the weight is
// dequantized once per call into a bf16 panel [N, K] in the workspace and the
// bf16 GEMM runs on it. Below it, every output tile dequantizes its own weight
// stages in registers inside the GEMM (the panel's write and re-read would cost
// more than the repeated dequantization saves).
constexpr int64_t kNf4PanelMinT = 512;
inline bool nf4_uses_panel(bool nf4, bool lossless, int64_t T) { return nf4 && lossless && T >= kNf4PanelMinT; }

// Lossless fp32 adapter on bf16 activations: the products run on bf16 MFMA
// over the hi/lo split (the t~ block of a group is then t_hi | t_hi | t_lo,
// 3 r_pad columns). Workspace bytes of that layout.
inline bool split_fp32_adapter(Elt act, Elt adapter, bool nf4) {
  return act == Elt::BF16 && adapter == Elt::F32 && !nf4;
}

struct LinearProblem {
  const void* x; int64_t ldx;
  const void* W;                                  // [N, K] act dtype (unused for 4-bit)
  const uint8_t* codes; const float* absmax; const float* codebook;  // 4-bit weight
  void* panel;       // 4-bit weight, lossless, T >= kNf4PanelMinT: bf16 [N, K] dequantized copy in the workspace
  const void* bias;
  void* y; int64_t ldy;
  int64_t T, N, K;
  Elt act, adapter;
  bool nf4;
  int n_groups;
  GroupDev g[kMaxGroups];
  void* work;        // t workspace, [T, ldt] in adapter dtype
  int64_t ldt;       // sum of r_pad over groups
};

// Lossless tier: t~ = RN_adt(s . x A^T) into the workspace, then the fused GEMM.
// phase 0 runs both, 1 only the rank-wide producer, 2 only the fused GEMM
// (which reads the t~ a phase-1 call left in the workspace).
hipError_t launch_lossless(const LinearProblem& p, hipStream_t s, int phase = 0);
// Exact tier: the ordered-fp64 separate-pass chain.
hipError_t launch_exact(const LinearProblem& p, hipStream_t s);
// Dense payload over n contiguous elements.
hipError_t launch_dense_patch(void* dst, Elt dst_t, const void* src, Elt src_t, int64_t n,
                              float strength32, int mode, hipStream_t s);

}  // namespace lora
