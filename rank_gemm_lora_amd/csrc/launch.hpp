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
  float bscale;      // lossless: legacy lora_B bias factor strength . request_scale, rounded to fp32
  float f[3];        // exact tier: alpha/rank, strength, request_scale, each rounded to fp32
  // Lossless tier, fp32 adapter on bf16 activations: bf16 split copies in the
  // workspace. A2 [2 r_pad, K]: row 2q = hi(A[q]), row 2q + 1 = lo(A[q]);
  // B2 [n_cols, 3 r_pad]: hi(B) | lo(B) | hi(B), each block r_pad wide
  // (hi(v) = RN_bf16(v), lo(v) = RN_bf16(v - hi(v)); padding zero).
  void* A2;
  void* B2;
  const void* Bb;    // legacy lora_B bias [n_cols] in the adapter dtype, or null
};

// Few tokens (lossless, bf16 activations, T <= kSkinnyMaxT): the weight read is
// the whole cost. Each wave multiplies 16 weight rows (or adapter A rows) over
// one K chunk by all the tokens, straight from global memory (a 4-bit weight is
// dequantized in registers); the K chunks write fp32 partial sums [S, T, .] to
// the workspace and a second kernel adds them in chunk order, forms the
// rank-wide intermediate, adds the rank-r update and the bias, and rounds once.
constexpr int64_t kSkinnyMaxT = 64;
constexpr int kSkinnyRows = 64;      // weight rows per workgroup (4 waves of 16)
constexpr int64_t kSkinnyMaxLdt = 4096;  // sum of the padded ranks (the finishing block holds 4 x ldt fp32 in LDS, <= 64 KB)
inline bool skinny_path(Elt act, bool lossless, int64_t T, int64_t ldt) {
  return lossless && act == Elt::BF16 && T > 0 && T <= kSkinnyMaxT && ldt <= kSkinnyMaxLdt;
}
// K chunk (a multiple of 128 elements, at least 512) and number of chunks S <= 32:
// about 32 chunks for long K, fixed by K alone, so the summation order of an output
// does not depend on N or on the adapters (a stacked call equals one call per
// group, bit for bit). Measured on MI355X at 64 tokens (HIP-graph replay):
// - the 512 floor halves the fp32 partial sums where K is short: 1536 -> 8960 with
//   chunks of 256 / 512 / 768 / 1024 (6 / 3 / 2 / 2 chunks) took 26.2 / 23.2 / 25.0 /
//   26.2 us with an adapter and 21.7 / 18.2 / 19.9 / 21.0 us without;
// - more chunks give the long-K layer more workgroups: 8960 -> 1536 with 8 / 14 / 18
//   chunks took 24.6 / 22.3 / 21.8 us with an adapter, 21.6 / 19.6 / 19.0 without.
constexpr int kSkinnyMaxChunks = 32;
inline void skinny_plan(int64_t K, int* S, int64_t* kchunk) {
  int64_t c = (K + kSkinnyMaxChunks - 1) / kSkinnyMaxChunks;
  c = (c + 127) / 128 * 128;
  c = c < 512 ? 512 : c;
  *kchunk = c;
  *S = static_cast<int>((K + c - 1) / c);
}
inline int64_t skinny_npad(int64_t N) { return (N + kSkinnyRows - 1) / kSkinnyRows * kSkinnyRows; }
// fp32 partial sums of the outputs [S, T, npad] followed by those of x.A^T [S, T, ldt].
inline size_t skinny_bytes(int64_t T, int64_t K, int64_t N, int64_t ldt) {
  int S;
  int64_t c;
  skinny_plan(K, &S, &c);
  return static_cast<size_t>(S) * static_cast<size_t>(T) * static_cast<size_t>(skinny_npad(N) + ldt) * 4;
}

// The rank-wide producer of the lossless bf16 path takes 128 tokens per
// workgroup; with fewer than 128 such tiles it also splits K (stages of 64
// elements, at least 4 per split, at most kMaxProducerSplits splits, chosen by T
// and K alone), each split writing fp32 partial sums [S, T, ldt] that a second
// kernel adds in split order before the scale and the rounding.
constexpr int kMaxProducerSplits = 8;
inline void producer_plan(int64_t T, int64_t K, int* S, int* ks) {
  const int64_t mt = (T + 127) / 128, nk = (K * 2 + 127) / 128;
  int64_t s = 1;
  if (mt > 0 && mt < 128) {
    s = (256 + mt - 1) / mt;
    s = s > kMaxProducerSplits ? kMaxProducerSplits : s;
    const int64_t smax = nk / 4 > 1 ? nk / 4 : 1;
    s = s > smax ? smax : s;
  }
  const int64_t k = nk > 0 ? (nk + s - 1) / s : 1;
  *ks = static_cast<int>(k);
  *S = nk > 0 ? static_cast<int>((nk + k - 1) / k) : 1;
}
inline size_t producer_partial_bytes(int64_t T, int64_t K, int64_t ldt) {
  int S, ks;
  producer_plan(T, K, &S, &ks);
  return S > 1 ? static_cast<size_t>(S) * static_cast<size_t>(T) * static_cast<size_t>(ldt) * 4 : 0;
}

// Lossless 4-bit weight beyond the skinny range, two ways:
// - the panel: the weight dequantized once per call into a bf16 copy [N, K] in the
//   workspace, then the bf16 GEMM over it (a write and a re-read of the bf16 weight);
// - in the GEMM: the hot kernel's 128 x 128 tile dequantizes each weight unit itself,
//   once per 128-token output tile (VALU work beside the MFMAs that grows with the
//   token count); bf16 adapters whose ranks are multiples of 8.
// Both give the same weight bits and the same outputs. The automatic choice takes the
// GEMM form up to kNf4InGemmMaxT tokens: measured on MI355X (4096 -> 14336, rank 16), it
// took 67 us against the panel path's 73 up to 256 tokens (the GEMMs are latency-bound
// there, one workgroup per CU, and the panel kernel costs 25 us), and from 320 tokens on the
// panel was faster (7% at 320-512, 1.7x at 8192, where the in-GEMM form is bound by its
// VALU work: 156 VALU instructions per 32 MFMAs of a stage).
enum Nf4Dequant : int { kNf4Auto = 0, kNf4Panel = 1, kNf4InGemm = 2 };
constexpr int64_t kNf4InGemmMaxT = 256;
inline bool nf4_beyond_skinny(bool nf4, bool lossless, int64_t T) { return nf4 && lossless && T > kSkinnyMaxT; }
inline bool nf4_uses_panel(bool nf4, bool lossless, int64_t T, bool in_gemm_ok, int mode) {
  if (!nf4_beyond_skinny(nf4, lossless, T)) return false;
  if (!in_gemm_ok || mode == kNf4Panel) return true;
  return mode == kNf4Auto && T > kNf4InGemmMaxT;
}

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
  void* panel;       // 4-bit weight, lossless, T > kSkinnyMaxT: bf16 [N, K] dequantized copy in the workspace
  float* skinny;     // skinny path: fp32 partial sums in the workspace (null otherwise)
  float* tpart;      // bf16 adapter, lossless: the producer's K-split partial sums (null: no split)
  float* bias32;     // lossless with legacy lora_B biases: b + sum_g u_g . c_g, fp32 [N] (null otherwise);
                     // the epilogues add it instead of `bias`
  const void* bias;
  void* y; int64_t ldy;
  int64_t T, N, K;
  Elt act, adapter;
  bool nf4;
  int n_groups;
  GroupDev g[kMaxGroups];
  void* work;        // t workspace, [T, ldt] in adapter dtype
  int64_t ldt;       // sum of r_pad over groups
  int tile;          // output tile of the hot GEMM: 0 chosen from the shape, 1 256 x 256, 2 128 x 128
};

// Lossless tier: t~ = RN_adt(s . x A^T) into the workspace, then the fused GEMM.
// phase 0 runs both, 1 only the rank-wide producer, 2 only the fused GEMM
// (which reads the t~ a phase-1 call left in the workspace).
hipError_t launch_lossless(const LinearProblem& p, hipStream_t s, int phase = 0);

// Lossless with legacy lora_B biases: p.bias32 = fp32(b) + u_g . fp32(c_g) summed in group order,
// u_g = strength_g . request_scale (the legacy vector does not take alpha / rank).
hipError_t launch_bias32(const LinearProblem& p, hipStream_t s);
// Exact tier: the ordered-fp64 separate-pass chain.
hipError_t launch_exact(const LinearProblem& p, hipStream_t s);
// Merge W <- RN_w(W + s . B.A): lossless (fp32 sum, one rounding) and exact tier.
hipError_t launch_merge(void* W, Elt wdt, int64_t N, int64_t K, const void* A, const void* B, int rank, Elt adt,
                        float s, hipStream_t st);
hipError_t launch_exact_merge(void* W, Elt wdt, int64_t N, int64_t K, const void* A, const void* B, int rank,
                              Elt adt, float s32, hipStream_t st);
// Dense payload over n contiguous elements.
hipError_t launch_dense_patch(void* dst, Elt dst_t, const void* src, Elt src_t, int64_t n,
                              float strength32, int mode, hipStream_t s);

}  // namespace lora
