// C-ABI of the fused LoRA linear library: argument validation, scale folding
// and dispatch to the gfx950 kernels. Every check runs before any launch, so a
// nonzero status means nothing was written.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstring>

#include "backward.hpp"
#include "lora_mi355x.h"
#include "launch.hpp"

namespace {

using lora::Elt;
using lora::GroupDev;
using lora::LinearProblem;

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
  bool empty() const { return lo == hi; }
};

Span span2d(const void* p, int64_t rows, int64_t ld, int64_t cols, int esize) {
  Span s;
  if (p == nullptr || rows <= 0 || cols <= 0) return s;
  s.lo = reinterpret_cast<uintptr_t>(p);
  s.hi = s.lo + static_cast<uintptr_t>(((rows - 1) * ld + cols) * esize);
  return s;
}

bool overlaps(const Span& a, const Span& b) {
  return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t a) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % a == 0; }

bool dtype_ok(int d) { return d == LORA_F32 || d == LORA_BF16; }
Elt to_elt(int d) { return d == LORA_BF16 ? Elt::BF16 : Elt::F32; }
int esz(int d) { return d == LORA_BF16 ? 2 : 4; }

bool finite_scale(double v) { return std::isfinite(v); }

// The staging kernels address one tile of rows with 32-bit byte offsets.
constexpr int64_t kMaxRowBytes = int64_t(1) << 22;

// Adapter description shared by the linear entry points.
struct Adapter {
  const void* A;
  const void* B;
  int32_t rank;
  double alpha;
  int64_t col_off, n_cols;
  double strength;
  const void* Bb;  // legacy lora_B bias [n_cols], or null
};

int fill_groups(LinearProblem& p, const Adapter* ads, int n, double request_scale) {
  p.n_groups = 0;
  int64_t tcol = 0;
  for (int i = 0; i < n; ++i) {
    const Adapter& a = ads[i];
    if (a.A == nullptr && a.B == nullptr) continue;  // no adapter on these columns
    const double strength = a.strength;
    const double s = (a.alpha / static_cast<double>(a.rank)) * strength * request_scale;
    if (s == 0.0) continue;  // a zero combined scale leaves the adapter inactive
    if (std::fabs(s) > FLT_MAX) return LORA_ERR_NONFINITE;
    if (a.Bb != nullptr && std::fabs(strength * request_scale) > FLT_MAX) return LORA_ERR_NONFINITE;
    GroupDev& g = p.g[p.n_groups++];
    g.A = a.A;
    g.B = a.B;
    g.col_off = a.col_off;
    g.n_cols = a.n_cols;
    g.rank = a.rank;
    g.r_pad = static_cast<int32_t>(lora::rank_pad(a.rank));
    g.t_col = static_cast<int32_t>(tcol);
    g.scale = static_cast<float>(s);
    g.bscale = static_cast<float>(strength * request_scale);
    g.f[0] = static_cast<float>(a.alpha / static_cast<double>(a.rank));
    g.f[1] = static_cast<float>(strength);
    g.f[2] = static_cast<float>(request_scale);
    g.Bb = a.Bb;
    tcol += g.r_pad;
  }
  p.ldt = tcol;
  return LORA_OK;
}

constexpr size_t kWsAlign = 256;
size_t round_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Workspace layout of a call. Usually t~ [T, sum r_pad] in the adapter dtype.
// Lossless fp32 adapters on bf16 activations: t~ [T, 3 sum r_pad] bf16, then the
// split copies A2 of every group ([2 r_pad, K] bf16), then B2 ([n_cols, 3 r_pad]
// bf16); assign_split() points the groups at them. A lossless 4-bit weight with
// T > kSkinnyMaxT that is dequantized once per call (nf4_uses_panel) adds its bf16
// panel [N, K] after all of that (256-byte aligned); the GEMM then sees a bf16
// weight, so an fp32 adapter (which always takes the panel) takes the split layout.
// The lossless bf16 producer splits K (fp32 partial sums after t~, 256-byte aligned).
bool producer_split(const LinearProblem& p, bool lossless) {
  return lossless && p.act == Elt::BF16 && p.adapter == Elt::BF16 && p.n_groups > 0 &&
         lora::producer_partial_bytes(p.T, p.K, p.ldt) > 0;
}

size_t adapter_bytes_for(const LinearProblem& p, bool lossless, bool gemm_nf4) {
  if (p.n_groups == 0 || p.T == 0) return 0;
  if (lossless && lora::split_fp32_adapter(p.act, p.adapter, gemm_nf4)) {
    size_t bytes = round_up(static_cast<size_t>(p.T) * static_cast<size_t>(3 * p.ldt) * 2);
    for (int i = 0; i < p.n_groups; ++i) bytes += round_up(static_cast<size_t>(2 * p.g[i].r_pad) * p.K * 2);
    for (int i = 0; i < p.n_groups; ++i) bytes += round_up(static_cast<size_t>(p.g[i].n_cols) * 3 * p.g[i].r_pad * 2);
    return bytes;
  }
  size_t bytes = static_cast<size_t>(p.T) * static_cast<size_t>(p.ldt) * static_cast<size_t>(lora::esize(p.adapter));
  if (producer_split(p, lossless)) bytes = round_up(bytes) + lora::producer_partial_bytes(p.T, p.K, p.ldt);
  return bytes;
}

size_t panel_bytes(int64_t N, int64_t K) { return static_cast<size_t>(N) * static_cast<size_t>(K) * 2; }

size_t workspace_rest_for(const LinearProblem& p, bool lossless, bool panel);

// Lossless: b + sum_g u_g . c_g (u_g = strength_g . request_scale) as one fp32
// vector [N] at the front of the workspace when an active adapter has a legacy
// lora_B bias.
bool needs_bias32(const LinearProblem& p, bool lossless) {
  if (!lossless) return false;
  for (int i = 0; i < p.n_groups; ++i)
    if (p.g[i].Bb != nullptr) return true;
  return false;
}

size_t workspace_bytes_for(const LinearProblem& p, bool lossless, bool panel) {
  if (p.T == 0) return 0;
  const size_t front = needs_bias32(p, lossless) ? round_up(static_cast<size_t>(p.N) * 4) : 0;
  return front + workspace_rest_for(p, lossless, panel);
}

// 4-bit weight dequantized inside the hot GEMM: bf16 adapter, ranks multiples of 8.
bool nf4_in_gemm_ok(const LinearProblem& p) {
  if (p.act != Elt::BF16 || p.adapter != Elt::BF16 || p.n_groups > 1) return false;
  return p.n_groups == 0 || p.g[0].rank % 8 == 0;
}

size_t workspace_rest_for(const LinearProblem& p, bool lossless, bool panel) {
  if (lora::skinny_path(p.act, lossless, p.T, p.ldt)) return lora::skinny_bytes(p.T, p.K, p.N, p.ldt);
  const size_t ad = adapter_bytes_for(p, lossless, p.nf4 && !panel);
  return panel ? round_up(ad) + panel_bytes(p.N, p.K) : ad;
}

void assign_split(LinearProblem& p) {
  char* w = static_cast<char*>(p.work);
  size_t off = round_up(static_cast<size_t>(p.T) * static_cast<size_t>(3 * p.ldt) * 2);
  for (int i = 0; i < p.n_groups; ++i) {
    p.g[i].A2 = w + off;
    off += round_up(static_cast<size_t>(2 * p.g[i].r_pad) * p.K * 2);
  }
  for (int i = 0; i < p.n_groups; ++i) {
    p.g[i].B2 = w + off;
    off += round_up(static_cast<size_t>(p.g[i].n_cols) * 3 * p.g[i].r_pad * 2);
  }
}

// Shared validation + dispatch for lora_linear_fwd / _stacked_fwd / _nf4_fwd.
int run_linear(const void* x, int64_t T, int64_t K, int64_t ldx, const void* W, const uint8_t* codes,
               const float* absmax, const float* codebook, bool nf4, int64_t N, const void* bias,
               const Adapter* ads, int n_ads, int adapter_dtype, double request_scale,
               void* y, int64_t ldy, int act_dtype, int quality, void* workspace, size_t workspace_bytes,
               void* stream, int phase = 0, bool overlap_ok = false, int tile = 0, int nf4_mode = 0) {
  if (!dtype_ok(act_dtype) || !dtype_ok(adapter_dtype)) return LORA_ERR_DTYPE;
  if (act_dtype == LORA_F32 && adapter_dtype != LORA_F32) return LORA_ERR_DTYPE;
  if (quality != LORA_LOSSLESS && quality != LORA_EXACT) return LORA_ERR_UNSUPPORTED;
  if (T < 0 || K < 1 || N < 1 || ldx < K || ldy < N) return LORA_ERR_SHAPE;
  if (!finite_scale(request_scale)) return LORA_ERR_NONFINITE;
  for (int i = 0; i < n_ads; ++i)
    if (!finite_scale(ads[i].strength)) return LORA_ERR_NONFINITE;
  if (nf4) {
    if (codes == nullptr || absmax == nullptr || codebook == nullptr) return LORA_ERR_NULL_PTR;
    if (K % 64 != 0) return LORA_ERR_SHAPE;
    if (nf4_mode != lora::kNf4Auto && nf4_mode != lora::kNf4Panel && nf4_mode != lora::kNf4InGemm)
      return LORA_ERR_UNSUPPORTED;
  } else if (W == nullptr) {
    return LORA_ERR_NULL_PTR;
  }
  if (T > 0 && (x == nullptr || y == nullptr)) return LORA_ERR_NULL_PTR;
  for (int i = 0; i < n_ads; ++i) {
    const Adapter& a = ads[i];
    if ((a.A == nullptr) != (a.B == nullptr)) return LORA_ERR_NULL_PTR;
    if (!finite_scale(a.alpha)) return LORA_ERR_NONFINITE;
    if (a.A == nullptr) continue;
    if (a.rank < 1) return LORA_ERR_SHAPE;
    if (a.rank > LORA_MAX_RANK) return LORA_ERR_UNSUPPORTED;
    if (a.n_cols < 1 || a.col_off < 0 || a.col_off + a.n_cols > N) return LORA_ERR_SHAPE;
  }
  // stacked groups must be disjoint (several adapters on one layer may overlap)
  for (int i = 0; i < n_ads && !overlap_ok; ++i)
    for (int j = i + 1; j < n_ads; ++j) {
      const Adapter &a = ads[i], &b = ads[j];
      if (a.A == nullptr || b.A == nullptr) continue;
      if (a.col_off < b.col_off + b.n_cols && b.col_off < a.col_off + a.n_cols) return LORA_ERR_SHAPE;
    }

  const int ea = esz(act_dtype), el = esz(adapter_dtype);
  if (ldx * ea > kMaxRowBytes || ldy * ea > kMaxRowBytes || K * 4 > kMaxRowBytes) return LORA_ERR_UNSUPPORTED;

  // alignment
  if (quality == LORA_LOSSLESS) {
    const int vec = 16 / ea;
    if (!aligned(x, 16) || !aligned(W, 16) || !aligned(y, ea) || !aligned(codes, 16)) return LORA_ERR_ALIGN;
    if (K % vec != 0 || ldx % vec != 0) return LORA_ERR_ALIGN;
    for (int i = 0; i < n_ads; ++i)
      if (!aligned(ads[i].A, 16) || !aligned(ads[i].B, 16) || !aligned(ads[i].Bb, el)) return LORA_ERR_ALIGN;
    if (!aligned(workspace, 16)) return LORA_ERR_ALIGN;
  } else {
    if (!aligned(x, ea) || !aligned(W, ea) || !aligned(y, ea)) return LORA_ERR_ALIGN;
    for (int i = 0; i < n_ads; ++i)
      if (!aligned(ads[i].A, el) || !aligned(ads[i].B, el) || !aligned(ads[i].Bb, el)) return LORA_ERR_ALIGN;
    if (!aligned(workspace, 4)) return LORA_ERR_ALIGN;
  }
  if (!aligned(bias, ea) || !aligned(absmax, 4) || !aligned(codebook, 4)) return LORA_ERR_ALIGN;

  LinearProblem p;
  std::memset(&p, 0, sizeof(p));
  p.x = x; p.ldx = ldx; p.W = W; p.codes = codes; p.absmax = absmax; p.codebook = codebook;
  p.bias = bias; p.y = y; p.ldy = ldy; p.T = T; p.N = N; p.K = K;
  p.act = to_elt(act_dtype); p.adapter = to_elt(adapter_dtype); p.nf4 = nf4; p.tile = tile;
  const int st = fill_groups(p, ads, n_ads, request_scale);
  if (st != LORA_OK) return st;

  const bool lossless = quality == LORA_LOSSLESS;
  const bool use_skinny = lora::skinny_path(p.act, lossless, T, p.ldt);
  const bool in_gemm_ok = nf4_in_gemm_ok(p);
  if (nf4 && lossless && nf4_mode == lora::kNf4InGemm && !in_gemm_ok) return LORA_ERR_UNSUPPORTED;
  const bool use_panel = !use_skinny && lora::nf4_uses_panel(nf4, lossless, T, in_gemm_ok, nf4_mode);
  const size_t need = workspace_bytes_for(p, lossless, use_panel);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LORA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  if (need > 0 && needs_bias32(p, lossless)) {
    p.bias32 = reinterpret_cast<float*>(ws);
    ws += round_up(static_cast<size_t>(N) * 4);
  }
  p.work = ws;
  if (use_skinny) {
    p.skinny = reinterpret_cast<float*>(ws);
  } else {
    if (p.n_groups > 0 && lossless && lora::split_fp32_adapter(p.act, p.adapter, nf4 && !use_panel)) assign_split(p);
    if (producer_split(p, lossless))
      p.tpart = reinterpret_cast<float*>(ws + round_up(static_cast<size_t>(T) * static_cast<size_t>(p.ldt) * 2));
    if (use_panel) p.panel = ws + round_up(adapter_bytes_for(p, lossless, false));
  }

  // the output must not overlap any input or the workspace
  if (T > 0) {
    const Span sy = span2d(y, T, ldy, N, ea);
    const Span sw = nf4 ? span2d(codes, N, K / 2, K / 2, 1) : span2d(W, N, K, K, ea);
    Span inputs[8] = {span2d(x, T, ldx, K, ea), sw, span2d(bias, 1, N, N, ea),
                      nf4 ? span2d(absmax, 1, N * K / 64, N * K / 64, 4) : Span{},
                      span2d(codebook, 1, 16, 16, 4),
                      need ? Span{reinterpret_cast<uintptr_t>(workspace),
                                  reinterpret_cast<uintptr_t>(workspace) + need} : Span{},
                      Span{}, Span{}};
    for (const Span& s : inputs)
      if (overlaps(sy, s)) return LORA_ERR_OVERLAP;
    const Span sws = inputs[5];
    for (int i = 0; i < n_ads; ++i) {
      const Adapter& a = ads[i];
      if (a.A == nullptr) continue;
      const Span sa = span2d(a.A, a.rank, K, K, el), sb = span2d(a.B, a.n_cols, a.rank, a.rank, el);
      const Span sc = span2d(a.Bb, 1, a.n_cols, a.n_cols, el);
      if (overlaps(sy, sa) || overlaps(sy, sb) || overlaps(sws, sa) || overlaps(sws, sb) || overlaps(sy, sc) ||
          overlaps(sws, sc))
        return LORA_ERR_OVERLAP;
    }
    for (int i = 0; i < 5; ++i)
      if (overlaps(sws, inputs[i])) return LORA_ERR_OVERLAP;
  }
  if (T == 0) return LORA_OK;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.bias32 != nullptr && phase != 1) {
    const hipError_t eb = lora::launch_bias32(p, s);
    if (eb != hipSuccess) return LORA_ERR_HIP;
  }
  const hipError_t e = (quality == LORA_EXACT) ? lora::launch_exact(p, s) : lora::launch_lossless(p, s, phase);
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

// Workspace of lora_linear_bwd: W^T (when dx is wanted), B^T, A^T, u~ (+ its producer's partial
// sums), t~ (+ partial sums), the token contractions' partial sums; each region 256-byte aligned.
struct BwdLayout {
  size_t wt = 0, bt = 0, at = 0, ut = 0, upart = 0, tt = 0, tpart = 0, qt = 0, tn = 0, total = 0;
  bool has_upart = false, has_tpart = false;
};

BwdLayout bwd_layout(int64_t T, int64_t K, int64_t N, int64_t rp, bool want_dx) {
  BwdLayout L;
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off = round_up(off + n);
    return o;
  };
  if (want_dx) L.wt = take(static_cast<size_t>(K) * N * 2);
  L.bt = take(static_cast<size_t>(rp) * N * 2);
  L.at = take(static_cast<size_t>(K) * rp * 2);
  L.ut = take(static_cast<size_t>(T) * rp * 2);
  const size_t up = lora::producer_partial_bytes(T, N, rp), tp = lora::producer_partial_bytes(T, K, rp);
  L.has_upart = up > 0;
  L.has_tpart = tp > 0;
  if (up > 0) L.upart = take(up);
  L.tt = take(static_cast<size_t>(T) * rp * 2);
  if (tp > 0) L.tpart = take(tp);
  L.qt = take(static_cast<size_t>(rp) * lora::tn_tpad(T) * 2);  // u~ or t~ transposed, one at a time
  L.tn = take(std::max(lora::tn_partial_bytes(T, K, static_cast<int>(rp), false),
                       lora::tn_partial_bytes(T, N, static_cast<int>(rp), true)));
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

int lora_linear_fwd(const void* x, int64_t T, int64_t K, int64_t ldx, const void* W, int64_t N, const void* bias,
                    const void* A, const void* B, int32_t rank, int32_t adapter_dtype, double alpha,
                    double strength, double request_scale, void* y, int64_t ldy, int32_t act_dtype,
                    int32_t quality, void* workspace, size_t workspace_bytes, void* stream) {
  const Adapter a{A, B, rank, alpha, 0, N, strength, nullptr};
  return run_linear(x, T, K, ldx, W, nullptr, nullptr, nullptr, false, N, bias, &a, 1, adapter_dtype,
                    request_scale, y, ldy, act_dtype, quality, workspace, workspace_bytes, stream);
}

int lora_linear_fwd_phase(int32_t phase, int32_t gemm_tile, const void* x, int64_t T, int64_t K, int64_t ldx,
                          const void* W, int64_t N, const void* bias, const void* A, const void* B, int32_t rank,
                          int32_t adapter_dtype, double alpha, double strength, double request_scale, void* y,
                          int64_t ldy, int32_t act_dtype, int32_t quality, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (phase < 0 || phase > 2 || gemm_tile < 0 || gemm_tile > 2) return LORA_ERR_UNSUPPORTED;
  if (quality != LORA_LOSSLESS) return LORA_ERR_UNSUPPORTED;
  const Adapter a{A, B, rank, alpha, 0, N, strength, nullptr};
  return run_linear(x, T, K, ldx, W, nullptr, nullptr, nullptr, false, N, bias, &a, 1, adapter_dtype,
                    request_scale, y, ldy, act_dtype, quality, workspace, workspace_bytes, stream, phase, false,
                    gemm_tile);
}

int lora_linear_stacked_fwd(const void* x, int64_t T, int64_t K, int64_t ldx, const void* W, int64_t N_total,
                            const void* bias, const lora_group* groups, int32_t n_groups, int32_t adapter_dtype,
                            double strength, double request_scale, void* y, int64_t ldy, int32_t act_dtype,
                            int32_t quality, void* workspace, size_t workspace_bytes, void* stream) {
  if (n_groups < 0) return LORA_ERR_SHAPE;
  if (n_groups > LORA_MAX_GROUPS) return LORA_ERR_UNSUPPORTED;
  if (n_groups > 0 && groups == nullptr) return LORA_ERR_NULL_PTR;
  Adapter ads[LORA_MAX_GROUPS];
  for (int i = 0; i < n_groups; ++i)
    ads[i] = Adapter{groups[i].A, groups[i].B, groups[i].rank, groups[i].alpha, groups[i].col_offset,
                     groups[i].n_cols, strength, nullptr};
  return run_linear(x, T, K, ldx, W, nullptr, nullptr, nullptr, false, N_total, bias, ads, n_groups,
                    adapter_dtype, request_scale, y, ldy, act_dtype, quality, workspace,
                    workspace_bytes, stream);
}

int lora_linear_multi_fwd(const void* x, int64_t T, int64_t K, int64_t ldx, const void* W, int64_t N,
                          const void* bias, const lora_adapter* adapters, int32_t n_adapters, int32_t adapter_dtype,
                          double request_scale, void* y, int64_t ldy, int32_t act_dtype, int32_t quality,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (n_adapters < 0) return LORA_ERR_SHAPE;
  if (n_adapters > LORA_MAX_GROUPS) return LORA_ERR_UNSUPPORTED;
  if (n_adapters > 0 && adapters == nullptr) return LORA_ERR_NULL_PTR;
  Adapter ads[LORA_MAX_GROUPS];
  for (int i = 0; i < n_adapters; ++i) {
    const lora_adapter& a = adapters[i];
    if (a.B_bias != nullptr && a.A == nullptr) return LORA_ERR_NULL_PTR;  // a bias without its adapter
    ads[i] = Adapter{a.A, a.B, a.rank, a.alpha, a.col_offset, a.n_cols, a.strength, a.B_bias};
  }
  return run_linear(x, T, K, ldx, W, nullptr, nullptr, nullptr, false, N, bias, ads, n_adapters, adapter_dtype,
                    request_scale, y, ldy, act_dtype, quality, workspace, workspace_bytes, stream, 0, true);
}

int lora_linear_nf4_fwd_ex(const void* x, int64_t T, int64_t K, int64_t ldx, const uint8_t* codes,
                           const float* absmax, const float* codebook, int32_t blocksize, int64_t N, const void* bias,
                           const void* A, const void* B, int32_t rank, int32_t adapter_dtype, double alpha,
                           double strength, double request_scale, void* y, int64_t ldy, int32_t quality,
                           int32_t dequant, void* workspace, size_t workspace_bytes, void* stream) {
  if (blocksize != 64) return LORA_ERR_UNSUPPORTED;
  const Adapter a{A, B, rank, alpha, 0, N, strength, nullptr};
  return run_linear(x, T, K, ldx, nullptr, codes, absmax, codebook, true, N, bias, &a, 1, adapter_dtype,
                    request_scale, y, ldy, LORA_BF16, quality, workspace, workspace_bytes, stream, 0, false, 0,
                    dequant);
}

int lora_linear_nf4_fwd(const void* x, int64_t T, int64_t K, int64_t ldx, const uint8_t* codes,
                        const float* absmax, const float* codebook, int32_t blocksize, int64_t N, const void* bias,
                        const void* A, const void* B, int32_t rank, int32_t adapter_dtype, double alpha,
                        double strength, double request_scale, void* y, int64_t ldy, int32_t quality,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return lora_linear_nf4_fwd_ex(x, T, K, ldx, codes, absmax, codebook, blocksize, N, bias, A, B, rank, adapter_dtype,
                                alpha, strength, request_scale, y, ldy, quality, LORA_NF4_AUTO, workspace,
                                workspace_bytes, stream);
}

int dense_patch_apply(void* dst, int32_t dst_dtype, const int64_t* dst_shape, int32_t dst_ndim, const void* src,
                      int32_t src_dtype, const int64_t* src_shape, int32_t src_ndim, double strength,
                      int32_t mode, void* stream) {
  if (!dtype_ok(dst_dtype) || !dtype_ok(src_dtype)) return LORA_ERR_DTYPE;
  if (mode != LORA_PATCH_ADD && mode != LORA_PATCH_REPLACE) return LORA_ERR_UNSUPPORTED;
  if (dst_ndim < 0 || src_ndim < 0) return LORA_ERR_SHAPE;
  if ((dst_ndim > 0 && dst_shape == nullptr) || (src_ndim > 0 && src_shape == nullptr)) return LORA_ERR_NULL_PTR;
  if (dst_ndim != src_ndim) return LORA_ERR_SHAPE;
  int64_t n = 1;
  for (int i = 0; i < dst_ndim; ++i) {
    if (dst_shape[i] < 0 || dst_shape[i] != src_shape[i]) return LORA_ERR_SHAPE;
    n *= dst_shape[i];
  }
  if (!std::isfinite(strength)) return LORA_ERR_NONFINITE;
  if (std::fabs(strength) > FLT_MAX) return LORA_ERR_NONFINITE;
  if (n > 0 && (dst == nullptr || src == nullptr)) return LORA_ERR_NULL_PTR;
  if (!aligned(dst, esz(dst_dtype)) || !aligned(src, esz(src_dtype))) return LORA_ERR_ALIGN;
  if (n > 0 && overlaps(span2d(dst, 1, n, n, esz(dst_dtype)), span2d(src, 1, n, n, esz(src_dtype))))
    return LORA_ERR_OVERLAP;
  if (n == 0) return LORA_OK;
  const hipError_t e = lora::launch_dense_patch(dst, to_elt(dst_dtype), src, to_elt(src_dtype), n,
                                                static_cast<float>(strength), mode,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

int lora_merge_apply(void* W, int32_t w_dtype, int64_t N, int64_t K, const void* A, const void* B, int32_t rank,
                     int32_t adapter_dtype, double alpha, double strength, int32_t quality, void* stream) {
  if (!dtype_ok(w_dtype) || !dtype_ok(adapter_dtype)) return LORA_ERR_DTYPE;
  if (quality != LORA_LOSSLESS && quality != LORA_EXACT) return LORA_ERR_UNSUPPORTED;
  if (N < 0 || K < 0) return LORA_ERR_SHAPE;
  if (!std::isfinite(alpha) || !std::isfinite(strength)) return LORA_ERR_NONFINITE;
  if (A == nullptr || B == nullptr || (N > 0 && K > 0 && W == nullptr)) return LORA_ERR_NULL_PTR;
  if (rank < 1) return LORA_ERR_SHAPE;
  if (rank > LORA_MAX_RANK || K * 4 > kMaxRowBytes) return LORA_ERR_UNSUPPORTED;
  const double s = (alpha / static_cast<double>(rank)) * strength;
  if (std::fabs(s) > FLT_MAX) return LORA_ERR_NONFINITE;
  const int ew = esz(w_dtype), el = esz(adapter_dtype);
  if (quality == LORA_LOSSLESS) {
    if (!aligned(W, 16) || !aligned(A, 16) || !aligned(B, 16)) return LORA_ERR_ALIGN;
    if (K % 8 != 0) return LORA_ERR_ALIGN;
  } else if (!aligned(W, ew) || !aligned(A, el) || !aligned(B, el)) {
    return LORA_ERR_ALIGN;
  }
  if (N == 0 || K == 0) return LORA_OK;
  const Span sw = span2d(W, N, K, K, ew);
  if (overlaps(sw, span2d(A, rank, K, K, el)) || overlaps(sw, span2d(B, N, rank, rank, el))) return LORA_ERR_OVERLAP;
  if (s == 0.0) return LORA_OK;  // a zero strength (or alpha) leaves the weight as it is
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = quality == LORA_EXACT
                           ? lora::launch_exact_merge(W, to_elt(w_dtype), N, K, A, B, rank, to_elt(adapter_dtype),
                                                      static_cast<float>(s), st)
                           : lora::launch_merge(W, to_elt(w_dtype), N, K, A, B, rank, to_elt(adapter_dtype),
                                                static_cast<float>(s), st);
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

int lora_linear_bwd(const void* x, int64_t T, int64_t K, int64_t ldx, const void* W, int64_t N, const void* A,
                    const void* B, int32_t rank, double alpha, double strength, double request_scale, const void* dy,
                    int64_t lddy, void* dx, int64_t lddx, float* dA, float* dB, float* db, const void* t_tilde,
                    int64_t ldt, void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 0 || K < 1 || N < 1 || ldx < K || lddy < N || (dx != nullptr && lddx < K)) return LORA_ERR_SHAPE;
  if (rank < 1) return LORA_ERR_SHAPE;
  if (rank > LORA_MAX_RANK || K * 4 > kMaxRowBytes || N * 4 > kMaxRowBytes || ldx * 2 > kMaxRowBytes ||
      lddy * 2 > kMaxRowBytes || lddx * 2 > kMaxRowBytes)
    return LORA_ERR_UNSUPPORTED;
  if (!finite_scale(alpha) || !finite_scale(strength) || !finite_scale(request_scale)) return LORA_ERR_NONFINITE;
  const double sd = (alpha / static_cast<double>(rank)) * strength * request_scale;
  if (std::fabs(sd) > FLT_MAX) return LORA_ERR_NONFINITE;
  if (A == nullptr || B == nullptr || (dx != nullptr && W == nullptr)) return LORA_ERR_NULL_PTR;
  if (T > 0 && (x == nullptr || dy == nullptr)) return LORA_ERR_NULL_PTR;
  if (!aligned(x, 16) || !aligned(W, 16) || !aligned(A, 16) || !aligned(B, 16) || !aligned(dy, 16) ||
      !aligned(dx, 2) || !aligned(dA, 4) || !aligned(dB, 4) || !aligned(db, 4) || !aligned(workspace, 16) ||
      !aligned(t_tilde, 2))
    return LORA_ERR_ALIGN;
  if (K % 8 != 0 || N % 8 != 0 || ldx % 8 != 0 || lddy % 8 != 0) return LORA_ERR_ALIGN;
  const int64_t rp = lora::rank_pad(rank);
  if (t_tilde != nullptr && (ldt < rp || ldt * 2 > kMaxRowBytes)) return LORA_ERR_SHAPE;
  const BwdLayout L = T > 0 ? bwd_layout(T, K, N, rp, dx != nullptr) : BwdLayout{};
  const size_t need = L.total;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LORA_ERR_WORKSPACE;
  // outputs must not overlap the inputs, the workspace or each other
  const Span outs[4] = {span2d(dx, T, lddx, K, 2), span2d(dA, 1, rank * K, rank * K, 4),
                        span2d(dB, 1, N * rank, N * rank, 4), span2d(db, 1, N, N, 4)};
  const Span wsp =
      need ? Span{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need} : Span{};
  const Span tts = t_tilde != nullptr ? span2d(t_tilde, T, ldt, rp, 2) : Span{};
  const Span ins[7] = {span2d(x, T, ldx, K, 2), span2d(W, N, K, K, 2), span2d(A, rank, K, K, 2),
                       span2d(B, N, rank, rank, 2), span2d(dy, T, lddy, N, 2), wsp, tts};
  if (overlaps(tts, wsp)) return LORA_ERR_OVERLAP;
  for (int i = 0; i < 4; ++i) {
    for (const Span& in : ins)
      if (overlaps(outs[i], in)) return LORA_ERR_OVERLAP;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outs[j])) return LORA_ERR_OVERLAP;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (T == 0) {  // an empty batch: zero gradients (by kernels: the call may be captured in a graph)
    hipError_t e = hipSuccess;
    if (dA != nullptr) e = lora::zero_fill(dA, static_cast<int64_t>(rank) * K, st);
    if (e == hipSuccess && dB != nullptr) e = lora::zero_fill(dB, N * static_cast<int64_t>(rank), st);
    if (e == hipSuccess && db != nullptr) e = lora::zero_fill(db, N, st);
    return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
  }
  char* ws = static_cast<char*>(workspace);
  auto* wt = reinterpret_cast<uint16_t*>(ws + L.wt);
  auto* bt = reinterpret_cast<uint16_t*>(ws + L.bt);
  auto* at = reinterpret_cast<uint16_t*>(ws + L.at);
  const float s32 = static_cast<float>(sd);
  hipError_t e = hipSuccess;
  // transposed copies: B^T [rp, N] (rows past the rank zero), A^T [K, rp] (columns past the rank zero), W^T [K, N]
  e = lora::transpose_pad(static_cast<const uint16_t*>(B), rank, N, rank, bt, N, rp, st);
  if (e == hipSuccess) e = lora::transpose_pad(static_cast<const uint16_t*>(A), K, rank, K, at, rp, K, st);
  if (e == hipSuccess && dx != nullptr)
    e = lora::transpose_pad(static_cast<const uint16_t*>(W), K, N, K, wt, N, K, st);
  if (e != hipSuccess) return LORA_ERR_HIP;
  // u~ = RN(s . dy.B) and, when wanted, dx = RN(dy.W + u~.A): the forward path over (dy, W^T, B^T, A^T)
  LinearProblem q;
  std::memset(&q, 0, sizeof(q));
  q.x = dy; q.ldx = lddy; q.W = wt; q.y = dx; q.ldy = lddx; q.T = T; q.K = N; q.N = K;
  q.act = Elt::BF16; q.adapter = Elt::BF16; q.n_groups = 1;
  GroupDev& gq = q.g[0];
  gq.A = bt; gq.B = at; gq.col_off = 0; gq.n_cols = K; gq.rank = static_cast<int32_t>(rp);
  gq.r_pad = static_cast<int32_t>(rp); gq.t_col = 0; gq.scale = s32;
  q.work = ws + L.ut; q.ldt = rp;
  if (L.has_upart) q.tpart = reinterpret_cast<float*>(ws + L.upart);
  e = lora::launch_lossless(q, st, dx != nullptr ? 0 : 1);
  if (e != hipSuccess) return LORA_ERR_HIP;
  if (dA == nullptr && dB == nullptr && db == nullptr) return LORA_OK;
  // t~ = RN(s . x.A^T): the forward's producer
  LinearProblem p2;
  std::memset(&p2, 0, sizeof(p2));
  p2.x = x; p2.ldx = ldx; p2.W = W; p2.T = T; p2.K = K; p2.N = N; p2.act = Elt::BF16; p2.adapter = Elt::BF16;
  p2.n_groups = 1;
  GroupDev& g2 = p2.g[0];
  g2.A = A; g2.B = B; g2.col_off = 0; g2.n_cols = N; g2.rank = rank; g2.r_pad = static_cast<int32_t>(rp);
  g2.t_col = 0; g2.scale = s32;
  p2.work = ws + L.tt; p2.ldt = rp;
  if (L.has_tpart) p2.tpart = reinterpret_cast<float*>(ws + L.tpart);
  // (the caller's copy of t~ from the forward, when given: the same bits, without a second read of x)
  const uint16_t* tt = t_tilde != nullptr ? static_cast<const uint16_t*>(t_tilde)
                                          : reinterpret_cast<const uint16_t*>(ws + L.tt);
  const int64_t ldtt = t_tilde != nullptr ? ldt : rp;
  if ((dB != nullptr || db != nullptr) && t_tilde == nullptr) {
    e = lora::launch_lossless(p2, st, 1);
    if (e != hipSuccess) return LORA_ERR_HIP;
  }
  float* part = reinterpret_cast<float*>(ws + L.tn);
  auto* qt = reinterpret_cast<uint16_t*>(ws + L.qt);
  const int64_t tpad = lora::tn_tpad(T);
  const int J = static_cast<int>(rp);
  // (dB before dA: dy was just read by the dx GEMM, and where it is small enough it is still in the
  // Infinity Cache; dA's read of x would evict it. 8960 -> 1536 backward: 927 against 935 us.)
  if (dB != nullptr || db != nullptr) {  // dB = dy^T t~ and db = column sums of dy
    e = lora::transpose_pad(tt, ldtt, T, rp, qt, tpad, rp, st);
    if (e == hipSuccess)
      e = lora::tn_contract(static_cast<const uint16_t*>(dy), lddy, N, qt, tpad, J, T, db != nullptr, part, dB, rank,
                            dB != nullptr ? rank : 0, false, db, st);
    if (e != hipSuccess) return LORA_ERR_HIP;
  }
  if (dA != nullptr) {  // dA = u~^T x: [K, rp] contraction written transposed into [rank, K]
    e = lora::transpose_pad(reinterpret_cast<const uint16_t*>(ws + L.ut), rp, T, rp, qt, tpad, rp, st);
    if (e == hipSuccess)
      e = lora::tn_contract(static_cast<const uint16_t*>(x), ldx, K, qt, tpad, J, T, false, part, dA, K, rank, true,
                            nullptr, st);
    if (e != hipSuccess) return LORA_ERR_HIP;
  }
  return LORA_OK;
}

size_t lora_linear_bwd_workspace_size(int64_t T, int64_t K, int64_t N, int32_t rank, int32_t want_dx) {
  if (T <= 0 || K <= 0 || N <= 0 || rank < 1) return 0;
  return bwd_layout(T, K, N, lora::rank_pad(rank), want_dx != 0).total;
}

size_t lora_linear_workspace_size(int64_t T, int64_t K, int64_t N, const int32_t* ranks, int32_t n_ranks,
                                  int32_t adapter_dtype, int32_t quality) {
  if (T <= 0 || K <= 0 || N <= 0 || n_ranks < 0 || (n_ranks > 0 && ranks == nullptr) || !dtype_ok(adapter_dtype))
    return 0;
  int64_t cols = 0;
  for (int i = 0; i < n_ranks; ++i)
    if (ranks[i] > 0) cols += lora::rank_pad(ranks[i]);
  // few tokens (lossless, bf16 activations): fp32 partial sums instead of the
  // intermediate; the activation dtype is not an argument, so the larger of the two.
  // A call takes the few-token layout when its ACTIVE adapters' padded ranks sum to at
  // most kSkinnyMaxLdt, whatever the ranks passed here add up to (an adapter with a
  // zero scale drops out), so that layout is sized for the largest such sum.
  const size_t skinny = (quality == LORA_LOSSLESS && T <= lora::kSkinnyMaxT)
                            ? lora::skinny_bytes(T, K, N, std::min<int64_t>(cols, lora::kSkinnyMaxLdt)) : 0;
  if (cols == 0) return skinny;
  if (quality == LORA_LOSSLESS && adapter_dtype == LORA_F32) {
    // the bf16-activation layout (the larger of the two an fp32 adapter can need);
    // every group's n_cols is at most N
    size_t bytes = round_up(static_cast<size_t>(T) * static_cast<size_t>(3 * cols) * 2);
    for (int i = 0; i < n_ranks; ++i) {
      if (ranks[i] <= 0) continue;
      const size_t rp = static_cast<size_t>(lora::rank_pad(ranks[i]));
      bytes += round_up(2 * rp * static_cast<size_t>(K) * 2) + round_up(static_cast<size_t>(N) * 3 * rp * 2);
    }
    return std::max(bytes, skinny);
  }
  size_t bytes = static_cast<size_t>(T) * static_cast<size_t>(cols) * static_cast<size_t>(esz(adapter_dtype));
  if (quality == LORA_LOSSLESS && adapter_dtype == LORA_BF16) {  // the producer's K-split partial sums
    const size_t part = lora::producer_partial_bytes(T, K, cols);
    if (part > 0) bytes = round_up(bytes) + part;
  }
  return std::max(bytes, skinny);
}

size_t lora_linear_nf4_workspace_size(int64_t T, int64_t K, int64_t N, int32_t rank, int32_t adapter_dtype,
                                      int32_t quality) {
  if (T <= 0 || K <= 0 || N <= 0 || !dtype_ok(adapter_dtype)) return 0;
  if (quality == LORA_LOSSLESS && T <= lora::kSkinnyMaxT)  // activations are bf16: the skinny path
    return lora::skinny_bytes(T, K, N, rank > 0 ? lora::rank_pad(rank) : 0);
  const size_t ad = rank > 0 ? lora_linear_workspace_size(T, K, N, &rank, 1, adapter_dtype, quality) : 0;
  // (the panel is included whenever a call could use it, so that the size serves either choice)
  if (!lora::nf4_beyond_skinny(true, quality == LORA_LOSSLESS, T)) return ad;
  return round_up(ad) + panel_bytes(N, K);
}

size_t lora_linear_multi_workspace_size(int64_t T, int64_t K, int64_t N, const lora_adapter* adapters,
                                        int32_t n_adapters, int32_t adapter_dtype, int32_t quality) {
  if (T <= 0 || K <= 0 || N <= 0 || n_adapters < 0 || n_adapters > LORA_MAX_GROUPS ||
      (n_adapters > 0 && adapters == nullptr))
    return 0;
  int32_t ranks[LORA_MAX_GROUPS];
  bool legacy = false;
  for (int i = 0; i < n_adapters; ++i) {
    ranks[i] = adapters[i].A != nullptr ? adapters[i].rank : 0;
    legacy = legacy || (adapters[i].A != nullptr && adapters[i].B_bias != nullptr && adapters[i].strength != 0.0);
  }
  const size_t rest = lora_linear_workspace_size(T, K, N, ranks, n_adapters, adapter_dtype, quality);
  return (legacy && quality == LORA_LOSSLESS) ? round_up(static_cast<size_t>(N) * 4) + rest : rest;
}

const char* lora_status_string(int status) {
  switch (status) {
    case LORA_OK: return "ok";
    case LORA_ERR_NULL_PTR: return "required pointer is NULL (or only one of A/B given)";
    case LORA_ERR_SHAPE: return "invalid shape, leading dimension or group layout";
    case LORA_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case LORA_ERR_NONFINITE: return "alpha, strength or request_scale is not finite";
    case LORA_ERR_ALIGN: return "pointer or stride misaligned";
    case LORA_ERR_OVERLAP: return "output overlaps an input or the workspace";
    case LORA_ERR_WORKSPACE: return "workspace missing or too small";
    case LORA_ERR_UNSUPPORTED: return "unsupported device, option or size";
    case LORA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int lora_device_check(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LORA_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LORA_ERR_HIP;
  return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? LORA_OK : LORA_ERR_UNSUPPORTED;
}

}  // extern "C"
