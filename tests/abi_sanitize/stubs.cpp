// Host-only stand-ins for the kernel launchers, linked with api.cpp in the
// sanitized build of the validation layer (no GPU code, no HIP launches). Each
// records the call and checks that every workspace region the host code hands
// to the kernels lies inside the buffer the caller passed; it then returns
// hipErrorInvalidValue (the bias-vector launcher: success, so that the fused
// launch after it is checked too), so a call that got past validation reports
// LORA_ERR_HIP.
#include <cstdio>
#include <cstdlib>

#include "backward.hpp"
#include "launch.hpp"
#include "stubs.hpp"

namespace stub {
Record rec;

void expect_inside(const void* p, size_t bytes, const char* what) {
  if (p == nullptr || bytes == 0) return;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p), hi = lo + bytes;
  if (lo < rec.ws_lo || hi > rec.ws_hi) {
    std::fprintf(stderr, "workspace region %s [%#lx, %#lx) outside the caller's [%#lx, %#lx)\n", what,
                 (unsigned long)lo, (unsigned long)hi, (unsigned long)rec.ws_lo, (unsigned long)rec.ws_hi);
    std::abort();
  }
}
}  // namespace stub

namespace lora {
namespace {
size_t ru(size_t v) { return (v + 255) / 256 * 256; }

void check_problem(const LinearProblem& p, bool lossless) {
  using stub::expect_inside;
  // the group table: padded ranks, t columns in order, inside the output
  int64_t tcol = 0;
  for (int i = 0; i < p.n_groups; ++i) {
    const GroupDev& g = p.g[i];
    if (g.r_pad != rank_pad(g.rank) || g.t_col != tcol || g.col_off < 0 || g.col_off + g.n_cols > p.N) {
      std::fprintf(stderr, "bad group %d\n", i);
      std::abort();
    }
    tcol += g.r_pad;
  }
  if (p.ldt != tcol) std::abort();
  if (p.bias32 != nullptr) expect_inside(p.bias32, static_cast<size_t>(p.N) * 4, "bias32");
  if (p.skinny != nullptr) {
    expect_inside(p.skinny, skinny_bytes(p.T, p.K, p.N, p.ldt), "skinny partial sums");
    return;
  }
  // (the hi/lo split layout of an fp32 adapter on bf16 activations: not for a 4-bit weight that
  // the GEMM dequantizes itself)
  const bool split = lossless && p.act == Elt::BF16 && p.adapter == Elt::F32 && p.n_groups > 0 &&
                     !(p.nf4 && p.panel == nullptr);
  if (p.n_groups > 0) {
    const size_t t = split ? static_cast<size_t>(p.T) * 3 * p.ldt * 2
                           : static_cast<size_t>(p.T) * p.ldt * esize(p.adapter);
    expect_inside(p.work, t, "t~");
  }
  if (p.tpart != nullptr) expect_inside(p.tpart, producer_partial_bytes(p.T, p.K, p.ldt), "producer partial sums");
  if (p.panel != nullptr) expect_inside(p.panel, static_cast<size_t>(p.N) * p.K * 2, "4-bit panel");
  if (split) {
    for (int i = 0; i < p.n_groups; ++i) {
      expect_inside(p.g[i].A2, static_cast<size_t>(2 * p.g[i].r_pad) * p.K * 2, "A split copy");
      expect_inside(p.g[i].B2, static_cast<size_t>(p.g[i].n_cols) * 3 * p.g[i].r_pad * 2, "B split copy");
    }
  }
  (void)ru;
}
}  // namespace

hipError_t launch_lossless(const LinearProblem& p, hipStream_t, int phase) {
  ++stub::rec.lossless;
  stub::rec.last_phase = phase;
  stub::rec.last_tile = p.tile;
  check_problem(p, true);
  return hipErrorInvalidValue;
}
hipError_t launch_bias32(const LinearProblem& p, hipStream_t) {
  ++stub::rec.bias32;
  check_problem(p, true);
  return hipSuccess;  // (the fused launch that follows is checked too)
}
hipError_t launch_exact(const LinearProblem& p, hipStream_t) {
  ++stub::rec.exact;
  check_problem(p, false);
  return hipErrorInvalidValue;
}
hipError_t launch_merge(void*, Elt, int64_t, int64_t, const void*, const void*, int, Elt, float, hipStream_t) {
  ++stub::rec.merge;
  return hipErrorInvalidValue;
}
hipError_t launch_exact_merge(void*, Elt, int64_t, int64_t, const void*, const void*, int, Elt, float, hipStream_t) {
  ++stub::rec.merge;
  return hipErrorInvalidValue;
}
hipError_t launch_dense_patch(void*, Elt, const void*, Elt, int64_t, float, int, hipStream_t) {
  ++stub::rec.patch;
  return hipErrorInvalidValue;
}
hipError_t zero_fill(float*, int64_t, hipStream_t) {  // (fills a gradient output, not the workspace)
  ++stub::rec.bwd;
  return hipSuccess;
}
hipError_t transpose_pad(const uint16_t*, int64_t, int64_t, int64_t, uint16_t* dst, int64_t Rpad, int64_t Cpad,
                         hipStream_t) {
  ++stub::rec.bwd;
  stub::expect_inside(dst, static_cast<size_t>(Rpad) * Cpad * 2, "transposed copy");
  return hipErrorInvalidValue;
}
hipError_t tn_contract(const uint16_t*, int64_t, int64_t, const uint16_t*, int64_t, int, int64_t, bool, float*,
                       float*, int64_t, int, bool, float*, hipStream_t) {
  ++stub::rec.bwd;
  return hipErrorInvalidValue;
}
}  // namespace lora
