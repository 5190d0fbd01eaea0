// Drives the C-ABI's validation layer in a host-only build under AddressSanitizer
// and UndefinedBehaviorSanitizer (api.cpp + stubs.cpp, no GPU code): every entry
// point with invalid arguments (each must return its status before any launch)
// and with valid ones (they reach a stub launcher, which checks the workspace
// layout and reports LORA_ERR_HIP). Then random calls: each sized by the
// documented workspace query must pass the workspace check, and every region it
// hands to the kernels must lie inside that workspace. Pointers are fake,
// well-separated addresses: nothing is dereferenced. Exit code 0 = all passed.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <random>
#include <vector>

#include "lora_mi355x.h"
#include "stubs.hpp"

namespace {

int failures = 0;

#define EXPECT(cond)                                                                \
  do {                                                                              \
    if (!(cond)) {                                                                  \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                                   \
    }                                                                               \
  } while (0)

// fake device addresses, 4 GiB apart, 256-byte aligned
void* at(int i) { return reinterpret_cast<void*>(uintptr_t(0x1000000000ull) + uintptr_t(i) * 0x100000000ull); }
char* X = static_cast<char*>(at(0));
char* W = static_cast<char*>(at(1));
char* Y = static_cast<char*>(at(2));
char* A = static_cast<char*>(at(3));
char* B = static_cast<char*>(at(4));
char* BIAS = static_cast<char*>(at(5));
char* WS = static_cast<char*>(at(6));
const double NaN = std::numeric_limits<double>::quiet_NaN();
const double Inf = std::numeric_limits<double>::infinity();

int fwd(int64_t T, int64_t K, int64_t N, int32_t r, int adt, int act, int q, size_t wsb, void* x = X, void* y = Y,
        double alpha = 16.0, double st = 1.0, double rs = 1.0, void* a = A, void* b = B, int64_t ldx = -1,
        int64_t ldy = -1) {
  stub::rec.ws_lo = reinterpret_cast<uintptr_t>(WS);
  stub::rec.ws_hi = stub::rec.ws_lo + wsb;
  return lora_linear_fwd(x, T, K, ldx < 0 ? K : ldx, W, N, BIAS, a, b, r, adt, alpha, st, rs, y, ldy < 0 ? N : ldy,
                         act, q, WS, wsb, nullptr);
}

void test_linear() {
  const size_t big = size_t(1) << 40;
  EXPECT(fwd(0, 128, 96, 8, LORA_BF16, LORA_BF16, LORA_LOSSLESS, 0) == LORA_OK);
  EXPECT(fwd(-1, 128, 96, 8, LORA_BF16, LORA_BF16, LORA_LOSSLESS, big) == LORA_ERR_SHAPE);
  EXPECT(fwd(64, 128, 96, 8, LORA_BF16, LORA_BF16, LORA_LOSSLESS, big, nullptr) == LORA_ERR_NULL_PTR);
  EXPECT(fwd(64, 128, 96, 8, LORA_BF16, LORA_F32, LORA_LOSSLESS, big) == LORA_ERR_DTYPE);
  EXPECT(fwd(64, 128, 96, 8, 7, LORA_BF16, LORA_LOSSLESS, big) == LORA_ERR_DTYPE);
  EXPECT(fwd(64, 128, 96, 8, LORA_BF16, LORA_BF16, 5, big) == LORA_ERR_UNSUPPORTED);
  EXPECT(fwd(64, 128, 96, 8, LORA_BF16, LORA_BF16, LORA_LOSSLESS, big, X, Y, NaN) == LORA_ERR_NONFINITE);
  EXPECT(fwd(64, 128, 96, 8, LORA_BF16, LORA_BF16, LORA_LOSSLESS, big, X, Y, 1.0, Inf) == LORA_ERR_NONFINITE);
  EXPECT(fwd(64, 128, 96, 8, LORA_BF16, LORA_BF16, LORA_LOSSLESS, big, X, Y, 1e300, 1e300) == LORA_ERR_NONFINITE);
  EXPECT(fwd(64, 128, 96, 0, LORA_BF16, LORA_BF16, LORA_LOSSLESS, big) == LORA_ERR_SHAPE);
  EXPECT(fwd(64, 128, 96, 2000, LORA_BF16, LORA_BF16, LORA_LOSSLESS, big) == LORA_ERR_UNSUPPORTED);
  EXPECT(fwd(64, 128, 96, 8, LORA_BF16, LORA_BF16, LORA_LOSSLESS, big, X + 2) == LORA_ERR_ALIGN);
  EXPECT(fwd(64, 128, 96, 8, LORA_BF16, LORA_BF16, LORA_LOSSLESS, big, X, X) == LORA_ERR_OVERLAP);
  EXPECT(fwd(64, 128, 96, 8, LORA_BF16, LORA_BF16, LORA_LOSSLESS, 16) == LORA_ERR_WORKSPACE);
  EXPECT(fwd(64, 128, 96, 8, LORA_BF16, LORA_BF16, LORA_LOSSLESS, big, X, Y, 1.0, 1.0, 1.0, A, nullptr) ==
         LORA_ERR_NULL_PTR);
  EXPECT(fwd(64, 100, 96, 8, LORA_BF16, LORA_BF16, LORA_LOSSLESS, big, X, Y, 1.0, 1.0, 1.0, A, B, 99) ==
         LORA_ERR_SHAPE);
  // a valid call reaches the launcher (the stub reports LORA_ERR_HIP)
  const int before = stub::rec.lossless;
  EXPECT(fwd(64, 128, 96, 8, LORA_BF16, LORA_BF16, LORA_LOSSLESS, big) == LORA_ERR_HIP);
  EXPECT(stub::rec.lossless == before + 1);
  EXPECT(fwd(64, 128, 96, 8, LORA_F32, LORA_F32, LORA_EXACT, big) == LORA_ERR_HIP);
  // phase entry point: phase and tile ranges
  int32_t rk = 8;
  const size_t need = lora_linear_workspace_size(300, 256, 520, &rk, 1, LORA_BF16, LORA_LOSSLESS);
  stub::rec.ws_lo = reinterpret_cast<uintptr_t>(WS);
  stub::rec.ws_hi = stub::rec.ws_lo + need;
  for (int ph = -1; ph <= 3; ++ph)
    for (int tile = -1; tile <= 3; ++tile) {
      const int st = lora_linear_fwd_phase(ph, tile, X, 300, 256, 256, W, 520, BIAS, A, B, 8, LORA_BF16, 16.0, 1.0,
                                           1.0, Y, 520, LORA_BF16, LORA_LOSSLESS, WS, need, nullptr);
      const bool ok = ph >= 0 && ph <= 2 && tile >= 0 && tile <= 2;
      EXPECT(st == (ok ? LORA_ERR_HIP : LORA_ERR_UNSUPPORTED));
      if (ok) EXPECT(stub::rec.last_phase == ph && stub::rec.last_tile == tile);
    }
}

void test_groups_and_adapters() {
  const size_t big = size_t(1) << 40;
  stub::rec.ws_lo = reinterpret_cast<uintptr_t>(WS);
  stub::rec.ws_hi = stub::rec.ws_lo + big;
  lora_group g[9];
  for (int i = 0; i < 9; ++i) g[i] = lora_group{A + i * 0x1000000, B + i * 0x1000000, 8, 0, 8.0, 100 * i, 100};
  EXPECT(lora_linear_stacked_fwd(X, 64, 128, 128, W, 300, nullptr, g, 3, LORA_BF16, 1.0, 1.0, Y, 300, LORA_BF16,
                                 LORA_LOSSLESS, WS, big, nullptr) == LORA_ERR_HIP);
  EXPECT(lora_linear_stacked_fwd(X, 64, 128, 128, W, 300, nullptr, g, 9, LORA_BF16, 1.0, 1.0, Y, 900, LORA_BF16,
                                 LORA_LOSSLESS, WS, big, nullptr) == LORA_ERR_UNSUPPORTED);
  EXPECT(lora_linear_stacked_fwd(X, 64, 128, 128, W, 300, nullptr, nullptr, 2, LORA_BF16, 1.0, 1.0, Y, 300,
                                 LORA_BF16, LORA_LOSSLESS, WS, big, nullptr) == LORA_ERR_NULL_PTR);
  g[1].col_offset = 50;  // overlaps group 0
  EXPECT(lora_linear_stacked_fwd(X, 64, 128, 128, W, 300, nullptr, g, 3, LORA_BF16, 1.0, 1.0, Y, 300, LORA_BF16,
                                 LORA_LOSSLESS, WS, big, nullptr) == LORA_ERR_SHAPE);
  lora_adapter ad[3];
  for (int i = 0; i < 3; ++i)
    ad[i] = lora_adapter{A + i * 0x1000000, B + i * 0x1000000, i == 1 ? BIAS : nullptr, 8, 0, 8.0, 0.5, 0, 300};
  // overlapping ranges are allowed for several adapters; the legacy vector needs the fp32 front vector
  const size_t mneed = lora_linear_multi_workspace_size(70, 128, 300, ad, 3, LORA_BF16, LORA_LOSSLESS);
  stub::rec.ws_hi = stub::rec.ws_lo + mneed;
  const int b32 = stub::rec.bias32;
  EXPECT(lora_linear_multi_fwd(X, 70, 128, 128, W, 300, nullptr, ad, 3, LORA_BF16, 1.0, Y, 300, LORA_BF16,
                               LORA_LOSSLESS, WS, mneed, nullptr) == LORA_ERR_HIP);
  EXPECT(stub::rec.bias32 == b32 + 1);
  ad[2].B_bias = BIAS;
  ad[2].A = nullptr;
  EXPECT(lora_linear_multi_fwd(X, 70, 128, 128, W, 300, nullptr, ad, 3, LORA_BF16, 1.0, Y, 300, LORA_BF16,
                               LORA_LOSSLESS, WS, big, nullptr) == LORA_ERR_NULL_PTR);
  ad[2].A = A + 2 * 0x1000000;
  {  // 64 tokens, 8 adapters of rank 1024 with 7 at strength 0: the active one takes the few-token
     // layout, which the query must cover although all the ranks together exceed its limit
    lora_adapter big8[8];
    int32_t r8[8];
    for (int i = 0; i < 8; ++i) {
      big8[i] = lora_adapter{A + i * 0x10000000, B + i * 0x10000000, nullptr, 1024, 0, 1024.0, i == 3 ? 1.0 : 0.0,
                             0, 8960};
      r8[i] = 1024;
    }
    const size_t q8 = lora_linear_workspace_size(64, 8960, 8960, r8, 8, LORA_BF16, LORA_LOSSLESS);
    EXPECT(lora_linear_multi_workspace_size(64, 8960, 8960, big8, 8, LORA_BF16, LORA_LOSSLESS) >= q8);
    stub::rec.ws_hi = stub::rec.ws_lo + q8;
    EXPECT(lora_linear_multi_fwd(X, 64, 8960, 8960, W, 8960, nullptr, big8, 8, LORA_BF16, 1.0, Y, 8960, LORA_BF16,
                                 LORA_LOSSLESS, WS, q8, nullptr) == LORA_ERR_HIP);
    stub::rec.ws_hi = stub::rec.ws_lo + big;
  }
  ad[1].strength = 1e30;  // finite s (alpha/rank = 1), but strength . request_scale of the legacy vector overflows
  EXPECT(lora_linear_multi_fwd(X, 70, 128, 128, W, 300, nullptr, ad, 3, LORA_BF16, 1e10, Y, 300, LORA_BF16,
                               LORA_LOSSLESS, WS, big, nullptr) == LORA_ERR_NONFINITE);
}

void test_nf4_patch_merge_bwd() {
  const size_t big = size_t(1) << 40;
  stub::rec.ws_lo = reinterpret_cast<uintptr_t>(WS);
  stub::rec.ws_hi = stub::rec.ws_lo + big;
  const uint8_t* codes = reinterpret_cast<const uint8_t*>(W);
  const float* am = reinterpret_cast<const float*>(at(7));
  const float* cb = reinterpret_cast<const float*>(at(8));
  EXPECT(lora_linear_nf4_fwd(X, 300, 256, 256, codes, am, cb, 32, 520, nullptr, A, B, 16, LORA_BF16, 32.0, 1.0, 1.0,
                             Y, 520, LORA_LOSSLESS, WS, big, nullptr) == LORA_ERR_UNSUPPORTED);
  EXPECT(lora_linear_nf4_fwd(X, 300, 200, 200, codes, am, cb, 64, 520, nullptr, A, B, 16, LORA_BF16, 32.0, 1.0, 1.0,
                             Y, 520, LORA_LOSSLESS, WS, big, nullptr) == LORA_ERR_SHAPE);
  EXPECT(lora_linear_nf4_fwd(X, 300, 256, 256, nullptr, am, cb, 64, 520, nullptr, A, B, 16, LORA_BF16, 32.0, 1.0,
                             1.0, Y, 520, LORA_LOSSLESS, WS, big, nullptr) == LORA_ERR_NULL_PTR);
  for (int64_t T : {1, 64, 65, 300}) {
    for (int adt : {LORA_BF16, LORA_F32}) {
      const size_t need = lora_linear_nf4_workspace_size(T, 256, 520, 16, adt, LORA_LOSSLESS);
      stub::rec.ws_hi = stub::rec.ws_lo + need;
      EXPECT(lora_linear_nf4_fwd(X, T, 256, 256, codes, am, cb, 64, 520, nullptr, A, B, 16, adt, 32.0, 1.0, 1.0, Y,
                                 520, LORA_LOSSLESS, WS, need, nullptr) == LORA_ERR_HIP);
    }
  }
  // where the 4-bit weight is dequantized: an unknown choice, the in-GEMM form without a bf16
  // adapter of a rank that is a multiple of 8, and the workspace each choice needs (the in-GEMM
  // form none of the panel)
  stub::rec.ws_hi = stub::rec.ws_lo + big;
  EXPECT(lora_linear_nf4_fwd_ex(X, 300, 256, 256, codes, am, cb, 64, 520, nullptr, A, B, 16, LORA_BF16, 32.0, 1.0,
                                1.0, Y, 520, LORA_LOSSLESS, 3, WS, big, nullptr) == LORA_ERR_UNSUPPORTED);
  EXPECT(lora_linear_nf4_fwd_ex(X, 300, 256, 256, codes, am, cb, 64, 520, nullptr, A, B, 16, LORA_F32, 32.0, 1.0,
                                1.0, Y, 520, LORA_LOSSLESS, LORA_NF4_IN_GEMM, WS, big, nullptr) == LORA_ERR_UNSUPPORTED);
  EXPECT(lora_linear_nf4_fwd_ex(X, 300, 256, 256, codes, am, cb, 64, 520, nullptr, A, B, 12, LORA_BF16, 32.0, 1.0,
                                1.0, Y, 520, LORA_LOSSLESS, LORA_NF4_IN_GEMM, WS, big, nullptr) == LORA_ERR_UNSUPPORTED);
  {
    const int32_t r16 = 16;
    const size_t small = lora_linear_workspace_size(300, 256, 520, &r16, 1, LORA_BF16, LORA_LOSSLESS);
    stub::rec.ws_hi = stub::rec.ws_lo + small;
    EXPECT(lora_linear_nf4_fwd_ex(X, 300, 256, 256, codes, am, cb, 64, 520, nullptr, A, B, 16, LORA_BF16, 32.0, 1.0,
                                  1.0, Y, 520, LORA_LOSSLESS, LORA_NF4_IN_GEMM, WS, small, nullptr) == LORA_ERR_HIP);
    EXPECT(lora_linear_nf4_fwd_ex(X, 300, 256, 256, codes, am, cb, 64, 520, nullptr, A, B, 16, LORA_BF16, 32.0, 1.0,
                                  1.0, Y, 520, LORA_LOSSLESS, LORA_NF4_PANEL, WS, small, nullptr) ==
           LORA_ERR_WORKSPACE);
  }
  const int64_t s34[2] = {3, 4}, s43[2] = {4, 3}, s12[1] = {12};
  EXPECT(dense_patch_apply(Y, LORA_BF16, s34, 2, X, LORA_BF16, s34, 2, 0.8, LORA_PATCH_ADD, nullptr) == LORA_ERR_HIP);
  EXPECT(dense_patch_apply(Y, LORA_BF16, s34, 2, X, LORA_BF16, s43, 2, 0.8, LORA_PATCH_ADD, nullptr) ==
         LORA_ERR_SHAPE);
  EXPECT(dense_patch_apply(Y, LORA_BF16, s34, 2, X, LORA_BF16, s12, 1, 0.8, LORA_PATCH_ADD, nullptr) ==
         LORA_ERR_SHAPE);
  EXPECT(dense_patch_apply(Y, LORA_BF16, s34, 2, X, LORA_BF16, s34, 2, NaN, LORA_PATCH_ADD, nullptr) ==
         LORA_ERR_NONFINITE);
  EXPECT(dense_patch_apply(Y, LORA_BF16, s34, 2, Y + 4, LORA_BF16, s34, 2, 0.8, LORA_PATCH_ADD, nullptr) ==
         LORA_ERR_OVERLAP);
  EXPECT(dense_patch_apply(Y, LORA_BF16, s34, 2, X, LORA_BF16, s34, 2, 0.8, 9, nullptr) == LORA_ERR_UNSUPPORTED);
  EXPECT(lora_merge_apply(W, LORA_BF16, 300, 128, A, B, 8, LORA_BF16, 8.0, 0.7, LORA_LOSSLESS, nullptr) ==
         LORA_ERR_HIP);
  EXPECT(lora_merge_apply(W, LORA_BF16, 300, 128, A, B, 8, LORA_BF16, 8.0, 0.0, LORA_LOSSLESS, nullptr) == LORA_OK);
  EXPECT(lora_merge_apply(W, LORA_BF16, 300, 128, W + 2, B, 8, LORA_BF16, 8.0, 0.7, LORA_EXACT, nullptr) ==
         LORA_ERR_OVERLAP);
  EXPECT(lora_merge_apply(W, LORA_BF16, 300, 130, A, B, 8, LORA_BF16, 8.0, 0.7, LORA_LOSSLESS, nullptr) ==
         LORA_ERR_ALIGN);
  float* dA = reinterpret_cast<float*>(at(9));
  float* dB = reinterpret_cast<float*>(at(10));
  float* db = reinterpret_cast<float*>(at(11));
  for (int want_dx : {0, 1}) {
    const size_t need = lora_linear_bwd_workspace_size(700, 256, 520, 24, want_dx);
    stub::rec.ws_hi = stub::rec.ws_lo + need;
    EXPECT(lora_linear_bwd(X, 700, 256, 256, W, 520, A, B, 24, 48.0, 0.8, 0.7, BIAS, 520, want_dx ? Y : nullptr, 256,
                           dA, dB, db, nullptr, 0, WS, need, nullptr) == LORA_ERR_HIP);
    EXPECT(lora_linear_bwd(X, 700, 256, 256, W, 520, A, B, 24, 48.0, 0.8, 0.7, BIAS, 520, want_dx ? Y : nullptr, 256,
                           dA, dB, db, nullptr, 0, WS, need - 1, nullptr) == LORA_ERR_WORKSPACE);
    // the forward's t~ given (rank 24 pads to 64 columns): the same launches without its producer
    EXPECT(lora_linear_bwd(X, 700, 256, 256, W, 520, A, B, 24, 48.0, 0.8, 0.7, BIAS, 520, want_dx ? Y : nullptr, 256,
                           dA, dB, db, at(12), 64, WS, need, nullptr) == LORA_ERR_HIP);
    EXPECT(lora_linear_bwd(X, 700, 256, 256, W, 520, A, B, 24, 48.0, 0.8, 0.7, BIAS, 520, want_dx ? Y : nullptr, 256,
                           dA, dB, db, at(12), 63, WS, need, nullptr) == LORA_ERR_SHAPE);
  }
  EXPECT(lora_linear_bwd(X, 700, 256, 256, W, 520, A, B, 24, 48.0, 0.8, 0.7, BIAS, 520, Y, 256, dA, dA, db, nullptr, 0,
                         WS, big, nullptr) == LORA_ERR_OVERLAP);
}

// Random valid calls: sized by the documented query, every call passes the workspace
// check and every region the stub sees lies inside the workspace.
void test_random_calls() {
  std::mt19937_64 rng(12345);
  auto pick = [&](std::initializer_list<int64_t> v) { return *(v.begin() + rng() % v.size()); };
  for (int it = 0; it < 4000; ++it) {
    const int64_t T = pick({1, 7, 33, 64, 65, 128, 300, 2048, 4352, 18871, 32760});
    const int64_t K = pick({64, 128, 192, 1536, 3072, 8960});
    const int64_t N = pick({1, 96, 300, 1536, 8960});
    const int q = rng() % 4 == 0 ? LORA_EXACT : LORA_LOSSLESS;
    const int act = rng() % 5 == 0 ? LORA_F32 : LORA_BF16;
    const int adt = act == LORA_F32 ? LORA_F32 : (rng() % 3 == 0 ? LORA_F32 : LORA_BF16);
    const int ng = 1 + static_cast<int>(rng() % 4);
    const bool multi = rng() % 2 == 0;
    lora_adapter ad[4];
    int32_t ranks[4];
    for (int i = 0; i < ng; ++i) {
      const int32_t r = static_cast<int32_t>(pick({1, 8, 16, 24, 64, 100, 128, 200}));
      const int64_t w = N / ng;
      const int64_t off = multi ? 0 : w * i;
      const int64_t nc = multi ? N : (i + 1 == ng ? N - off : w);
      const double st = rng() % 4 == 0 ? 0.0 : 0.8;
      ad[i] = lora_adapter{A + i * 0x1000000, B + i * 0x1000000, (multi && rng() % 2) ? BIAS : nullptr, r, 0,
                           2.0 * r, st, off, nc > 0 ? nc : 1};
      ranks[i] = r;
    }
    if (!multi && N / ng < 1) continue;
    size_t need = multi ? lora_linear_multi_workspace_size(T, K, N, ad, ng, adt, q)
                        : lora_linear_workspace_size(T, K, N, ranks, ng, adt, q);
    stub::rec.ws_lo = reinterpret_cast<uintptr_t>(WS);
    stub::rec.ws_hi = stub::rec.ws_lo + need;
    int st;
    if (multi) {
      st = lora_linear_multi_fwd(X, T, K, K, W, N, BIAS, ad, ng, adt, 0.7, Y, N, act, q, WS, need, nullptr);
    } else {
      lora_group g[4];
      for (int i = 0; i < ng; ++i)
        g[i] = lora_group{ad[i].A, ad[i].B, ad[i].rank, 0, ad[i].alpha, ad[i].col_offset, ad[i].n_cols};
      st = lora_linear_stacked_fwd(X, T, K, K, W, N, BIAS, g, ng, adt, ad[0].strength, 0.7, Y, N, act, q, WS, need,
                                   nullptr);
    }
    if (st != LORA_ERR_HIP) {
      std::fprintf(stderr, "random call %d: T=%ld K=%ld N=%ld groups=%d multi=%d act=%d adt=%d q=%d -> status %d\n",
                   it, (long)T, (long)K, (long)N, ng, (int)multi, act, adt, q, st);
      ++failures;
    }
  }
  // workspace queries at the extremes do not overflow or trap
  int32_t r = 1024;
  (void)lora_linear_workspace_size(int64_t(1) << 31, int64_t(1) << 20, int64_t(1) << 20, &r, 1, LORA_F32,
                                   LORA_LOSSLESS);
  (void)lora_linear_nf4_workspace_size(int64_t(1) << 31, int64_t(1) << 20, int64_t(1) << 20, 1024, LORA_F32,
                                       LORA_LOSSLESS);
  (void)lora_linear_bwd_workspace_size(int64_t(1) << 31, int64_t(1) << 20, int64_t(1) << 20, 1024, 1);
  EXPECT(lora_linear_workspace_size(0, 128, 96, &r, 1, LORA_BF16, LORA_LOSSLESS) == 0);
  EXPECT(lora_linear_workspace_size(64, 128, 96, nullptr, 2, LORA_BF16, LORA_LOSSLESS) == 0);
}

}  // namespace

int main() {
  test_linear();
  test_groups_and_adapters();
  test_nf4_patch_merge_bwd();
  test_random_calls();
  for (int s = -1; s <= 10; ++s) EXPECT(lora_status_string(s) != nullptr);
  std::printf("validation layer under sanitizers: %d failures (launcher stand-ins reached: %d lossless, %d exact, "
              "%d bias, %d merge, %d patch, %d backward)\n",
              failures, stub::rec.lossless, stub::rec.exact, stub::rec.bias32, stub::rec.merge, stub::rec.patch,
              stub::rec.bwd);
  return failures == 0 ? 0 : 1;
}
