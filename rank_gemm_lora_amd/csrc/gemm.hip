// Lossless tier of the fused LoRA linear on gfx950 (CDNA4).
//
// SGLang PR #43501 ("Add the dynamic LoRA delta inside the second GEMM",
// Modifications): the combined scale (alpha/rank . strength . request scale)
// multiplies the rank-wide intermediate x.A^T, and the second LoRA product is
// accumulated straight onto the base output, so the [tokens, out] delta never
// exists. Here the accumulation happens inside the base GEMM itself:
//
//   lora_down_kernel   t~[T, r] = RN_adt( s . x.A^T )      (fp32 accumulate, one rounding)
//   fused_gemm_kernel  acc = x.W^T  (K loop over `in`)
//                      acc += t~.B^T (K-extension over the rank, same accumulator)
//                      y = RN_dt(acc + b)                    (bias in the epilogue)
//
// Both kernels are NT GEMMs with K-contiguous operands, which is the native
// operand layout of the MFMA units: lane l of v_mfma_f32_32x32x16_bf16 takes 8
// consecutive k of one row of each operand. The MFMA "A" operand carries
// output columns (rows of W / B / A), the "B" operand carries tokens (rows of
// x / t~), so each lane ends with 4 consecutive output columns of one token
// and stores them as one 8-byte (bf16) or 16-byte (fp32) write.
//
// Staging: every operand row is staged 128 bytes per K step (64 bf16 or 32
// fp32) into LDS, with the 16-byte chunk index XOR-swizzled by row so the
// 16-byte LDS reads of a wave spread over all banks. x and W tiles are copied
// global->LDS directly by buffer_load ... lds (no VGPR round trip), double
// buffered; out-of-range rows and K tails read as zero through the buffer
// resource's range check.
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "launch.hpp"

namespace lora {
namespace {

constexpr int kRowBytes = 128;  // staged bytes per operand row per K step
constexpr int kChunks = 8;      // 16-byte chunks per staged row
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kChunks + (chunk ^ ((row >> 1) & 7));
}

template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN, WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int NI = WN / 32, NJ = WM / 32;
  static constexpr int X_BYTES = BM * kRowBytes, W_BYTES = BN * kRowBytes;
  static constexpr int STAGE_BYTES = X_BYTES + W_BYTES;
  static constexpr int GROUP_M = 4;  // m-tiles enumerated together (L2 reuse of W)
};

// Physical workgroup ids are dealt round-robin to the 8 XCDs. Remap so each XCD
// receives a contiguous run of logical tiles (tiles sharing x rows / W rows then
// share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int pid, int G) {
  const int q = G / 8, rem = G % 8;
  const int xcd = pid % 8, idx = pid / 8;
  return (xcd < rem) ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

// Copy ROWS x 128 bytes (bytes [kb0, kb0 + 128) of each row) into a swizzled LDS
// tile with buffer_load_dwordx4 ... lds. Rows >= rows_valid and bytes >= kb_valid
// are out of the resource's range and arrive as zeros.
template <int ROWS, int THREADS>
__device__ __forceinline__ void dma_stage(char* lds_tile, __amdgpu_buffer_rsrc_t rsrc,
                                          uint32_t ld_bytes, int rows_valid, int kb0, int kb_valid) {
  constexpr int SLOTS = ROWS * kChunks;
  static_assert(SLOTS % THREADS == 0, "tile not divisible among threads");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int WAVES = THREADS / 64;
#pragma unroll
  for (int it = 0; it < SLOTS / THREADS; ++it) {
    const int slot0 = (it * WAVES + wave) * 64;  // wave-uniform LDS destination
    const int s = slot0 + lane;
    const int row = s >> 3;
    const int c = (s & 7) ^ ((row >> 1) & 7);
    const int kb = kb0 + c * 16;
    const uint32_t voff = (row < rows_valid && kb < kb_valid)
                              ? static_cast<uint32_t>(row) * ld_bytes + static_cast<uint32_t>(kb)
                              : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds_tile + slot0 * 16), 16, voff, 0, 0, 0);
  }
}

// One 128-byte K step of MFMA work from two swizzled LDS tiles.
template <class C, typename T>
struct Mma;

template <class C>
struct Mma<C, bf16_bits> {
  __device__ __forceinline__ static void stage(f32x16 (&acc)[C::NI][C::NJ], const char* lw, const char* lx,
                                               int wn0, int wm0, int lane) {
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 a[C::NI], b[C::NJ];
#pragma unroll
      for (int i = 0; i < C::NI; ++i) a[i] = *(const bf16x8*)(lw + swz(wn0 + i * 32 + r, kk * 2 + h) * 16);
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) b[j] = *(const bf16x8*)(lx + swz(wm0 + j * 32 + r, kk * 2 + h) * 16);
#pragma unroll
      for (int i = 0; i < C::NI; ++i)
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
};

template <class C>
struct Mma<C, float> {
  // Lane half h takes logical k = h*16 + s (s = 0..15) of the 32 staged k, the
  // same for both operands, so the sum over k is the full dot product.
  __device__ __forceinline__ static void stage(f32x16 (&acc)[C::NI][C::NJ], const char* lw, const char* lx,
                                               int wn0, int wm0, int lane) {
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      f32x4 a[C::NI], b[C::NJ];
#pragma unroll
      for (int i = 0; i < C::NI; ++i) a[i] = *(const f32x4*)(lw + swz(wn0 + i * 32 + r, h * 4 + c4) * 16);
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) b[j] = *(const f32x4*)(lx + swz(wm0 + j * 32 + r, h * 4 + c4) * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < C::NI; ++i)
#pragma unroll
          for (int j = 0; j < C::NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
    }
  }
};

// Stage BN rows of the LoRA B matrix (group g) as the W-side operand of one
// K-extension step: row n of the tile is output column n0 + n; it holds
// B_g[n0 + n - col_off][q0 .. q0 + 128/e) for columns inside the group and
// q < rank, zero elsewhere. Goes through VGPRs (B's row stride need not be a
// multiple of 16 bytes).
template <int ROWS, int THREADS, typename TL>
__device__ __forceinline__ void stage_lora_b(char* lds_tile, const GroupDev& g, int64_t n0, int rows_valid,
                                             int q0) {
  constexpr int EPC = 16 / sizeof(TL);  // elements per 16-byte chunk
  constexpr int SLOTS = ROWS * kChunks;
  const TL* B = static_cast<const TL*>(g.B);
  const bool vec_ok = ((g.rank * static_cast<int>(sizeof(TL))) % 16) == 0;
#pragma unroll
  for (int it = 0; it < SLOTS / THREADS; ++it) {
    const int s = it * THREADS + threadIdx.x;
    const int row = s >> 3, c = s & 7;
    const int64_t n = n0 + row - g.col_off;  // row of B_g
    const int q = q0 + c * EPC;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < rows_valid && n >= 0 && n < g.n_cols && q < g.rank) {
      const TL* src = B + n * g.rank + q;
      if (vec_ok && q + EPC <= g.rank) {
        v = *reinterpret_cast<const u32x4*>(src);
      } else {
        TL tmp[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) tmp[e] = (q + e < g.rank) ? src[e] : TL(0);
        v = *reinterpret_cast<const u32x4*>(tmp);
      }
    }
    *reinterpret_cast<u32x4*>(lds_tile + swz(row, c) * 16) = v;
  }
}

template <class C, typename TA>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[C::NI][C::NJ], const LinearProblem& p, int64_t m0,
                                         int64_t n0, int wm0, int wn0, int lane) {
  const int r = lane & 31, h = lane >> 5;
  const TA* bias = static_cast<const TA*>(p.bias);
  TA* y = static_cast<TA*>(p.y);
  // 4 consecutive outputs go out as one 8-byte (bf16) / 16-byte (fp32) store when
  // every row start keeps that alignment; otherwise element by element.
  const bool vec_store = (p.ldy % 4 == 0) && (reinterpret_cast<uintptr_t>(p.y) % (4 * sizeof(TA)) == 0);
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int64_t n = n0 + wn0 + i * 32 + gq * 8 + h * 4;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (p.bias32 != nullptr) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < p.N) bv[e] = p.bias32[n + e];
      } else if (bias != nullptr) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (n + e < p.N) {
            if constexpr (sizeof(TA) == 2) bv[e] = bf16_to_f32(bias[n + e]);
            else bv[e] = bias[n + e];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) {
        const int64_t m = m0 + wm0 + j * 32 + r;
        if (m >= p.T) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][gq * 4 + e] + bv[e];
        TA* dst = y + m * p.ldy + n;
        if (vec_store && n + 3 < p.N) {
          if constexpr (sizeof(TA) == 2) {
            uint2 w;
            w.x = pack_bf16x2(v[0], v[1]);
            w.y = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<uint2*>(dst) = w;
          } else {
            *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (n + e < p.N) {
              if constexpr (sizeof(TA) == 2) dst[e] = f32_to_bf16_rne(v[e]);
              else dst[e] = v[e];
            }
          }
        }
      }
    }
  }
}

template <class C, typename TA, typename TL>
__global__ __launch_bounds__(C::THREADS) void fused_gemm_kernel(LinearProblem p, int mt, int nt) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::STAGE_BYTES];

  const int G = mt * nt;
  const int L = xcd_remap(blockIdx.x, G);
  const int gsize = C::GROUP_M * nt;
  const int grp = L / gsize;
  const int first_m = grp * C::GROUP_M;
  const int gm = min(C::GROUP_M, mt - first_m);
  const int within = L - grp * gsize;
  const int m_idx = first_m + within % gm;
  const int n_idx = within / gm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave % C::WAVES_M) * C::WM;
  const int wn0 = (wave / C::WAVES_M) * C::WN;
  const int64_t m0 = static_cast<int64_t>(m_idx) * C::BM;
  const int64_t n0 = static_cast<int64_t>(n_idx) * C::BN;
  const int rows_m = static_cast<int>(min<int64_t>(C::BM, p.T - m0));
  const int rows_n = static_cast<int>(min<int64_t>(C::BN, p.N - n0));

  f32x16 acc[C::NI][C::NJ];
#pragma unroll
  for (int i = 0; i < C::NI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // stage buffer b: x tile at smem + b * STAGE_BYTES, W tile right after it
  auto bufx = [&](int b) { return smem + b * C::STAGE_BYTES; };
  auto bufw = [&](int b) { return smem + b * C::STAGE_BYTES + C::X_BYTES; };

  // ---------------- base GEMM: K loop over `in`
  constexpr int EA = sizeof(TA);
  const int kb_total = static_cast<int>(p.K * EA);
  const int nk = (kb_total + kRowBytes - 1) / kRowBytes;
  const uint32_t ldx_b = static_cast<uint32_t>(p.ldx * EA);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(static_cast<const char*>(p.x) + m0 * p.ldx * EA, static_cast<uint32_t>(rows_m) * ldx_b);

  const uint32_t ldw_b = static_cast<uint32_t>(p.K * EA);
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(static_cast<const char*>(p.W) + n0 * p.K * EA, static_cast<uint32_t>(rows_n) * ldw_b);
  dma_stage<C::BM, C::THREADS>(bufx(0), xr, ldx_b, rows_m, 0, kb_total);
  dma_stage<C::BN, C::THREADS>(bufw(0), wr, ldw_b, rows_n, 0, kb_total);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmem();
    __syncthreads();
    if (kt + 1 < nk) {
      dma_stage<C::BM, C::THREADS>(bufx((kt + 1) & 1), xr, ldx_b, rows_m, (kt + 1) * kRowBytes, kb_total);
      dma_stage<C::BN, C::THREADS>(bufw((kt + 1) & 1), wr, ldw_b, rows_n, (kt + 1) * kRowBytes, kb_total);
    }
    Mma<C, TA>::stage(acc, bufw(kt & 1), bufx(kt & 1), wn0, wm0, lane);
  }

  // ---------------- K-extension: acc += t~ . B^T for every group touching this tile
  constexpr int EL = sizeof(TL);
  const uint32_t ldt_b = static_cast<uint32_t>(p.ldt * EL);
  for (int gi = 0; gi < p.n_groups; ++gi) {
    const GroupDev& g = p.g[gi];
    if (g.col_off >= n0 + rows_n || g.col_off + g.n_cols <= n0) continue;
    const __amdgpu_buffer_rsrc_t tr = make_rsrc(
        static_cast<const char*>(p.work) + (m0 * p.ldt + g.t_col) * EL, static_cast<uint32_t>(rows_m) * ldt_b);
    const int nst = g.r_pad * EL / kRowBytes;
    for (int st = 0; st < nst; ++st) {
      __syncthreads();  // every wave is done reading the previous stage
      dma_stage<C::BM, C::THREADS>(bufx(0), tr, ldt_b, rows_m, st * kRowBytes, g.r_pad * EL);
      stage_lora_b<C::BN, C::THREADS, TL>(bufw(0), g, n0, rows_n, st * (kRowBytes / EL));
      wait_vmem();
      __syncthreads();
      Mma<C, TL>::stage(acc, bufw(0), bufx(0), wn0, wm0, lane);
    }
  }

  // ---------------- epilogue: + bias (fp32), one rounding, store
  epilogue<C, TA>(acc, p, m0, n0, wm0, wn0, lane);
}

// ---------------------------------------------------------------------------
// t~[m, t_col + q] = RN_adt( s . sum_k x[m,k] A_g[q,k] ), zero for rank <= q < r_pad.
// Grid: (ceil(T / 256), n_groups, ceil(max r_pad / 128)). 4 waves; wave w owns
// tokens [64w, 64w + 64) and all (up to 128) rank columns of the block.
// TX: x element type; CT: compute/adapter type (bf16 MFMA, or fp32 MFMA with x
// widened exactly to fp32).
constexpr int kDownBM = 256;
constexpr int kDownBQ = 128;
using DownCfg = Cfg<kDownBM, kDownBQ, 64, 128>;  // WAVES_M = 4, WAVES_N = 1

template <typename TX, typename CT>
__device__ __forceinline__ void down_load_x(u32x4 (&rx)[8], const TX* x, int64_t ldx, int64_t m0, int rows_m,
                                            int64_t K, int k0) {
  constexpr int EPC = 16 / sizeof(CT);
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int s = it * 256 + threadIdx.x;
    const int row = s >> 3, c = s & 7;
    const int64_t k = k0 + c * EPC;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < rows_m && k < K) {
      const TX* src = x + (m0 + row) * ldx + k;
      if constexpr (sizeof(TX) == sizeof(CT)) {
        v = *reinterpret_cast<const u32x4*>(src);  // K is a multiple of EPC (alignment rule)
      } else {
        // bf16 -> fp32 widening of 4 elements (8 bytes)
        const uint2 w = *reinterpret_cast<const uint2*>(src);
        v = u32x4{w.x << 16, w.x & 0xffff0000u, w.y << 16, w.y & 0xffff0000u};
      }
    }
    rx[it] = v;
  }
}

template <typename CT>
__device__ __forceinline__ void down_load_a(u32x4 (&ra)[4], const GroupDev& g, int q_base, int64_t K, int k0) {
  constexpr int EPC = 16 / sizeof(CT);
  const CT* A = static_cast<const CT*>(g.A);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int s = it * 256 + threadIdx.x;
    const int row = s >> 3, c = s & 7;
    const int q = q_base + row;
    const int64_t k = k0 + c * EPC;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (q < g.rank && k < K) v = *reinterpret_cast<const u32x4*>(A + q * K + k);
    ra[it] = v;
  }
}

template <typename TX, typename CT>
__global__ __launch_bounds__(256) void lora_down_kernel(LinearProblem p) {
  __shared__ __attribute__((aligned(1024))) char lx[kDownBM * kRowBytes];
  __shared__ __attribute__((aligned(1024))) char la[kDownBQ * kRowBytes];
  using C = DownCfg;
  const GroupDev& g = p.g[blockIdx.y];
  const int q_base = blockIdx.z * kDownBQ;
  if (q_base >= g.r_pad) return;
  const int nq = min(kDownBQ, g.r_pad - q_base);
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * kDownBM;
  const int rows_m = static_cast<int>(min<int64_t>(kDownBM, p.T - m0));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = wave * 64;
  const TX* x = static_cast<const TX*>(p.x);

  f32x16 acc[C::NI][C::NJ];
#pragma unroll
  for (int i = 0; i < C::NI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  constexpr int EPS = kRowBytes / sizeof(CT);  // k per stage
  const int nk = static_cast<int>((p.K + EPS - 1) / EPS);
  u32x4 rx[8], ra[4];
  down_load_x<TX, CT>(rx, x, p.ldx, m0, rows_m, p.K, 0);
  down_load_a<CT>(ra, g, q_base, p.K, 0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int s = it * 256 + threadIdx.x;
      *reinterpret_cast<u32x4*>(lx + swz(s >> 3, s & 7) * 16) = rx[it];
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int s = it * 256 + threadIdx.x;
      *reinterpret_cast<u32x4*>(la + swz(s >> 3, s & 7) * 16) = ra[it];
    }
    __syncthreads();
    if (kt + 1 < nk) {
      down_load_x<TX, CT>(rx, x, p.ldx, m0, rows_m, p.K, (kt + 1) * EPS);
      down_load_a<CT>(ra, g, q_base, p.K, (kt + 1) * EPS);
    }
    Mma<C, CT>::stage(acc, la, lx, 0, wm0, lane);
  }

  // D[i = q][j = token]: lane holds q = i*32 + 8*gq + 4*h + e for token j*32 + r.
  const int r = lane & 31, h = lane >> 5;
  const float s = g.scale;
  const bool unit = (s == 1.0f);
  CT* t = static_cast<CT*>(p.work);
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) {
    const int64_t m = m0 + wm0 + j * 32 + r;
    if (m >= p.T) continue;
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
      if (i * 32 >= nq) continue;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int q = q_base + i * 32 + gq * 8 + h * 4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = unit ? acc[i][j][gq * 4 + e] : acc[i][j][gq * 4 + e] * s;
        CT* dst = t + m * p.ldt + g.t_col + q;
        if constexpr (sizeof(CT) == 2) {
          uint2 w;
          w.x = pack_bf16x2(v[0], v[1]);
          w.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(dst) = w;
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Pipelined kernel for the hot configuration (bf16 activations and adapters,
// dense weight, rank a multiple of 8).
//
// K advances RB bytes of every operand row per stage through a ring of S LDS
// stages filled by buffer_load ... lds; up to S - 1 stages of loads are in
// flight while one is consumed. A stage holds RB / 32 MFMA steps of 16 k whose
// fragments alternate between two register sets; the barrier that publishes
// the next stage sits inside the last step, so LDS latency and the barrier
// hide behind MFMA work. The LoRA K-extension (t~ rows against B rows of every
// group meeting the tile) is simply more stages of the same ring.
namespace pipe {

template <int BM_, int BN_, int WM_, int WN_, int RB_, int S_>
struct PCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, RB = RB_, S = S_;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN, WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int NI = WN / 32, NJ = WM / 32;
  static constexpr int CPR = RB / 16;      // 16-byte chunks per staged row
  static constexpr int RPL = 256 / RB;     // staged rows per 256-byte line of the 64 LDS banks
  static constexpr int KK = RB / 32;       // 16-k MFMA steps per stage
  static constexpr int X_BYTES = BM * RB, STAGE_BYTES = (BM + BN) * RB;
  static constexpr int LPS = (BM + BN) * CPR / THREADS;  // buffer loads per thread per stage
  static constexpr int GROUP_M = 4;
  static_assert(KK % 2 == 0, "fragment sets alternate across stages");
  static_assert((BM * CPR / 64) % WAVES == 0 && (BN * CPR / 64) % WAVES == 0, "uneven load split");
  static_assert(S * STAGE_BYTES <= 160 * 1024, "LDS");
  static_assert((S - 2) * LPS <= 63, "vmcnt range");
};

// Chunk index XORed with (row / RPL) % CPR: the 16-byte reads of 16 consecutive
// rows at one chunk (one quarter of a wave's ds_read_b128) hit distinct banks.
template <class P>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * P::CPR + (chunk ^ ((row / P::RPL) % P::CPR));
}

// Tile rows [row_lo, row_hi) come from source row (row + shift), bytes
// [kb0, kb0 + RB) of it; other rows and bytes >= kb_valid read as zero.
template <class P, int ROWS>
__device__ __forceinline__ void dma(char* lds, __amdgpu_buffer_rsrc_t rsrc, uint32_t ld_bytes, int row_lo,
                                    int row_hi, int shift, int kb0, int kb_valid) {
  constexpr int INSTR = ROWS * P::CPR / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int it = 0; it < INSTR / P::WAVES; ++it) {
    const int slot0 = (it * P::WAVES + wave) * 64;  // wave-uniform LDS destination
    const int sl = slot0 + lane;
    const int row = sl / P::CPR;
    const int c = (sl % P::CPR) ^ ((row / P::RPL) % P::CPR);
    const int kb = kb0 + c * 16;
    const uint32_t voff = (row >= row_lo && row < row_hi && kb < kb_valid)
                              ? static_cast<uint32_t>(row + shift) * ld_bytes + static_cast<uint32_t>(kb)
                              : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + slot0 * 16), 16, voff, 0, 0, 0);
  }
}

template <class P>
struct Frags {
  bf16x8 a[P::NI], b[P::NJ];
};

template <class P>
__device__ __forceinline__ void load_frags(Frags<P>& f, const char* stage, int kk, int wn0, int wm0, int lane) {
  const int r = lane & 31, h = lane >> 5;
  const char* lx = stage;
  const char* lw = stage + P::X_BYTES;
#pragma unroll
  for (int i = 0; i < P::NI; ++i) f.a[i] = *(const bf16x8*)(lw + swz<P>(wn0 + i * 32 + r, kk * 2 + h) * 16);
#pragma unroll
  for (int j = 0; j < P::NJ; ++j) f.b[j] = *(const bf16x8*)(lx + swz<P>(wm0 + j * 32 + r, kk * 2 + h) * 16);
}

template <class P>
__device__ __forceinline__ void mfma_frags(f32x16 (&acc)[P::NI][P::NJ], const Frags<P>& f) {
#pragma unroll
  for (int i = 0; i < P::NI; ++i)
#pragma unroll
    for (int j = 0; j < P::NJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Scheduling hint for a block "NI + NJ fragment reads + NI * NJ MFMAs": the reads
// go out two at a time behind the first MFMAs and complete while the rest run.
template <class P>
__device__ __forceinline__ void interleave_reads_with_mfma() {
  constexpr int R = P::NI + P::NJ, M = P::NI * P::NJ;
#pragma unroll
  for (int i = 0; i < R / 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 DS reads
  }
  __builtin_amdgcn_sched_group_barrier(0x008, M - R / 2, 0);
}

// Cache-policy operand of the buffer intrinsics on gfx950: bit 1 = nt (streaming).
constexpr int kCachePolicyNT = 2;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] bits 3:0, expcnt bits 6:4,
// lgkmcnt bits 11:8, vmcnt[5:4] bits 15:14); counters not named stay at their
// maximum, i.e. are not waited for. Using the builtin (not inline asm) lets the
// compiler's own wait insertion see these waits.
constexpr int waitcnt_vm(int n) { return (n & 0xf) | ((n >> 4) << 14) | 0x70 | 0xf00; }
constexpr int kWaitLgkm0 = 0xc07f;

// Wait until at most `n` stages of this thread's buffer loads are outstanding.
template <int LPS>
__device__ __forceinline__ void wait_stages(int n) {
  if (n >= 4) __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * LPS > 63 ? 63 : 4 * LPS));
  else if (n == 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * LPS > 63 ? 63 : 3 * LPS));
  else if (n == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPS));
  else if (n == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPS));
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// Workgroup barrier without the release/acquire fences of __syncthreads (those
// would also wait for the loads of later stages). LDS reads of this wave are
// complete before it arrives.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// v unchanged, through an empty asm: values computed from it stay where they
// are written instead of being hoisted out of loops into long-lived registers.
// (The asm exists only in the device pass; the host pass has no such operand.)
__device__ __forceinline__ int opaque_int(int v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(v));
#endif
  return v;
}

// Per-lane byte offsets of one operand tile's rows for the buffer_load ... lds
// copies (k offset 0); rows outside [row_lo, row_hi) get an offset past the
// resource range. The k offset of a stage travels in the scalar soffset.
template <class P, int ROWS>
struct TileOffsets {
  static constexpr int N = ROWS * P::CPR / 64 / P::WAVES;
  uint32_t v[N];
  __device__ __forceinline__ void init(uint32_t ld_bytes, int row_lo, int row_hi, int shift) {
    const int lane = opaque_int(threadIdx.x & 63);
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int sl = (it * P::WAVES + wave) * 64 + lane;
      const int row = sl / P::CPR;
      const int c = (sl % P::CPR) ^ ((row / P::RPL) % P::CPR);
      v[it] = (row >= row_lo && row < row_hi) ? static_cast<uint32_t>(row + shift) * ld_bytes + c * 16
                                              : 0x80000000u;
    }
  }
  // One of the N copy instructions of a stage (no K tail).
  __device__ __forceinline__ void load_one(int it, char* lds, __amdgpu_buffer_rsrc_t rsrc, int kb0) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slot0 = (it * P::WAVES + wave) * 64;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + slot0 * 16), 16, v[it], kb0, 0, 0);
  }
  // Copy the stage at byte offset kb0 into lds. With a K tail, chunks at or past
  // kb_valid are redirected out of range as well.
  __device__ __forceinline__ void load(char* lds, __amdgpu_buffer_rsrc_t rsrc, int kb0, bool tail, int kb_valid) const {
    const int lane = opaque_int(threadIdx.x & 63);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // When each copy instruction covers a whole number of swizzle periods of rows
    // the lane's chunk is the same in all of them.
    constexpr bool same_chunk = (P::WAVES * 64 / P::CPR / P::RPL) % P::CPR == 0;
    const int c0 = (lane % P::CPR) ^ (((wave * 64 + lane) / P::CPR / P::RPL) % P::CPR);
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int slot0 = (it * P::WAVES + wave) * 64;
      uint32_t voff = v[it];
      if (tail) {
        int c = c0;
        if (!same_chunk) {
          const int sl = slot0 + lane;
          const int row = sl / P::CPR;
          c = (sl % P::CPR) ^ ((row / P::RPL) % P::CPR);
        }
        if (kb0 + c * 16 >= kb_valid) voff = 0x80000000u;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + slot0 * 16), 16, voff, kb0, 0, 0);
    }
  }
};

template <class P>
__global__ __launch_bounds__(P::THREADS) void gemm_pipe_kernel(LinearProblem p, int mt, int nt) {
  __shared__ __attribute__((aligned(1024))) char smem[P::S * P::STAGE_BYTES];

  const int G = mt * nt;
  const int L = xcd_remap(blockIdx.x, G);
  const int gsize = P::GROUP_M * nt;
  const int grp = L / gsize;
  const int first_m = grp * P::GROUP_M;
  const int gm = min(P::GROUP_M, mt - first_m);
  const int within = L - grp * gsize;
  const int m_idx = first_m + within % gm;
  const int n_idx = within / gm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave % P::WAVES_M) * P::WM;
  const int wn0 = (wave / P::WAVES_M) * P::WN;
  const int64_t m0 = static_cast<int64_t>(m_idx) * P::BM;
  const int64_t n0 = static_cast<int64_t>(n_idx) * P::BN;
  const int rows_m = static_cast<int>(min<int64_t>(P::BM, p.T - m0));
  const int rows_n = static_cast<int>(min<int64_t>(P::BN, p.N - n0));

  // main stages
  const int kb_total = static_cast<int>(p.K * 2);
  const int nk = (kb_total + P::RB - 1) / P::RB;
  const bool k_tail = (kb_total % P::RB) != 0;
  const uint32_t ldx_b = static_cast<uint32_t>(p.ldx * 2), ldw_b = static_cast<uint32_t>(p.K * 2);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(static_cast<const char*>(p.x) + m0 * p.ldx * 2, static_cast<uint32_t>(rows_m) * ldx_b);
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(static_cast<const char*>(p.W) + n0 * p.K * 2, static_cast<uint32_t>(rows_n) * ldw_b);
  TileOffsets<P, P::BM> ox;
  TileOffsets<P, P::BN> ow;
  ox.init(ldx_b, 0, rows_m, 0);
  ow.init(ldw_b, 0, rows_n, 0);
  // K-extension stages: 2 * r_pad / RB per group whose columns meet the tile
  int n_ext = 0;
  for (int gi = 0; gi < p.n_groups; ++gi) {
    const GroupDev& g = p.g[gi];
    if (g.col_off < n0 + rows_n && g.col_off + g.n_cols > n0) n_ext += g.r_pad * 2 / P::RB;
  }
  const int NS = nk + n_ext;
  const uint32_t ldt_b = static_cast<uint32_t>(p.ldt * 2);

  auto issue_main = [&](int s) {
    char* bx = smem + (s % P::S) * P::STAGE_BYTES;
    const bool tail = k_tail && s == nk - 1;
    ox.load(bx, xr, s * P::RB, tail, kb_total);
    ow.load(bx + P::X_BYTES, wr, s * P::RB, tail, kb_total);
  };
  auto issue_ext = [&](int s) {
    char* bx = smem + (s % P::S) * P::STAGE_BYTES;
    int e = s - nk;
    for (int gi = 0; gi < p.n_groups; ++gi) {
      const GroupDev& g = p.g[gi];
      if (!(g.col_off < n0 + rows_n && g.col_off + g.n_cols > n0)) continue;
      const int ns = g.r_pad * 2 / P::RB;
      if (e >= ns) {
        e -= ns;
        continue;
      }
      const __amdgpu_buffer_rsrc_t tr = make_rsrc(static_cast<const char*>(p.work) + (m0 * p.ldt + g.t_col) * 2,
                                                  static_cast<uint32_t>(rows_m) * ldt_b);
      dma<P, P::BM>(bx, tr, ldt_b, 0, rows_m, 0, e * P::RB, g.r_pad * 2);
      const uint32_t ldb_b = static_cast<uint32_t>(g.rank * 2);
      const __amdgpu_buffer_rsrc_t br = make_rsrc(g.B, static_cast<uint32_t>(g.n_cols) * ldb_b);
      const int lo = static_cast<int>(max<int64_t>(0, g.col_off - n0));
      const int hi = static_cast<int>(min<int64_t>(rows_n, g.col_off + g.n_cols - n0));
      dma<P, P::BN>(bx + P::X_BYTES, br, ldb_b, lo, hi, static_cast<int>(n0 - g.col_off), e * P::RB, g.rank * 2);
      return;
    }
  };
  auto issue = [&](int s) {
    if (s < nk) issue_main(s);
    else issue_ext(s);
  };

  f32x16 acc[P::NI][P::NJ];
#pragma unroll
  for (int i = 0; i < P::NI; ++i)
#pragma unroll
    for (int j = 0; j < P::NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // prologue: the first S stages in flight, wait for stage 0
  for (int s = 0; s < P::S && s < NS; ++s) issue(s);
  wait_stages<P::LPS>(min(NS, P::S) - 1);
  stage_barrier();
  Frags<P> fr[2];
  load_frags<P>(fr[0], smem, 0, wn0, wm0, lane);

  // one stage of MFMA work; in its last 16-k step the next stage is published by
  // a barrier and (steady state) stage j + S is issued into the freed buffer
  auto run_stage = [&](int j, bool steady) {
    const char* st = smem + (j % P::S) * P::STAGE_BYTES;
#pragma unroll
    for (int kk = 0; kk < P::KK; ++kk) {
      if (kk + 1 < P::KK) {
        load_frags<P>(fr[(kk + 1) & 1], st, kk + 1, wn0, wm0, lane);
      } else {
        if (steady) {
          wait_stages<P::LPS>(P::S - 2);
        } else {
          wait_stages<P::LPS>(min(NS - j - 2, P::S - 2));
        }
        stage_barrier();  // stage j + 1 visible; every wave is done reading stage j
        if (steady) {
          if (j + P::S < nk) issue_main(j + P::S);
          else issue_ext(j + P::S);
        }
        load_frags<P>(fr[(kk + 1) & 1], smem + ((j + 1) % P::S) * P::STAGE_BYTES, 0, wn0, wm0, lane);
      }
      mfma_frags<P>(acc, fr[kk & 1]);
      interleave_reads_with_mfma<P>();
    }
  };
  int j = 0;
  for (; j + P::S < NS; ++j) run_stage(j, true);
  for (; j + 1 < NS; ++j) run_stage(j, false);
  {
    const char* st = smem + ((NS - 1) % P::S) * P::STAGE_BYTES;
#pragma unroll
    for (int kk = 0; kk < P::KK; ++kk) {
      if (kk + 1 < P::KK) load_frags<P>(fr[(kk + 1) & 1], st, kk + 1, wn0, wm0, lane);
      mfma_frags<P>(acc, fr[kk & 1]);
    }
  }

  // epilogue: + bias (fp32), one rounding, store
  epilogue<Cfg<P::BM, P::BN, P::WM, P::WN>, bf16_bits>(acc, p, m0, n0, wm0, wn0, lane);
}


// ---------------------------------------------------------------------------
// One copy instruction `it` of a staged tile whose rows come from source row
// (row + shift) for rows in [row_lo, row_hi), bytes [kb0, kb_valid); other
// lanes read as zero (K-extension units: t~ rows and LoRA B rows).
template <class P, int ROWS>
__device__ __forceinline__ void dma_one(int it, char* lds, __amdgpu_buffer_rsrc_t rsrc, uint32_t ld_bytes,
                                        int row_lo, int row_hi, int shift, int kb0, int kb_valid) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot0 = (it * P::WAVES + wave) * 64;
  const int sl = slot0 + lane;
  const int row = sl / P::CPR;
  const int c = (sl % P::CPR) ^ ((row / P::RPL) % P::CPR);
  const int kb = kb0 + c * 16;
  const uint32_t voff = (row >= row_lo && row < row_hi && kb < kb_valid)
                            ? static_cast<uint32_t>(row + shift) * ld_bytes + static_cast<uint32_t>(kb)
                            : 0x80000000u;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + slot0 * 16), 16, voff, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// The hot kernel on v_mfma_f32_16x16x32_bf16: 256 x 256 tile, 4 waves of
// 128 x 128; the x part and the W part of a 64-k stage are separate units of a
// ring of five 32 KB LDS slots (unit 2s = x rows of stage s, 2s + 1 = W rows,
// slot = unit mod 5), 128-byte rows; each wave holds 8 x 8 blocks of 16 x 16
// (4 accumulators per lane each) and a 64-k stage is two 32-k steps of 64 MFMAs.
// Under a sustained MFMA load this instruction runs at a clearly higher clock
// than the 32 x 32 x 16 one for the same work per cycle (measured on MI355X:
// about 2.05 against 1.77 GHz with LDS operand reads), which is where the
// kernel's throughput is decided once the copies are hidden.
template <int BM_, int BN_, int WM_, int WN_, int RB_, int SLOTS_, int OCC_ = 1>
struct QCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, RB = RB_, SLOTS = SLOTS_;
  static constexpr int OCC = OCC_;                    // workgroups resident per CU (waves per SIMD)
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN, WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int NI = WN / 16, NJ = WM / 16;   // 16 x 16 blocks per wave
  static constexpr int CPR = RB / 16, RPL = 256 / RB;
  static constexpr int KK = RB / 64;                  // 32-k MFMA steps per stage
  static constexpr int SLOT_BYTES = BM * RB;
  static constexpr int GROUP_M = 4;
  static_assert(BM == BN && RB == 128 && KK == 2, "x and W units share one slot size; two k-steps per stage");
  static_assert((BM * CPR / 64) % WAVES == 0, "uneven load split");
  static_assert(SLOTS == 5 && OCC * SLOTS * SLOT_BYTES <= 160 * 1024, "LDS");
};

template <class P>
struct Frags16 {
  bf16x8 a[P::NI], b[P::NJ];
};

// Operand fragments of 32-k step kk: lane (r = lane % 16, q = lane / 16) holds
// k = 8q .. 8q + 7 of row r of each 16-row block, i.e. 16-byte chunk 4 kk + q.
// With 128-byte rows the swizzle term (row / 2) % 8 is the same for every
// 16-row block, so block i sits at a fixed 2048-byte offset from the lane's
// block-0 address, and k-step 1 is k-step 0's address with byte bit 6 flipped.
struct FragOffsets {
  uint32_t x, w;  // byte offsets of this lane's k-step-0 chunk in block 0 of an x / W slot
};

template <class P>
__device__ __forceinline__ FragOffsets frag_offsets(int wn0, int wm0, int lane) {
  const int r = lane & 15, q = lane >> 4;
  const int c = q ^ ((r >> 1) & 7);
  return FragOffsets{static_cast<uint32_t>(((wm0 + r) * P::CPR + c) * 16),
                     static_cast<uint32_t>(((wn0 + r) * P::CPR + c) * 16)};
}

template <class P>
__device__ __forceinline__ void ring_frags16(Frags16<P>& f, const char* xs, const char* ws, int kk,
                                             FragOffsets o) {
  const uint32_t flip = kk ? 64u : 0u;
#pragma unroll
  for (int i = 0; i < P::NI; ++i) f.a[i] = *(const bf16x8*)(ws + (o.w ^ flip) + i * 2048);
#pragma unroll
  for (int j = 0; j < P::NJ; ++j) f.b[j] = *(const bf16x8*)(xs + (o.x ^ flip) + j * 2048);
}

template <class P>
__device__ __forceinline__ void mfma_frags16(f32x4 (&acc)[P::NI][P::NJ], const Frags16<P>& f) {
#pragma unroll
  for (int i = 0; i < P::NI; ++i)
#pragma unroll
    for (int j = 0; j < P::NJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// A staged 16-byte chunk with its two 8-byte halves back in column order (swapped when sw).
__device__ __forceinline__ u32x4 unswap_halves(u32x4 v, int sw) {
  return sw ? u32x4{v[2], v[3], v[0], v[1]} : v;
}

// 4-bit weight inside the hot kernel. One 64-element block of a weight row (one 64-k stage)
// has one scale a, so its 16 possible values RN_bf16(RN_f32(codebook[c] . a)) form a table,
// built with the same multiply and conversion as the panel kernel (the two paths give the
// same weight bits). The table is kept as low and high bytes of the entries, four per
// register (lo[i] byte j = low byte of entry 4i + j), so that a byte permute looks up four
// codes of bits 0-2 at once among 8 entries; bit 3 picks the half.
struct Nf4Table {
  uint32_t lo[4], hi[4];
};

// f(0), f(1), .., f(N - 1) with compile-time indices: a loop unrolled whatever the size of its
// body (past a size, the compiler's own full unrolling gives up and leaves the index a run-time
// value, which turns register arrays indexed by it into scratch memory).
template <class F, int... I>
__device__ __forceinline__ void unrolled_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void unrolled(F& f) {
  unrolled_impl(f, std::make_integer_sequence<int, N>{});
}

// Empty asm on a value: the instructions that produce it stay in the MFMA bundle where they
// are placed (the compiler would otherwise sink them toward their use, past the bundles the
// work is spread over, or to the LDS writes after the barrier).
__device__ __forceinline__ void pin(uint32_t& v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(v));
#endif
}

// The table in 11 sub-steps of at most 3 VALU instructions: s < 8 scales entries 2s and 2s + 1
// and rounds them to a bf16 pair (two multiplies, one conversion); s = 8, 9, 10 split the pairs
// into low and high bytes (3, 3 and 2 byte permutes).
constexpr int kNf4TableSteps = 11;
struct Nf4TableBuild {
  uint32_t t[8];
};
__device__ __forceinline__ void nf4_table_step(Nf4TableBuild& b, Nf4Table& r, const float (&cb)[16], float a,
                                               int s) {
  if (s < 8) {
    b.t[s] = pack_bf16x2(cb[2 * s] * a, cb[2 * s + 1] * a);
    pin(b.t[s]);
    return;
  }
  // lo[i] holds bytes 0 and 2 (the low bytes of entries 4i, 4i + 1) of t[2i], then of t[2i + 1];
  // hi[i] the high bytes
  auto lo = [&](int i) {
    r.lo[i] = __builtin_amdgcn_perm(b.t[2 * i + 1], b.t[2 * i], 0x06040200u);
    pin(r.lo[i]);
  };
  auto hi = [&](int i) {
    r.hi[i] = __builtin_amdgcn_perm(b.t[2 * i + 1], b.t[2 * i], 0x07050301u);
    pin(r.hi[i]);
  };
  if (s == 8) {
    lo(0), hi(0), lo(1);
  } else if (s == 9) {
    hi(1), lo(2), hi(2);
  } else {
    lo(3), hi(3);
  }
}

// Eight weight elements from one code word (byte j: element 2j in bits 0-3, 2j + 1 in bits
// 4-7) as four bf16 pairs in element order, in 9 sub-steps of at most 4 VALU instructions.
// v_perm_b32 (S0, S1, sel): output byte i is byte sel_i of the 8 bytes S1 (0-3), S0 (4-7);
// selectors 8-11 give 0xff or 0 by the sign bit of bytes 1, 3, 5, 7. Sub-steps 0-3 gather the
// codes four to a register as bytes, in element order (0, 1, 4, 5) and (2, 3, 6, 7), and turn
// their bit 3 into byte masks through those sign selectors (bit 3 of element 2j + h is bit
// 8j + 4h + 3 of the word, shifted to a sign position); 4-7 look the two groups up, low and high
// bytes, in the half that bit 3 picks; 8 interleaves the bytes back into bf16 values.
constexpr int kNf4WordSteps = 9;
struct Nf4Word {
  uint32_t wr4, xa, xb, ma, mb, la, ha, lb, hb;
};
__device__ __forceinline__ void nf4_word_step(Nf4Word& s, u32x4& out, uint32_t w, const Nf4Table& tb, int step) {
  auto pick = [](uint32_t m, uint32_t hi_half, uint32_t lo_half) { return (hi_half & m) | (lo_half & ~m); };
  auto look = [&](const uint32_t (&t)[4], uint32_t x, uint32_t m) {
    return pick(m, __builtin_amdgcn_perm(t[3], t[2], x), __builtin_amdgcn_perm(t[1], t[0], x));
  };
  switch (step) {
    case 0:
      s.wr4 = w >> 4;
      s.xa = __builtin_amdgcn_perm(s.wr4, w, 0x06020400u);  // elements 0, 1, 4, 5
      pin(s.wr4);
      pin(s.xa);
      break;
    case 1:
      s.xa &= 0x07070707u;
      s.xb = __builtin_amdgcn_perm(s.wr4, w, 0x07030501u) & 0x07070707u;  // elements 2, 3, 6, 7
      pin(s.xa);
      pin(s.xb);
      break;
    case 2:
      s.ma = __builtin_amdgcn_perm(w << 8, w << 12, 0x0B090A08u);
      pin(s.ma);
      break;
    case 3:
      s.mb = __builtin_amdgcn_perm(w, w << 4, 0x0B090A08u);
      pin(s.mb);
      break;
    case 4:
      s.la = look(tb.lo, s.xa, s.ma);
      pin(s.la);
      break;
    case 5:
      s.ha = look(tb.hi, s.xa, s.ma);
      pin(s.ha);
      break;
    case 6:
      s.lb = look(tb.lo, s.xb, s.mb);
      pin(s.lb);
      break;
    case 7:
      s.hb = look(tb.hi, s.xb, s.mb);
      pin(s.hb);
      break;
    default:  // interleave low and high bytes back into bf16 values
      out = u32x4{__builtin_amdgcn_perm(s.ha, s.la, 0x05010400u), __builtin_amdgcn_perm(s.hb, s.lb, 0x05010400u),
                  __builtin_amdgcn_perm(s.ha, s.la, 0x07030602u), __builtin_amdgcn_perm(s.hb, s.lb, 0x07030602u)};
#if defined(__HIP_DEVICE_COMPILE__)
      asm volatile("" : "+v"(out[0]), "+v"(out[1]), "+v"(out[2]), "+v"(out[3]));
#endif
  }
}

template <int WPT>
struct Nf4Codes {
  u32x4 q[WPT / 4];  // word j is q[j / 4][j % 4]
  float a;
};

// Per-thread share of a 4-bit weight tile: TPR threads per weight row, each with WPT code words
// (8 elements each) of the row's 64-k stage, and the block's scale.
template <class P>
struct Nf4Share {
  static constexpr int TPR = P::THREADS / P::BN, WPT = 8 / TPR;
  static_assert(P::THREADS % P::BN == 0 && (WPT == 4 || WPT == 8), "one or two threads per weight row");
  uint32_t cvo, avo;  // byte offsets of this thread's code words and scale at main stage 0 (past the range: no row)
  int row, half;
  __device__ __forceinline__ void init(int tid, int rows_n, int64_t K) {
    row = tid / TPR;
    half = tid % TPR;
    const bool in = row < rows_n;
    cvo = in ? static_cast<uint32_t>(row * (K / 2) + half * WPT * 4) : 0x80000000u;
    avo = in ? static_cast<uint32_t>(row * (K / 64) * 4) : 0x80000000u;
  }
  // Loads of main stage s (WPT / 4 + 1 buffer loads, issued in this order).
  __device__ __forceinline__ void load(Nf4Codes<WPT>& c, __amdgpu_buffer_rsrc_t cr, __amdgpu_buffer_rsrc_t ar,
                                       int s) const {
#pragma unroll
    for (int i = 0; i < WPT / 4; ++i)
      c.q[i] = __builtin_amdgcn_raw_buffer_load_b128(cr, cvo + i * 16, s * 32, 0);
    c.a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ar, avo, s * 4, 0));
  }
  // LDS byte offset of this thread's logical chunk j of its row in a weight slot (the copy layout:
  // 128-byte rows, 16-byte chunk c of row r at position c ^ ((r / 2) % 8)).
  __device__ __forceinline__ uint32_t lds_off(int j) const {
    return static_cast<uint32_t>(row * 128 + (((half * WPT + j) ^ ((row >> 1) & 7)) * 16));
  }
};

// Epilogue of the 16 x 16 layout: lane (r, q) of block (i, j) holds outputs
// i*16 + 4q .. +3 of token j*16 + r. Bias in fp32 (no add without a bias), one
// rounding, staged in the wave's 32 KB of LDS as token rows (16-byte chunks
// XOR-swizzled by row), then written as whole 256-byte output rows, as in the
// 32 x 32 epilogue.
// BIAS: 0 none, 1 the bf16 bias, 2 the fp32 bias vector p.bias32.
template <class P, int BIAS>
__device__ __forceinline__ void stage_out16(const f32x4 (&acc)[P::NI][P::NJ], const LinearProblem& p, int64_t n0,
                                            int wn0, int lane, char* st) {
  const int r = lane & 15, q = lane >> 4;
  const bf16_bits* bias = static_cast<const bf16_bits*>(p.bias);
#pragma unroll
  for (int i = 0; i < P::NI; ++i) {
    const int cl = i * 16 + q * 4;  // first of 4 columns, local to the wave block
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (BIAS == 2) {
      const int64_t n = n0 + wn0 + cl;
      if (n + 3 < p.N) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(p.bias32 + n);  // 16-byte aligned: n is a multiple of 4
        bv[0] = w[0]; bv[1] = w[1]; bv[2] = w[2]; bv[3] = w[3];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < p.N) bv[e] = p.bias32[n + e];
      }
    } else if (BIAS == 1) {
      const int64_t n = n0 + wn0 + cl;
      if (n + 3 < p.N) {
        const uint2 w = *reinterpret_cast<const uint2*>(bias + n);  // 8-byte aligned: n is a multiple of 4
        bv[0] = __uint_as_float(w.x << 16); bv[1] = __uint_as_float(w.x & 0xffff0000u);
        bv[2] = __uint_as_float(w.y << 16); bv[3] = __uint_as_float(w.y & 0xffff0000u);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < p.N) bv[e] = bf16_to_f32(bias[n + e]);
      }
    }
#pragma unroll
    for (int j = 0; j < P::NJ; ++j) {
      const int row = j * 16 + r;
      uint2 w;
      if (BIAS != 0) {
        w.x = pack_bf16x2(acc[i][j][0] + bv[0], acc[i][j][1] + bv[1]);
        w.y = pack_bf16x2(acc[i][j][2] + bv[2], acc[i][j][3] + bv[3]);
      } else {
        w.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        w.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
      }
      // 16-byte chunk XOR-swizzled by row; the two 8-byte halves of a chunk swap places in rows
      // 8 .. 15 of every 16, so that the 16 lanes of one write (rows r = 0 .. 15, one half each)
      // cover all 32 banks
      const int chunk = (cl >> 3) ^ (row & 15);
      *reinterpret_cast<uint2*>(st + row * 256 + chunk * 16 + ((q & 1) ^ ((row >> 3) & 1)) * 8) = w;
    }
    __builtin_amdgcn_sched_barrier(0);  // keeps accumulator reads from being hoisted (register pressure)
  }
}

template <class P>
__device__ __forceinline__ void epilogue_lds16(const f32x4 (&acc)[P::NI][P::NJ], const LinearProblem& p,
                                               int64_t m0, int64_t n0, int wm0, int wn0, int lane, int wave,
                                               char* smem) {
  static_assert(P::WM == 128 && P::WN == 128, "staging written for 128 x 128 wave blocks");
  char* st = smem + wave * (128 * 256);
  // (only this wave reads its staging, and a wave's LDS operations run in
  // order, so the reads below see the writes without a wait)
  if (p.bias32 != nullptr) stage_out16<P, 2>(acc, p, n0, wn0, lane, st);
  else if (p.bias != nullptr) stage_out16<P, 1>(acc, p, n0, wn0, lane, st);
  else stage_out16<P, 0>(acc, p, n0, wn0, lane, st);
  const int c = lane & 15, rr = lane >> 4;
  const int64_t mb = m0 + wm0;  // first token of the wave block
  const int64_t n = n0 + wn0 + c * 8;
  bf16_bits* y = static_cast<bf16_bits*>(p.y);
  const bool aligned16 = (reinterpret_cast<uintptr_t>(p.y) % 16 == 0) && (p.ldy % 8 == 0);
  if (aligned16 && n0 + wn0 + 128 <= p.N) {
    // all 128 columns exist: buffer stores over the block's valid rows; a row past
    // T has its offset (in the per-lane offset, which the range check covers)
    // beyond the range and is dropped
    const int64_t rows = min<int64_t>(128, p.T - mb);
    if (rows <= 0) return;
    const uint32_t ldb = static_cast<uint32_t>(p.ldy * 2);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y + mb * p.ldy + n0 + wn0, static_cast<uint32_t>(rows) * ldb);
#pragma unroll 8
    for (int it = 0; it < 32; ++it) {
      const int row = it * 4 + rr;
      const u32x4 v = unswap_halves(*reinterpret_cast<const u32x4*>(st + row * 256 + ((c ^ (row & 15)) * 16)),
                                    (row >> 3) & 1);
      // non-temporal (cache-policy bit nt): an output of hundreds of MB does not stay in the
      // Infinity Cache, where its dirty lines would be written back while the next kernel
      // streams its own inputs (measured: the next layer's producer 142 -> 106 us)
      __builtin_amdgcn_raw_buffer_store_b128(v, yr, static_cast<uint32_t>(row) * ldb + static_cast<uint32_t>(c) * 16, 0,
                                             kCachePolicyNT);
    }
    return;
  }
#pragma unroll 8
  for (int it = 0; it < 32; ++it) {
    const int row = it * 4 + rr;
    const u32x4 v = unswap_halves(*reinterpret_cast<const u32x4*>(st + row * 256 + ((c ^ (row & 15)) * 16)),
                                  (row >> 3) & 1);
    const int64_t m = mb + row;
    if (m < p.T) {
      bf16_bits* dst = y + m * p.ldy + n;
      if (aligned16 && n + 7 < p.N) {
        *reinterpret_cast<u32x4*>(dst) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < p.N) dst[e] = static_cast<bf16_bits>(v[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

// Epilogue of 64 x 64 wave blocks (the 128 x 128 tile): lane (r, q) of block (i, j) holds
// outputs i*16 + 4q .. +3 of token j*16 + r. Bias in fp32 (no add without a bias), one
// rounding, staged in the wave's 8 KB of LDS as token rows of 128 bytes (16-byte chunks
// XOR-swizzled by row / 2, so that 16 consecutive rows of one chunk column and 8 rows of one
// row pair spread over the banks), then written as whole 128-byte output row pieces.
template <class P, int BIAS>
__device__ __forceinline__ void stage_out16s(const f32x4 (&acc)[P::NI][P::NJ], const LinearProblem& p, int64_t n0,
                                             int wn0, int lane, char* st) {
  const int r = lane & 15, q = lane >> 4;
  const bf16_bits* bias = static_cast<const bf16_bits*>(p.bias);
#pragma unroll
  for (int i = 0; i < P::NI; ++i) {
    const int cl = i * 16 + q * 4;  // first of 4 columns, local to the wave block
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    const int64_t n = n0 + wn0 + cl;
    if (BIAS == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < p.N) bv[e] = p.bias32[n + e];
    } else if (BIAS == 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < p.N) bv[e] = bf16_to_f32(bias[n + e]);
    }
#pragma unroll
    for (int j = 0; j < P::NJ; ++j) {
      const int row = j * 16 + r;
      uint2 w;
      if (BIAS != 0) {
        w.x = pack_bf16x2(acc[i][j][0] + bv[0], acc[i][j][1] + bv[1]);
        w.y = pack_bf16x2(acc[i][j][2] + bv[2], acc[i][j][3] + bv[3]);
      } else {
        w.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        w.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
      }
      // (halves swapped in odd rows: the 16 lanes of one write then cover all 32 banks)
      const int chunk = (cl >> 3) ^ ((row >> 1) & 7);
      *reinterpret_cast<uint2*>(st + row * 128 + chunk * 16 + ((q & 1) ^ (row & 1)) * 8) = w;
    }
  }
}

template <class P>
__device__ __forceinline__ void epilogue_lds16s(const f32x4 (&acc)[P::NI][P::NJ], const LinearProblem& p,
                                                int64_t m0, int64_t n0, int wm0, int wn0, int lane, int wave,
                                                char* smem) {
  static_assert(P::WM == 64 && P::WN == 64, "staging written for 64 x 64 wave blocks");
  char* st = smem + wave * (64 * 128);
  // (only this wave reads its staging, and a wave's LDS operations run in
  // order, so the reads below see the writes without a wait)
  if (p.bias32 != nullptr) stage_out16s<P, 2>(acc, p, n0, wn0, lane, st);
  else if (p.bias != nullptr) stage_out16s<P, 1>(acc, p, n0, wn0, lane, st);
  else stage_out16s<P, 0>(acc, p, n0, wn0, lane, st);
  const int c = lane & 7, rr = lane >> 3;
  const int64_t mb = m0 + wm0;  // first token of the wave block
  const int64_t n = n0 + wn0 + c * 8;
  bf16_bits* y = static_cast<bf16_bits*>(p.y);
  const bool aligned16 = (reinterpret_cast<uintptr_t>(p.y) % 16 == 0) && (p.ldy % 8 == 0);
  if (aligned16 && n0 + wn0 + 64 <= p.N) {
    // all 64 columns exist: buffer stores over the block's valid rows; a row past T
    // has its offset beyond the range and is dropped
    const int64_t rows = min<int64_t>(64, p.T - mb);
    if (rows <= 0) return;
    const uint32_t ldb = static_cast<uint32_t>(p.ldy * 2);
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y + mb * p.ldy + n0 + wn0, static_cast<uint32_t>(rows) * ldb);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int row = it * 8 + rr;
      const u32x4 v = unswap_halves(*reinterpret_cast<const u32x4*>(st + row * 128 + ((c ^ ((row >> 1) & 7)) * 16)),
                                    row & 1);
      __builtin_amdgcn_raw_buffer_store_b128(v, yr, static_cast<uint32_t>(row) * ldb + static_cast<uint32_t>(c) * 16, 0,
                                             kCachePolicyNT);
    }
    return;
  }
  for (int it = 0; it < 8; ++it) {
    const int row = it * 8 + rr;
    const u32x4 v = unswap_halves(*reinterpret_cast<const u32x4*>(st + row * 128 + ((c ^ ((row >> 1) & 7)) * 16)),
                                  row & 1);
    const int64_t m = mb + row;
    if (m < p.T) {
      bf16_bits* dst = y + m * p.ldy + n;
      if (aligned16 && n + 7 < p.N) {
        *reinterpret_cast<u32x4*>(dst) = v;
      } else {
        for (int e = 0; e < 8; ++e)
          if (n + e < p.N) dst[e] = static_cast<bf16_bits>(v[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

// K-extension plan of one adapter group for one output tile: where its t~
// columns and B rows are, which tile rows its B rows cover, and how many
// 64-k stages its padded rank takes.
struct ExtPlan {
  const char* B;
  int tcb, tpb, rkb, n_cols, lo, hi, sh, ns;
};

// Copies of K-extension stage e of group g through precomputed per-lane
// offsets: t~ rows (every padded column exists) into xdst, B rows (chunks past
// the rank read as zero) into wdst.
template <class P>
__device__ __forceinline__ void ext_stage_loads(const ExtPlan& g, int e, const TileOffsets<P, P::BM>& ot,
                                                __amdgpu_buffer_rsrc_t tr, char* xdst, char* wdst) {
#pragma unroll
  for (int l = 0; l < TileOffsets<P, P::BM>::N; ++l) ot.load_one(l, xdst, tr, g.tcb + e * P::RB);
  TileOffsets<P, P::BN> ob;
  ob.init(static_cast<uint32_t>(g.rkb), g.lo, g.hi, g.sh);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(g.B, static_cast<uint32_t>(g.n_cols) * static_cast<uint32_t>(g.rkb));
  ob.load(wdst, br, e * P::RB, (e + 1) * P::RB > g.rkb, g.rkb);
}

// Stage t of the 16 x 16 kernel is 2 NB MFMA bundles (NB = NI NJ per k-step: 64 for
// the 256 x 256 tile, 16 for the 128 x 128 tile). Copies, one every LS-th bundle:
// the NL loads of x of stage t + 2 in the first half (its slot was released by the
// previous stage's barrier), the NL of W of stage t + 2 in the second (into the slot
// of x of stage t, released by this stage's barrier at the first bundle of k-step 1).
// The barrier waits for everything but the x loads of this stage. Fragment reads:
// k-step 1 of this stage one every RS-th bundle of k-step 0, k-step 0 of stage t + 1
// one every RS-th bundle after the barrier. Both tiles accumulate every output in the
// same order (K-extension stages, then the main stages, 32 k per MFMA), so they give
// bitwise-identical results.
// NF4: the base weight is 4-bit codes with one fp32 scale per 64-element block (K a multiple
// of 64). A main stage's weight unit is then written by the waves themselves instead of
// copied: the codes of the weight unit of stage t + 2 are loaded into registers at the start
// of stage t - 1 (after the wait for that stage's own codes, before its x copies), dequantized
// during stage t in sub-steps of a few VALU instructions, one or two per MFMA bundle, and each
// word written into the slot that the barrier of stage t releases, where the copies would have
// gone. The weight is the panel kernel's, bit for bit, and so is the result.
template <class P, bool NF4 = false>
__global__ __launch_bounds__(P::THREADS, P::OCC) void gemm_flow16_kernel(LinearProblem p, int mt, int nt) {
  static_assert(P::WAVES == 4, "schedule written for 4 waves");
  __shared__ __attribute__((aligned(1024))) char smem[P::SLOTS * P::SLOT_BYTES];
  constexpr int NL = TileOffsets<P, P::BM>::N;  // copy loads per wave per unit
  constexpr int NB = P::NI * P::NJ;             // MFMA bundles per k-step
  constexpr int RS = NB / (P::NI + P::NJ);      // bundles per fragment read
  constexpr int LS = NB / NL;                   // bundles per copy load
  static_assert(NB % (P::NI + P::NJ) == 0 && NB % NL == 0 && LS % 2 == 0 && RS >= 2, "bundle schedule");

  const int G = mt * nt;
  const int L = xcd_remap(blockIdx.x, G);
  const int gsize = P::GROUP_M * nt;
  const int grp = L / gsize;
  const int first_m = grp * P::GROUP_M;
  const int gm = min(P::GROUP_M, mt - first_m);
  const int within = L - grp * gsize;
  const int m_idx = first_m + within % gm;
  const int n_idx = within / gm;

  // (the wave index through readfirstlane: the compiler then knows it, and all
  // that derives from it -- wave block origin, output resource -- is wave-uniform)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave % P::WAVES_M) * P::WM;
  const int wn0 = (wave / P::WAVES_M) * P::WN;
  const int64_t m0 = static_cast<int64_t>(m_idx) * P::BM;
  const int64_t n0 = static_cast<int64_t>(n_idx) * P::BN;
  const int rows_m = static_cast<int>(min<int64_t>(P::BM, p.T - m0));
  const int rows_n = static_cast<int>(min<int64_t>(P::BN, p.N - n0));

  const int kb_total = static_cast<int>(p.K * 2);
  const int nk = (kb_total + P::RB - 1) / P::RB;
  const bool k_tail = (kb_total % P::RB) != 0;
  const uint32_t ldx_b = static_cast<uint32_t>(p.ldx * 2), ldw_b = static_cast<uint32_t>(p.K * 2);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(static_cast<const char*>(p.x) + m0 * p.ldx * 2, static_cast<uint32_t>(rows_m) * ldx_b);
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(static_cast<const char*>(p.W) + n0 * p.K * 2, static_cast<uint32_t>(rows_n) * ldw_b);
  TileOffsets<P, P::BM> ox;
  TileOffsets<P, P::BN> ow;
  ox.init(ldx_b, 0, rows_m, 0);
  if constexpr (!NF4) ow.init(ldw_b, 0, rows_n, 0);
  using Share = Nf4Share<P>;
  constexpr int WPT = Share::WPT;
  constexpr int NC = WPT / 4 + 1;  // code loads per stage
  Share nfs;
  Nf4Codes<WPT> c_load, c_work;     // codes of a later stage in flight; codes being dequantized
  u32x4 dq[WPT];                    // dequantized weight words of stage t + 2, until written
  float cb[16];
  const __amdgpu_buffer_rsrc_t cr =
      make_rsrc(NF4 ? p.codes + n0 * (p.K / 2) : nullptr, NF4 ? static_cast<uint32_t>(rows_n * (p.K / 2)) : 0u);
  const __amdgpu_buffer_rsrc_t ar =
      make_rsrc(NF4 ? p.absmax + n0 * (p.K / 64) : nullptr, NF4 ? static_cast<uint32_t>(rows_n * (p.K / 64) * 4) : 0u);
  if constexpr (NF4) {
    nfs.init(tid, rows_n, p.K);
#pragma unroll
    for (int c = 0; c < 16; ++c) cb[c] = p.codebook[c];
  }

  // K-extension plan of this tile: the (at most two) groups whose columns meet it.
  const uint32_t ldt_b = static_cast<uint32_t>(p.ldt * 2);
  int gs0 = p.n_groups, gs1 = p.n_groups;
  for (int gi = 0; gi < p.n_groups; ++gi) {
    if (!(p.g[gi].col_off < n0 + rows_n && p.g[gi].col_off + p.g[gi].n_cols > n0)) continue;
    if (gs0 == p.n_groups) {
      gs0 = gi;
    } else {
      gs1 = gi;
      break;
    }
  }
  auto ext_group = [&](int gi) {
    ExtPlan e{nullptr, 0, 0, 0, 0, 0, 0, 0, 0};
    if (gi < p.n_groups) {
      const GroupDev& g = p.g[gi];
      e.B = static_cast<const char*>(g.B);
      e.tcb = g.t_col * 2;
      e.tpb = g.r_pad * 2;
      e.rkb = g.rank * 2;
      e.n_cols = static_cast<int>(g.n_cols);
      e.lo = static_cast<int>(max<int64_t>(0, g.col_off - n0));
      e.hi = static_cast<int>(min<int64_t>(rows_n, g.col_off + g.n_cols - n0));
      e.sh = static_cast<int>(n0 - g.col_off);
      e.ns = g.r_pad * 2 / P::RB;
    }
    return e;
  };
  const ExtPlan eg0 = ext_group(gs0), eg1 = ext_group(gs1);
  // Stage order: the K-extension stages first, then the main stages (s >= NE is main stage s - NE).
  const int NE = eg0.ns + eg1.ns;
  const int NS = NE + nk;
  const int NU = 2 * NS;
  const __amdgpu_buffer_rsrc_t tr =
      make_rsrc(static_cast<const char*>(p.work) + m0 * p.ldt * 2, static_cast<uint32_t>(rows_m) * ldt_b);
  // K-extension stages after the prologue's (more than two): per-lane copy offsets of the t~ rows
  // and of the B rows of each of the tile's two groups, computed once per tile, so that a copy
  // takes a select and a K-tail mask instead of its whole offset arithmetic (a 4-bit weight, with
  // its one adapter and the dequantization's registers, keeps the per-copy arithmetic)
  TileOffsets<P, P::BM> oxe;
  TileOffsets<P, P::BN> ob0, ob1;
  if constexpr (!NF4) {
    oxe.init(ldt_b, 0, rows_m, 0);
    ob0.init(static_cast<uint32_t>(eg0.rkb), eg0.lo, eg0.hi, eg0.sh);
    ob1.init(static_cast<uint32_t>(eg1.rkb), eg1.lo, eg1.hi, eg1.sh);
  }
  const __amdgpu_buffer_rsrc_t br0 =
      make_rsrc(eg0.B, static_cast<uint32_t>(eg0.n_cols) * static_cast<uint32_t>(eg0.rkb));
  const __amdgpu_buffer_rsrc_t br1 =
      make_rsrc(eg1.B, static_cast<uint32_t>(eg1.n_cols) * static_cast<uint32_t>(eg1.rkb));
  // this lane's 16-byte chunk of a B row, the same in every copy instruction of a unit (each
  // instruction covers whole swizzle periods of rows)
  static_assert((P::WAVES * 64 / P::CPR / P::RPL) % P::CPR == 0, "one chunk per lane across a unit");
  const int c_ext = (lane % P::CPR) ^ (((wave * 64 + lane) / P::CPR / P::RPL) % P::CPR);

  auto slot = [&](int u) { return smem + (u % P::SLOTS) * P::SLOT_BYTES; };
  auto issue_load = [&](int u, int l) {
    if (u >= NU) return;
    char* dst = slot(u);
    const int s = u >> 1;
    const bool is_w = (u & 1) != 0;
    if (s >= NE) {
      const int kb = (s - NE) * P::RB;
      if (is_w) {
        if constexpr (!NF4) dma_one<P, P::BN>(l, dst, wr, ldw_b, 0, rows_n, 0, kb, kb_total);
      } else {
        dma_one<P, P::BM>(l, dst, xr, ldx_b, 0, rows_m, 0, kb, kb_total);
      }
      return;
    }
    const bool second = s >= eg0.ns;
    const ExtPlan& g = second ? eg1 : eg0;
    const int e = second ? s - eg0.ns : s;
    if (!is_w) {
      dma_one<P, P::BM>(l, dst, tr, ldt_b, 0, rows_m, 0, g.tcb + e * P::RB, g.tcb + g.tpb);
    } else {
      const __amdgpu_buffer_rsrc_t br = make_rsrc(g.B, static_cast<uint32_t>(g.n_cols) * static_cast<uint32_t>(g.rkb));
      dma_one<P, P::BN>(l, dst, br, static_cast<uint32_t>(g.rkb), g.lo, g.hi, g.sh, e * P::RB, g.rkb);
    }
  };

  f32x4 acc[P::NI][P::NJ];
#pragma unroll
  for (int i = 0; i < P::NI; ++i)
#pragma unroll
    for (int j = 0; j < P::NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;

  // NF4: the dequantized words of a main stage's weight unit go to LDS (thread share of row)
  auto nf4_write = [&](char* wslot, int j) {
    *reinterpret_cast<u32x4*>(wslot + nfs.lds_off(j)) = dq[j];
  };
  Nf4TableBuild tbb;
  Nf4Table tb;
  Nf4Word wst;
  // Sub-step g of the dequantization of one weight unit: the table's, then each word's.
  constexpr int NSUB = kNf4TableSteps + kNf4WordSteps * WPT;
  auto nf4_sub = [&](const Nf4Codes<WPT>& c, int g) {
    if (g < kNf4TableSteps) {
      nf4_table_step(tbb, tb, cb, c.a, g);
    } else if (g < NSUB) {
      const int j = (g - kNf4TableSteps) / kNf4WordSteps;
      nf4_word_step(wst, dq[j], c.q[j / 4][j % 4], tb, (g - kNf4TableSteps) % kNf4WordSteps);
    }
  };

  // prologue: units 0 .. 3 (stages 0 and 1). Up to two K-extension stages (ranks
  // up to 128) use precomputed per-lane offsets like the main stages; more
  // extension stages take the generic path.
  if constexpr (NF4) {
    // copies of the x units and of K-extension weight units; main weight units of stages 0
    // and 1 dequantized here; the codes of the first main stage from 2 on loaded for the
    // first stage that dequantizes (K-extension stages load no codes: the compiler's own
    // waits before the first use of loaded registers then stay exact)
    for (int u = 0; u < 4; ++u) {
      if ((u & 1) && (u >> 1) >= NE) continue;
      for (int l = 0; l < NL; ++l) issue_load(u, l);
    }
    for (int s = 0; s < 2 && s < NS; ++s) {
      if (s < NE) continue;
      nfs.load(c_work, cr, ar, s - NE);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      auto sub = [&](int g) { nf4_sub(c_work, g); };
      unrolled<NSUB>(sub);
#pragma unroll
      for (int j = 0; j < WPT; ++j) nf4_write(smem + (2 * s + 1) * P::SLOT_BYTES, j);
    }
    const int s_first = NE > 2 ? NE : 2;
    if (s_first < NS) nfs.load(c_load, cr, ar, s_first - NE);
  } else if (NE == 0 && nk - (k_tail ? 1 : 0) >= 2) {
#pragma unroll
    for (int l = 0; l < NL; ++l) ox.load_one(l, smem, xr, 0);
#pragma unroll
    for (int l = 0; l < NL; ++l) ow.load_one(l, smem + P::SLOT_BYTES, wr, 0);
#pragma unroll
    for (int l = 0; l < NL; ++l) ox.load_one(l, smem + 2 * P::SLOT_BYTES, xr, P::RB);
#pragma unroll
    for (int l = 0; l < NL; ++l) ow.load_one(l, smem + 3 * P::SLOT_BYTES, wr, P::RB);
  } else if (NE == 1 || NE == 2) {
    TileOffsets<P, P::BM> ot;
    ot.init(ldt_b, 0, rows_m, 0);
    ext_stage_loads<P>(eg0, 0, ot, tr, smem, smem + P::SLOT_BYTES);
    if (NE == 1) {  // main stage 0 (it is the K-tail stage when K < 64)
      const bool tail0 = k_tail && nk == 1;
      ox.load(smem + 2 * P::SLOT_BYTES, xr, 0, tail0, kb_total);
      ow.load(smem + 3 * P::SLOT_BYTES, wr, 0, tail0, kb_total);
    } else if (eg0.ns == 2) {
      ext_stage_loads<P>(eg0, 1, ot, tr, smem + 2 * P::SLOT_BYTES, smem + 3 * P::SLOT_BYTES);
    } else {
      ext_stage_loads<P>(eg1, 0, ot, tr, smem + 2 * P::SLOT_BYTES, smem + 3 * P::SLOT_BYTES);
    }
  } else {
    for (int u = 0; u < 4; ++u)
      for (int l = 0; l < NL; ++l) issue_load(u, l);
  }
  if (NU > 2 && !NF4) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NL));  // stage 0 landed; stage 1 may be in flight
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  stage_barrier();
  const FragOffsets fo = frag_offsets<P>(wn0, wm0, lane);
  Frags16<P> fr[2];
  // fragment q of a k-step, in order of first use: a0, b0 .. b(NJ-1), a1 .. a(NI-1)
  auto read_frag = [&](Frags16<P>& f, int q, const char* xs, const char* ws, int kk) {
    const uint32_t flip = kk ? 64u : 0u;
    if (q == 0 || q > P::NJ) {
      const int ia = q == 0 ? 0 : q - P::NJ;
      f.a[ia] = *(const bf16x8*)(ws + (fo.w ^ flip) + ia * 2048);
    } else {
      f.b[q - 1] = *(const bf16x8*)(xs + (fo.x ^ flip) + (q - 1) * 2048);
    }
  };
#pragma unroll
  for (int q = 0; q < P::NI + P::NJ; ++q) read_frag(fr[0], q, slot(0), slot(1), 0);

  // stages t < NE - 2 copy K-extension units (stage t + 2); stages from t_end on
  // copy the last main units or nothing
  const int t_ext = NE > 2 ? NE - 2 : 0;
  const int t_end = NE + nk - 2 - (k_tail ? 1 : 0);

  // stage t whose copies all belong to main stage t + 2 - NE, which is neither
  // past the last nor the K-tail stage
  // (ext: the copies of this stage are K-extension units, issued through issue_load; a
  // compile-time choice, so the main stages keep their precomputed-offset copies)
  auto stage = [&](int t, int a, auto ext) {
    constexpr bool EXT = decltype(ext)::value;
    const int b1 = a == 4 ? 0 : a + 1;           // W of stage t
    const int a2 = a >= 3 ? a - 3 : a + 2;       // x of stage t + 1
    const int b2 = a2 == 4 ? 0 : a2 + 1;         // W of stage t + 1
    const int a3 = b2 == 4 ? 0 : b2 + 1;         // x of stage t + 2
    const char* xs = smem + a * P::SLOT_BYTES;
    const char* ws = smem + b1 * P::SLOT_BYTES;
    const char* xs2 = smem + a2 * P::SLOT_BYTES;
    const char* ws2 = smem + b2 * P::SLOT_BYTES;
    const int kb2 = (t + 2 - NE) * P::RB;
    char* const xdst = smem + a3 * P::SLOT_BYTES;
    char* const wdst = smem + a * P::SLOT_BYTES;
    // K-extension stage: its copies belong to extension stage e2 of group 0 or 1 (t + 2 < NE)
    const int s2 = t + 2;
    const bool g2 = EXT && s2 >= eg0.ns;
    const int e2 = g2 ? s2 - eg0.ns : s2;
    const int kbx2 = (g2 ? eg1.tcb : eg0.tcb) + e2 * P::RB;  // t~ columns of the stage
    const int kbw2 = e2 * P::RB;                              // B columns of the stage
    const int rkb2 = g2 ? eg1.rkb : eg0.rkb;
    auto ext_w_copy = [&](int it) {  // copy `it` of the B unit; chunks past the rank read zero
      const int slot0 = (it * P::WAVES + wave) * 64;
      uint32_t v = g2 ? ob1.v[it] : ob0.v[it];
      if (kbw2 + c_ext * 16 >= rkb2) v = 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(g2 ? br1 : br0, (lds_void*)(wdst + slot0 * 16), 16, v, kbw2, 0, 0);
    };
    // NF4: a main stage dequantizes the codes of stage t + 2 (loaded during stage t - 1, or by
    // the prologue for the first one) and loads those of stage t + 3 first thing, before its x
    // copies.
    constexpr bool DQ = NF4 && !EXT;
    const bool load_c = DQ && t + 3 < NS;
    // the dequantization sub-steps run SPB per bundle (one for the 256 x 256 tile's 128 bundles,
    // two for the 128 x 128 tile's 32), ending two bundles before the stage does, so that few
    // dequantized words wait in registers for the barrier; word j is written to the slot the
    // barrier releases at the bundle after its last sub-step, at the earliest at bundle j + 1 of
    // k-step 1 (bundles counted from the start of the stage)
    constexpr int SPB = NB >= 64 ? 1 : 2;
    constexpr int START = 2 * NB - 2 - ((NSUB - 1) / SPB + 1);
    auto write_bundle = [](int j) {
      const int done = START + (kNf4TableSteps + kNf4WordSteps * (j + 1) - 1) / SPB;
      return done + 1 > NB + 1 + j ? done + 1 : NB + 1 + j;
    };
    static_assert(!NF4 || (START >= 1 && START + (NSUB - 1) / SPB + 1 < 2 * NB && NB + WPT < 2 * NB),
                  "dequantization schedule");
    auto sub_steps = [&](int b) {  // the sub-steps of bundle b of the stage
      if (b < START) return;
#pragma unroll
      for (int q = 0; q < SPB; ++q) nf4_sub(c_work, SPB * (b - START) + q);
    };
    auto k0 = [&](int m) {  // bundle m of k-step 0
      const int i = m / P::NJ, j = m % P::NJ;
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[0].a[i], fr[0].b[j], acc[i][j], 0, 0, 0);
      if constexpr (DQ) __builtin_amdgcn_sched_barrier(0);  // (the bundle's VALU work after its MFMA)
      if (m % RS == 0) read_frag(fr[1], m / RS, xs, ws, 1);
      if constexpr (NF4) {
        if (m == 0) {
          if constexpr (DQ) {
            // the codes of stage t + 2 landed: loads issued after them are the previous stage's x
            // copies (the prologue waited for its own)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(NL));
            c_work = c_load;
#if defined(__HIP_DEVICE_COMPILE__)
            // (the copy stays here, after the wait, so that the next load may reuse the registers)
#pragma unroll
            for (int i = 0; i < WPT / 4; ++i)
              asm volatile("" : "+v"(c_work.q[i][0]), "+v"(c_work.q[i][1]), "+v"(c_work.q[i][2]), "+v"(c_work.q[i][3]));
            asm volatile("" : "+v"(c_work.a));
#endif
          }
          if (load_c) nfs.load(c_load, cr, ar, t + 3 - NE);
        }
        if constexpr (DQ) sub_steps(m);
      }
      if (m % LS == LS / 2) {
        if constexpr (EXT && NF4) issue_load(2 * t + 4, m / LS);
        else if constexpr (EXT) oxe.load_one(m / LS, xdst, tr, kbx2);
        else ox.load_one(m / LS, xdst, xr, kb2);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto k1 = [&](int m) {  // bundle m of k-step 1
      const int i = m / P::NJ, j = m % P::NJ;
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr[1].a[i], fr[1].b[j], acc[i][j], 0, 0, 0);
      if constexpr (DQ) {
        __builtin_amdgcn_sched_barrier(0);
        sub_steps(NB + m);
      }
      if (m == 0) {
        __builtin_amdgcn_sched_barrier(0);
        // x of stage t + 2 (and codes loaded by this stage) may still be in flight
        if (load_c) __builtin_amdgcn_s_waitcnt(waitcnt_vm(NL + NC));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(NL));
        stage_barrier();  // stage t + 1 landed and visible; every wave is done reading stage t
      } else if (m % RS == 1) {
        read_frag(fr[0], m / RS, xs2, ws2, 0);
      }
      if constexpr (DQ) {
#pragma unroll
        for (int w = 0; w < WPT; ++w)
          if (write_bundle(w) == NB + m) nf4_write(wdst, w);
      }
      if (m % LS == LS / 2) {
        if constexpr (EXT && NF4) issue_load(2 * t + 5, m / LS);
        else if constexpr (EXT) ext_w_copy(m / LS);
        else if constexpr (!NF4) ow.load_one(m / LS, wdst, wr, kb2);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NF4) {
      unrolled<NB>(k0);
      unrolled<NB>(k1);
    } else {
      // (one loop per k-step: one loop over both is past the compiler's full-unroll limit)
#pragma unroll
      for (int m = 0; m < NB; ++m) k0(m);
#pragma unroll
      for (int m = 0; m < NB; ++m) k1(m);
    }
  };

  // The last stages: their copies (if any) are whole main units, one of them
  // possibly the K-tail stage, so they go through the precomputed offsets.
  auto main_unit = [&](int u) {
    if (u >= NU) return;
    // (NF4: K is a multiple of 64, so the stages from t_end on have no units left to load)
    if constexpr (NF4) return;
    const int kb = ((u >> 1) - NE) * P::RB;
    const bool tl = k_tail && (u >> 1) == NS - 1;
    if (u & 1) ow.load(slot(u), wr, kb, tl, kb_total);
    else ox.load(slot(u), xr, kb, tl, kb_total);
  };
  auto tail_stage = [&](int t, int a) {
    const int b1 = a == 4 ? 0 : a + 1;
    const int a2 = a >= 3 ? a - 3 : a + 2;
    const int b2 = a2 == 4 ? 0 : a2 + 1;
    const char* xs = smem + a * P::SLOT_BYTES;
    const char* ws = smem + b1 * P::SLOT_BYTES;
    main_unit(2 * t + 4);
    ring_frags16<P>(fr[1], xs, ws, 1, fo);
    mfma_frags16<P>(acc, fr[0]);
    if (2 * t + 4 < NU) __builtin_amdgcn_s_waitcnt(waitcnt_vm(NL));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    stage_barrier();  // stage t + 1 landed and visible; every wave is done reading stage t
    main_unit(2 * t + 5);
    ring_frags16<P>(fr[0], smem + a2 * P::SLOT_BYTES, smem + b2 * P::SLOT_BYTES, 0, fo);
    mfma_frags16<P>(acc, fr[1]);
  };

  int a = 0;  // slot of x of stage t
  int t = 0;
  for (; t < t_ext && t + 1 < NS; ++t) {
    stage(t, a, std::true_type{});
    a = a >= 3 ? a - 3 : a + 2;
  }
  for (; t < t_end && t + 1 < NS; ++t) {
    stage(t, a, std::false_type{});
    a = a >= 3 ? a - 3 : a + 2;
  }
  for (; t + 1 < NS; ++t) {
    tail_stage(t, a);
    a = a >= 3 ? a - 3 : a + 2;
  }
  {  // last stage: no refill, no barrier
    const char* xs = smem + a * P::SLOT_BYTES;
    const char* ws = smem + (a == 4 ? 0 : a + 1) * P::SLOT_BYTES;
    ring_frags16<P>(fr[1], xs, ws, 1, fo);
    mfma_frags16<P>(acc, fr[0]);
    mfma_frags16<P>(acc, fr[1]);
  }

  __syncthreads();  // every wave is done reading the ring; LDS becomes the staging area
  if constexpr (P::WM == 128) epilogue_lds16<P>(acc, p, m0, n0, wm0, wn0, lane, wave, smem);
  else epilogue_lds16s<P>(acc, p, m0, n0, wm0, wn0, lane, wave, smem);
}

template <class P, bool NF4 = false>
hipError_t launch_flow16(const LinearProblem& p, hipStream_t s) {
  const int mt = static_cast<int>((p.T + P::BM - 1) / P::BM);
  const int nt = static_cast<int>((p.N + P::BN - 1) / P::BN);
  hipLaunchKernelGGL((gemm_flow16_kernel<P, NF4>), dim3(mt * nt), dim3(P::THREADS), 0, s, p, mt, nt);
  return hipGetLastError();
}


// General pipelined kernel (used when more than two adapter groups meet one tile).
using HotCfg = PCfg<256, 256, 64, 128, 64, 4>;
using Flow16Cfg = QCfg<256, 256, 128, 128, 128, 5>;
// 128 x 128 tiles, 4 waves of 64 x 64, two workgroups per CU: for layers whose
// 256 x 256 tiles would leave compute units idle (few tokens or narrow outputs).
using Flow16SCfg = QCfg<128, 128, 64, 64, 128, 5, 2>;

// Compute units of the current device (0 when the query fails).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

// Largest number of adapter groups whose columns meet one BN-wide output tile.
int max_groups_per_tile(const LinearProblem& p, int bn) {
  int worst = 0;
  for (int i = 0; i < p.n_groups; ++i) {
    const int64_t t_lo = p.g[i].col_off / bn, t_hi = (p.g[i].col_off + p.g[i].n_cols - 1) / bn;
    for (const int64_t t : {t_lo, t_hi}) {  // a tile meeting several groups holds an end of one of them
      int c = 0;
      for (int j = 0; j < p.n_groups; ++j)
        if (p.g[j].col_off < (t + 1) * bn && p.g[j].col_off + p.g[j].n_cols > t * bn) ++c;
      worst = c > worst ? c : worst;
    }
  }
  return worst;
}

// The hot kernel's entry point, named here so that its launch stub is always
// emitted (a kernel template used only through a launcher has lost it before).
template __global__ void gemm_flow16_kernel<Flow16Cfg>(LinearProblem, int, int);
template __global__ void gemm_flow16_kernel<Flow16SCfg>(LinearProblem, int, int);
template __global__ void gemm_flow16_kernel<Flow16SCfg, true>(LinearProblem, int, int);
template __global__ void gemm_flow16_kernel<Flow16Cfg, true>(LinearProblem, int, int);

hipError_t launch(const LinearProblem& p, hipStream_t s) {
  if (max_groups_per_tile(p, Flow16Cfg::BN) <= 2) {
    // The output tile (both give the same bits): 256 x 256, one workgroup per CU, or 128 x 128,
    // two per CU. The larger does more MFMA work per LDS byte; the smaller ran at 0.77-0.92 of
    // its rate on MI355X (1536- and 8960-wide inputs) but fills the last wave of tiles better and
    // pads fewer rows when T is not a multiple of 256. Estimated time, in units of one 128 x 128
    // tile's MFMA work (padding included) at the larger tile's rate: waves of 256 x 256 tiles
    // (one per CU) take 4 each, waves of 128 x 128 tiles (two per CU at 0.85 of the rate) take
    // 2 / 0.85. The smaller is taken when its estimate is lower (or when asked for). With T a
    // multiple of 256 this is the smaller tile's wave fill, discounted by 0.85, beating the
    // larger's; up to 128 tokens the smaller always wins (the larger's rows are half padding).
    const int64_t cus = device_cus();
    const int64_t t256 = ((p.T + 255) / 256) * ((p.N + 255) / 256);
    const int64_t t128 = ((p.T + 127) / 128) * ((p.N + 127) / 128);
    const double est256 = 4.0 * static_cast<double>((t256 + cus - 1) / (cus > 0 ? cus : 1));
    const double est128 = 2.0 / 0.85 * static_cast<double>((t128 + 2 * cus - 1) / (cus > 0 ? 2 * cus : 1));
    const bool small = p.tile == 2 || (p.tile == 0 && cus > 0 && est128 < est256);
    if (p.nf4) return small ? launch_flow16<Flow16SCfg, true>(p, s) : launch_flow16<Flow16Cfg, true>(p, s);
    return small ? launch_flow16<Flow16SCfg>(p, s) : launch_flow16<Flow16Cfg>(p, s);
  }
  if (p.nf4) return hipErrorInvalidValue;  // (a 4-bit weight has one adapter group)
  using P = HotCfg;
  const int mt = static_cast<int>((p.T + P::BM - 1) / P::BM);
  const int nt = static_cast<int>((p.N + P::BN - 1) / P::BN);
  hipLaunchKernelGGL(gemm_pipe_kernel<P>, dim3(mt * nt), dim3(P::THREADS), 0, s, p, mt, nt);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Rank-wide producer for the hot path: t~[m, t_col + q] = RN_bf16(s . sum_k x[m,k] A_g[q,k])
// for 128-token blocks and 128 adapter rows per workgroup, streamed with the
// same LDS ring (128-byte stages, 3 deep). Rows past the rank read as zero, so
// the padded columns of t~ come out as zeros. HBM-bound: it reads x once per
// 128-row chunk of each group.
namespace down {
// 128 tokens per workgroup, 4 waves along tokens; adapter rows per task: 64 (5-deep
// ring, ~64 KB of x in flight per CU) when every group's padded rank is 64, else 128.
using DP64 = PCfg<128, 64, 32, 64, 128, 5>;
using DP128 = PCfg<128, 128, 32, 128, 128, 4>;

// One pipelined K loop over NS stages for config P; issue(s) fills ring slot s % S.
template <class P, class Issue>
__device__ __forceinline__ void pipe_loop(f32x16 (&acc)[P::NI][P::NJ], char* smem, int NS, Issue&& issue,
                                          int wn0, int wm0, int lane) {
#pragma unroll
  for (int i = 0; i < P::NI; ++i)
#pragma unroll
    for (int j = 0; j < P::NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  for (int s = 0; s < P::S && s < NS; ++s) issue(s);
  wait_stages<P::LPS>(min(NS, P::S) - 1);
  stage_barrier();
  Frags<P> fr[2];
  load_frags<P>(fr[0], smem, 0, wn0, wm0, lane);
  auto run_stage = [&](int j, bool steady) {
    const char* st = smem + (j % P::S) * P::STAGE_BYTES;
#pragma unroll
    for (int kk = 0; kk < P::KK; ++kk) {
      if (kk + 1 < P::KK) {
        load_frags<P>(fr[(kk + 1) & 1], st, kk + 1, wn0, wm0, lane);
      } else {
        if (steady) wait_stages<P::LPS>(P::S - 2);
        else wait_stages<P::LPS>(min(NS - j - 2, P::S - 2));
        stage_barrier();
        if (steady) issue(j + P::S);
        load_frags<P>(fr[(kk + 1) & 1], smem + ((j + 1) % P::S) * P::STAGE_BYTES, 0, wn0, wm0, lane);
      }
      mfma_frags<P>(acc, fr[kk & 1]);
      interleave_reads_with_mfma<P>();
    }
  };
  int j = 0;
  for (; j + P::S < NS; ++j) run_stage(j, true);
  for (; j + 1 < NS; ++j) run_stage(j, false);
  const char* st = smem + ((NS - 1) % P::S) * P::STAGE_BYTES;
#pragma unroll
  for (int kk = 0; kk < P::KK; ++kk) {
    if (kk + 1 < P::KK) load_frags<P>(fr[(kk + 1) & 1], st, kk + 1, wn0, wm0, lane);
    mfma_frags<P>(acc, fr[kk & 1]);
  }
}

// Rows of A a group's producer tasks cover: its padded rank, or with SPLIT
// (fp32 adapter on bf16 activations) the 2 r_pad interleaved hi / lo rows of
// its bf16 split copy.
template <bool SPLIT>
__device__ __forceinline__ int producer_rows(const GroupDev& g) { return SPLIT ? 2 * g.r_pad : g.r_pad; }

// grid: (ceil(T / BM), total chunks of BN adapter rows over all groups)
// grid z: K splits of ks stages each (gridDim.z > 1 only without SPLIT): each
// writes its fp32 partial sums of x.A^T to p.tpart [z, T, ldt] and
// down_finish_kernel adds them.
template <class DP, bool SPLIT>
__global__ __launch_bounds__(DP::THREADS) void down_kernel(LinearProblem p, int ks) {
  using P = DP;
  __shared__ __attribute__((aligned(1024))) char smem[P::S * P::STAGE_BYTES];
  int c = static_cast<int>(blockIdx.y), gi = 0;
  while (gi + 1 < p.n_groups && c >= (producer_rows<SPLIT>(p.g[gi]) + P::BN - 1) / P::BN) {
    c -= (producer_rows<SPLIT>(p.g[gi]) + P::BN - 1) / P::BN;
    ++gi;
  }
  const GroupDev& g = p.g[gi];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = (wave % P::WAVES_M) * P::WM, wn0 = (wave / P::WAVES_M) * P::WN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * P::BM;
  const int rows_m = static_cast<int>(min<int64_t>(P::BM, p.T - m0));
  const int q0 = c * P::BN;
  const int rows_q = min(P::BN, (SPLIT ? 2 * g.r_pad : g.rank) - q0);
  const int kb_total = static_cast<int>(p.K * 2);
  const int nk = (kb_total + P::RB - 1) / P::RB;
  const bool k_tail = (kb_total % P::RB) != 0;
  const uint32_t ldx_b = static_cast<uint32_t>(p.ldx * 2), lda_b = static_cast<uint32_t>(p.K * 2);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(static_cast<const char*>(p.x) + m0 * p.ldx * 2, static_cast<uint32_t>(rows_m) * ldx_b);
  const char* a_src = static_cast<const char*>(SPLIT ? g.A2 : g.A);
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(a_src + static_cast<int64_t>(q0) * p.K * 2,
                                              static_cast<uint32_t>(max(rows_q, 0)) * lda_b);
  TileOffsets<P, P::BM> ox;
  TileOffsets<P, P::BN> oa;
  ox.init(ldx_b, 0, rows_m, 0);
  oa.init(lda_b, 0, rows_q, 0);
  const int s_lo = static_cast<int>(blockIdx.z) * ks;  // this split's stages [s_lo, s_lo + ns)
  const int ns = min(nk, s_lo + ks) - s_lo;
  auto issue = [&](int s) {
    char* bx = smem + (s % P::S) * P::STAGE_BYTES;
    const bool tail = k_tail && s_lo + s == nk - 1;
    ox.load(bx, xr, (s_lo + s) * P::RB, tail, kb_total);
    oa.load(bx + P::X_BYTES, ar, (s_lo + s) * P::RB, tail, kb_total);
  };
  f32x16 acc[P::NI][P::NJ];
  pipe_loop<P>(acc, smem, ns, issue, wn0, wm0, lane);

  // D[i = adapter row][j = token]: lane holds rows q0 + wn0 + 32 i + 8 gq + 4 h + e of token wm0 + r
  const int r = lane & 31, h = lane >> 5;
  const int64_t m = m0 + wm0 + r;
  if (m >= p.T) return;
  if (!SPLIT && gridDim.z > 1) {  // partial sums of this K split, unscaled
    float* part = p.tpart + (static_cast<int64_t>(blockIdx.z) * p.T + m) * p.ldt + g.t_col;
#pragma unroll
    for (int i = 0; i < P::NI; ++i)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int q = q0 + wn0 + i * 32 + gq * 8 + h * 4;
        if (q >= g.r_pad) continue;
        *reinterpret_cast<f32x4*>(part + q) =
            f32x4{acc[i][0][gq * 4], acc[i][0][gq * 4 + 1], acc[i][0][gq * 4 + 2], acc[i][0][gq * 4 + 3]};
      }
    return;
  }
  const float sc = g.scale;
  const bool unit = sc == 1.0f;
  bf16_bits* t = static_cast<bf16_bits*>(p.work);
  if (SPLIT) {
    // rows 2q, 2q + 1 hold x.hi(A[q]) and x.lo(A[q]): t = their fp32 sum, t~ = RN_f32(s t),
    // written as hi(t~) | hi(t~) | lo(t~) into the group's three r_pad-wide blocks
    bf16_bits* row = t + m * (3 * p.ldt) + 3 * g.t_col;
#pragma unroll
    for (int i = 0; i < P::NI; ++i) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int q = (q0 + wn0 + i * 32 + gq * 8 + h * 4) / 2;  // first of this lane's 2 ranks
        if (q >= g.r_pad) continue;
        bf16_bits hi[2], lo[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float tv = acc[i][0][gq * 4 + 2 * e] + acc[i][0][gq * 4 + 2 * e + 1];
          const float ts = unit ? tv : tv * sc;
          hi[e] = f32_to_bf16_rne(ts);
          lo[e] = f32_to_bf16_rne(ts - bf16_to_f32(hi[e]));
        }
        const uint32_t whi = static_cast<uint32_t>(hi[0]) | (static_cast<uint32_t>(hi[1]) << 16);
        const uint32_t wlo = static_cast<uint32_t>(lo[0]) | (static_cast<uint32_t>(lo[1]) << 16);
        *reinterpret_cast<uint32_t*>(row + q) = whi;
        *reinterpret_cast<uint32_t*>(row + g.r_pad + q) = whi;
        *reinterpret_cast<uint32_t*>(row + 2 * g.r_pad + q) = wlo;
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < P::NI; ++i) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int q = q0 + wn0 + i * 32 + gq * 8 + h * 4;
      if (q >= g.r_pad) continue;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = unit ? acc[i][0][gq * 4 + e] : acc[i][0][gq * 4 + e] * sc;
      uint2 w;
      w.x = pack_bf16x2(v[0], v[1]);
      w.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(t + m * p.ldt + g.t_col + q) = w;
    }
  }
}

// t~ = RN_bf16(s . sum of the K splits' partial sums, in split order): 4 columns per thread.
// The split count S is a template parameter, so all S loads of a thread issue before the first
// wait (with a run-time count each load sat behind a branch whose join waited for it).
template <int S>
__global__ __launch_bounds__(256) void down_finish_kernel(LinearProblem p) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= p.T * p.ldt) return;
  const int64_t m = i / p.ldt;
  const int col = static_cast<int>(i - m * p.ldt);
  f32x4 v[S];
#pragma unroll
  for (int z = 0; z < S; ++z) v[z] = *reinterpret_cast<const f32x4*>(p.tpart + (z * p.T + m) * p.ldt + col);
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int z = 0; z < S; ++z) sum += v[z];
  int gi = 0;
  while (gi + 1 < p.n_groups && col >= p.g[gi + 1].t_col) ++gi;
  const float sc = p.g[gi].scale;
  if (sc != 1.0f) sum *= sc;
  uint2 w;
  w.x = pack_bf16x2(sum[0], sum[1]);
  w.y = pack_bf16x2(sum[2], sum[3]);
  *reinterpret_cast<uint2*>(static_cast<bf16_bits*>(p.work) + i) = w;
}

// One instance of the finishing kernel per split count 2 .. kMaxProducerSplits; n selects it.
template <int S = 2>
hipError_t launch_down_finish(const LinearProblem& p, hipStream_t s, dim3 grid, int n) {
  if constexpr (S > kMaxProducerSplits) {
    return hipErrorInvalidValue;
  } else {
    if (n != S) return launch_down_finish<S + 1>(p, s, grid, n);
    hipLaunchKernelGGL((down_finish_kernel<S>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
  }
}

template <class DP, bool SPLIT>
hipError_t launch_cfg(const LinearProblem& p, hipStream_t s) {
  int chunks = 0;
  for (int i = 0; i < p.n_groups; ++i) chunks += ((SPLIT ? 2 * p.g[i].r_pad : p.g[i].r_pad) + DP::BN - 1) / DP::BN;
  int S = 1, ks = (static_cast<int>(p.K * 2) + DP::RB - 1) / DP::RB;
  if (!SPLIT && p.tpart != nullptr) producer_plan(p.T, p.K, &S, &ks);
  const dim3 grid(static_cast<unsigned>((p.T + DP::BM - 1) / DP::BM), static_cast<unsigned>(chunks),
                  static_cast<unsigned>(S));
  hipLaunchKernelGGL((down_kernel<DP, SPLIT>), grid, dim3(DP::THREADS), 0, s, p, ks);
  if (S > 1) {
    const int64_t quads = p.T * p.ldt / 4;
    return launch_down_finish(p, s, dim3(static_cast<unsigned>((quads + 255) / 256)), S);
  }
  return hipGetLastError();
}

hipError_t launch(const LinearProblem& p, hipStream_t s) {
  bool narrow = true;
  for (int i = 0; i < p.n_groups; ++i) narrow = narrow && p.g[i].r_pad <= DP64::BN;
  return narrow ? launch_cfg<DP64, false>(p, s) : launch_cfg<DP128, false>(p, s);
}

// fp32 adapter on bf16 activations: t~ as hi | hi | lo from the split copies of A
hipError_t launch_split(const LinearProblem& p, hipStream_t s) { return launch_cfg<DP128, true>(p, s); }
}  // namespace down
}  // namespace pipe

using MainCfg = Cfg<256, 256, 128, 64>;  // 8 waves: 2 along tokens x 4 along outputs

template <typename TA, typename TL>
hipError_t launch_fused(const LinearProblem& p, hipStream_t s) {
  using C = MainCfg;
  const int mt = static_cast<int>((p.T + C::BM - 1) / C::BM);
  const int nt = static_cast<int>((p.N + C::BN - 1) / C::BN);
  hipLaunchKernelGGL((fused_gemm_kernel<C, TA, TL>), dim3(mt * nt), dim3(C::THREADS), 0, s, p, mt, nt);
  return hipGetLastError();
}

template <typename TX, typename CT>
hipError_t launch_down(const LinearProblem& p, hipStream_t s) {
  int max_rpad = 0;
  for (int i = 0; i < p.n_groups; ++i) max_rpad = max_rpad > p.g[i].r_pad ? max_rpad : p.g[i].r_pad;
  const dim3 grid(static_cast<unsigned>((p.T + kDownBM - 1) / kDownBM), static_cast<unsigned>(p.n_groups),
                  static_cast<unsigned>((max_rpad + kDownBQ - 1) / kDownBQ));
  hipLaunchKernelGGL((lora_down_kernel<TX, CT>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Few tokens (skinny_path): row block b of 64 rows, 4 waves of 16; blocks
// b < nbw are weight rows, the rest the padded A rows of the groups in order
// (block b - nbw starts at column 64 (b - nbw) of the rank-wide layout). Grid y
// is the K chunk (a multiple of 128). Weight fragments go from global memory
// straight to registers through range-checked buffer loads (rows past the end
// and k past the chunk read as zeros), one 128-k group ahead of the MFMAs. The
// tokens' 128-k slice of a group is copied once per workgroup into LDS (two
// buffers, 16-byte pieces of a token row XOR-swizzled by the token's low 4 bits;
// tokens past T and k past the chunk read as zeros) and the 4 waves read their
// fragments from there. Within a group lane (r, q) takes the 32 consecutive k at 32 q and
// feeds them to v_mfma_f32_16x16x32_bf16 as 4 steps of 8 (step s: k = 32 q +
// 8 s + 0..7) for row r (the "A" operand) and for token 16 tb + r (the "B"
// operand) alike, so each step sums 32 distinct k and the 4 steps cover the
// group: the same dot product, with each lane's weight bytes contiguous (16
// code bytes of a 4-bit row, 64 bytes of a bf16 row, 128 of an fp32 A row).
// After the chunk a lane holds the partial sums of rows 4q .. 4q + 3 of token
// 16 tb + r. A 4-bit weight is looked up as byte pairs in an LDS table,
// multiplied by its block's absmax in fp32 and rounded to bf16; an fp32 A row
// is split exactly into hi = RN_bf16(v) and lo = RN_bf16(v - hi), both through
// the MFMA into the same fp32 sum.
__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }

constexpr uint32_t kOutOfRange = 0x80000000u;  // a buffer offset past every range: the load returns zeros
enum { kRowsBf16 = 0, kRowsNf4 = 1, kRowsF32 = 2 };

template <int KIND, int TB>
struct SkGroup {
  static constexpr int NW = KIND == kRowsBf16 ? 4 : (KIND == kRowsNf4 ? 1 : 8);  // 16-byte pieces of the row
  u32x4 w[NW];
  float am;          // 4-bit: the block's absmax
  u32x4 x[TB][4];    // token fragments of the 4 steps (read from LDS just before the MFMAs)
};

// LDS copy of a group's token slice: 16 tb + r tokens x 256 bytes, piece p of token row t
// at position p ^ (t & 15).
constexpr int kSkXBytes = 64 * 256;

struct SkSrc {
  __amdgpu_buffer_rsrc_t w, am, x;  // rows of this wave (from its first row), absmax likewise, all tokens
  uint32_t w_row_b, ldx_b;          // row strides in bytes
  int64_t K;
};

template <int KIND, int TB, bool XLDS>
__device__ __forceinline__ void sk_load(SkGroup<KIND, TB>& f, const SkSrc& src, int r, int q, int64_t kg,
                                        int64_t k_hi) {
  const int64_t kl = kg + 32 * q;  // the lane's first k of the group
  const uint32_t row = static_cast<uint32_t>(r) * src.w_row_b;
  if constexpr (KIND == kRowsNf4) {
    // K and the chunk ends are multiples of 64: the lane's 32 elements are all in
    // or all out, and sit inside one 64-element block
    const bool in = kl < k_hi;
    f.w[0] = __builtin_amdgcn_raw_buffer_load_b128(src.w, in ? row + static_cast<uint32_t>(kl / 2) : kOutOfRange, 0, 0);
    const uint32_t blk = static_cast<uint32_t>((static_cast<int64_t>(r) * src.K + kl) / 64);
    f.am = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(src.am, in ? blk * 4 : kOutOfRange, 0, 0));
  } else {
    constexpr int EB = KIND == kRowsF32 ? 4 : 2;  // element bytes; K is a multiple of 8 (whole pieces)
#pragma unroll
    for (int i = 0; i < SkGroup<KIND, TB>::NW; ++i) {
      const int64_t ke = kl + i * (16 / EB);
      f.w[i] = __builtin_amdgcn_raw_buffer_load_b128(
          src.w, ke < k_hi ? row + static_cast<uint32_t>(ke * EB) : kOutOfRange, 0, 0);
    }
  }
  if constexpr (!XLDS) {  // token fragments straight from global memory (L2)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int64_t ke = kl + 8 * st;
        const uint32_t off = static_cast<uint32_t>(tb * 16 + r) * src.ldx_b + static_cast<uint32_t>(ke * 2);
        f.x[tb][st] = __builtin_amdgcn_raw_buffer_load_b128(src.x, ke < k_hi ? off : kOutOfRange, 0, 0);
      }
  }
}

// Copy of the token slice of the group at kg into the LDS buffer xb: TB pieces per thread.
template <int TB>
__device__ __forceinline__ void sk_stage_x(char* xb, const SkSrc& src, int64_t kg, int64_t k_hi) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int it = 0; it < TB; ++it) {
    const int slot0 = it * 256 + wave * 64;  // wave-uniform LDS destination (16-byte slots)
    const int sl = slot0 + lane;
    const int row = sl >> 4, gp = (sl & 15) ^ (row & 15);  // token row, piece of the row it holds
    const int64_t ke = kg + 8 * gp;
    const uint32_t voff = ke < k_hi ? static_cast<uint32_t>(row) * src.ldx_b + static_cast<uint32_t>(ke * 2) : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.x, (lds_void*)(xb + slot0 * 16), 16, voff, 0, 0, 0);
  }
}

// This lane's token fragments of a staged group: token 16 tb + r, pieces 4 q + st.
template <int KIND, int TB>
__device__ __forceinline__ void sk_read_x(SkGroup<KIND, TB>& f, const char* xb, int r, int q) {
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int st = 0; st < 4; ++st)
      f.x[tb][st] = *reinterpret_cast<const u32x4*>(xb + ((tb * 16 + r) * 16 + ((4 * q + st) ^ r)) * 16);
}

template <int KIND, int TB>
__device__ __forceinline__ void sk_mma(f32x4 (&acc)[TB], const SkGroup<KIND, TB>& f, const f32x2* pair) {
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    if constexpr (KIND == kRowsF32) {
      const u32x4 v0 = f.w[2 * st], v1 = f.w[2 * st + 1];
      const float v[8] = {__uint_as_float(v0[0]), __uint_as_float(v0[1]), __uint_as_float(v0[2]),
                          __uint_as_float(v0[3]), __uint_as_float(v1[0]), __uint_as_float(v1[1]),
                          __uint_as_float(v1[2]), __uint_as_float(v1[3])};
      u32x4 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16_bits h0 = f32_to_bf16_rne(v[2 * e]), h1 = f32_to_bf16_rne(v[2 * e + 1]);
        const bf16_bits l0 = f32_to_bf16_rne(v[2 * e] - bf16_to_f32(h0));
        const bf16_bits l1 = f32_to_bf16_rne(v[2 * e + 1] - bf16_to_f32(h1));
        hi[e] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
        lo[e] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
      }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const bf16x8 xf = __builtin_bit_cast(bf16x8, f.x[tb][st]);
        acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi), xf, acc[tb], 0, 0, 0);
        acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lo), xf, acc[tb], 0, 0, 0);
      }
    } else {
      bf16x8 a;
      if constexpr (KIND == kRowsNf4) {
        const uint32_t w = f.w[0][st];  // 4 code bytes: elements 8 st .. 8 st + 7 of the lane's 32
        u32x4 o;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {  // byte bb: element 2 bb in bits 0-3, 2 bb + 1 in bits 4-7
          const f32x2 v = pair[(w >> (8 * bb)) & 0xffu];
          o[bb] = pack_bf16x2(v[0] * f.am, v[1] * f.am);
        }
        a = __builtin_bit_cast(bf16x8, o);
      } else {
        a = __builtin_bit_cast(bf16x8, f.w[st]);
      }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, f.x[tb][st]), acc[tb], 0, 0, 0);
    }
  }
}

// The chunk [k_lo, k_hi) of this wave's 16 rows, one group of loads ahead. With XLDS every
// wave of the workgroup runs the same groups (the token slices are shared through LDS);
// without it (at most 8 tokens, where the slice is at most 2 KB) each wave loads its token
// fragments itself and no barrier is needed.
template <int KIND, int TB, bool XLDS>
__device__ __forceinline__ void sk_chunk(f32x4 (&acc)[TB], const SkSrc& src, int r, int q, int64_t k_lo,
                                         int64_t k_hi, const f32x2* pair, char* xs) {
  SkGroup<KIND, TB> cur;
  if constexpr (!XLDS) {
    sk_load<KIND, TB, false>(cur, src, r, q, k_lo, k_hi);
    int64_t kg = k_lo;
    for (; kg + 128 < k_hi; kg += 128) {
      SkGroup<KIND, TB> nxt;
      sk_load<KIND, TB, false>(nxt, src, r, q, kg + 128, k_hi);
      sk_mma<KIND, TB>(acc, cur, pair);
      cur = nxt;
    }
    sk_mma<KIND, TB>(acc, cur, pair);
  } else {
    sk_stage_x<TB>(xs, src, k_lo, k_hi);
    sk_load<KIND, TB, true>(cur, src, r, q, k_lo, k_hi);
    __builtin_amdgcn_s_waitcnt(pipe::waitcnt_vm(0));
    __syncthreads();  // the first token slice is in LDS for every wave
    int64_t kg = k_lo;
    int b = 0;
    for (; kg + 128 < k_hi; kg += 128) {
      SkGroup<KIND, TB> nxt;
      // (buffer b ^ 1 was last read before the previous barrier)
      sk_stage_x<TB>(xs + (b ^ 1) * kSkXBytes, src, kg + 128, k_hi);
      sk_load<KIND, TB, true>(nxt, src, r, q, kg + 128, k_hi);
      sk_read_x<KIND, TB>(cur, xs + b * kSkXBytes, r, q);
      sk_mma<KIND, TB>(acc, cur, pair);
      __builtin_amdgcn_s_waitcnt(pipe::waitcnt_vm(0));
      __syncthreads();  // the next slice landed; every wave is done reading this one
      cur = nxt;
      b ^= 1;
    }
    sk_read_x<KIND, TB>(cur, xs + b * kSkXBytes, r, q);
    sk_mma<KIND, TB>(acc, cur, pair);
  }
}

template <bool NF4, bool AF32, int TB, bool XLDS>
__global__ __launch_bounds__(256) void skinny_kernel(LinearProblem p, int nbw, int64_t kchunk, int64_t npad) {
  __shared__ f32x2 pair[256];
  __shared__ __attribute__((aligned(16))) char xs[XLDS ? 2 * kSkXBytes : 16];
  if constexpr (NF4) {
    pair[threadIdx.x] = f32x2{p.codebook[threadIdx.x & 15], p.codebook[threadIdx.x >> 4]};
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int split = blockIdx.y;
  const int64_t k_lo = split * kchunk;
  const int64_t k_hi = min<int64_t>(p.K, k_lo + kchunk);
  f32x4 acc[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  SkSrc src;
  src.K = p.K;
  src.ldx_b = static_cast<uint32_t>(p.ldx * 2);
  src.x = make_rsrc(p.x, static_cast<uint32_t>(p.T) * src.ldx_b);
  const int b = blockIdx.x;
  if (b < nbw) {
    const int64_t n0 = static_cast<int64_t>(b) * kSkinnyRows + wave * 16;
    // (wave-uniform by construction; readfirstlane keeps the buffer descriptors in scalar registers)
    const int64_t rows = __builtin_amdgcn_readfirstlane(static_cast<int>(max<int64_t>(0, min<int64_t>(16, p.N - n0))));
    if constexpr (NF4) {
      src.w_row_b = static_cast<uint32_t>(p.K / 2);
      src.w = make_rsrc(p.codes + n0 * (p.K / 2), static_cast<uint32_t>(rows) * src.w_row_b);
      src.am = make_rsrc(p.absmax + n0 * (p.K / 64), static_cast<uint32_t>(rows * (p.K / 64) * 4));
      sk_chunk<kRowsNf4, TB, XLDS>(acc, src, r, q, k_lo, k_hi, pair, xs);
    } else {
      src.w_row_b = static_cast<uint32_t>(p.K * 2);
      src.w = make_rsrc(static_cast<const bf16_bits*>(p.W) + n0 * p.K, static_cast<uint32_t>(rows) * src.w_row_b);
      sk_chunk<kRowsBf16, TB, XLDS>(acc, src, r, q, k_lo, k_hi, pair, xs);
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int64_t t = tb * 16 + r;
      if (t < p.T) *reinterpret_cast<f32x4*>(p.skinny + (split * p.T + t) * npad + n0 + 4 * q) = acc[tb];
    }
    return;
  }
  // adapter rows: x . A_g^T into the rank-wide partial sums
  const int rb = (b - nbw) * kSkinnyRows;
  int gi = 0;
  while (gi + 1 < p.n_groups && rb >= p.g[gi + 1].t_col) ++gi;
  const GroupDev& g = p.g[gi];
  const int q0 = rb - g.t_col + wave * 16;  // first A row of this wave
  const int64_t rows = __builtin_amdgcn_readfirstlane(max(0, min(16, g.rank - q0)));
  if constexpr (AF32) {
    src.w_row_b = static_cast<uint32_t>(p.K * 4);
    src.w = make_rsrc(static_cast<const float*>(g.A) + static_cast<int64_t>(q0) * p.K,
                      static_cast<uint32_t>(rows) * src.w_row_b);
    sk_chunk<kRowsF32, TB, XLDS>(acc, src, r, q, k_lo, k_hi, pair, xs);
  } else {
    src.w_row_b = static_cast<uint32_t>(p.K * 2);
    src.w = make_rsrc(static_cast<const bf16_bits*>(g.A) + static_cast<int64_t>(q0) * p.K,
                      static_cast<uint32_t>(rows) * src.w_row_b);
    sk_chunk<kRowsBf16, TB, XLDS>(acc, src, r, q, k_lo, k_hi, pair, xs);
  }
  float* pt = p.skinny + static_cast<int64_t>(gridDim.y) * p.T * npad;
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int64_t t = tb * 16 + r;
    if (t < p.T) *reinterpret_cast<f32x4*>(pt + (split * p.T + t) * p.ldt + g.t_col + q0 + 4 * q) = acc[tb];
  }
}

// Second kernel of the skinny path: grid (ceil(N / 256), ceil(T / TOK)), TOK = 4
// tokens per block. The block first forms t~ = RN_adt(s . t) of its TOK tokens in LDS (t = the K
// chunks' partial sums added in chunk order), then each thread takes one output
// column: acc = the weight partial sums in chunk order, += t~ . B_g^T in fp32
// (rank index ascending) for the group covering the column, + bias, one
// rounding. Token rows past T repeat the last token and columns past N read
// column N - 1 (valid memory); neither is stored. The chunk count S is a
// template parameter, so a thread issues all its partial-sum loads before it
// waits for any of them; each 8-rank piece of t~ is read from LDS as 16-byte
// vectors before its FMAs. (Both measured on MI355X, with the same bits: a
// 64-token FFN-up call went from 29.1 to 26.4 us, FFN down from 26.4 to 24.3.)
template <bool AF32, int kFinishTokens, int S>
__global__ __launch_bounds__(256) void skinny_finish_kernel(LinearProblem p, int64_t npad) {
  extern __shared__ float tt[];  // [kFinishTokens, ldt]
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kFinishTokens;
  const int ldt = static_cast<int>(p.ldt);
  const float* pt = p.skinny + static_cast<int64_t>(S) * p.T * npad;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  // this thread's weight partial sums, loaded first: their latency overlaps the t~ phase.
  // Every load is issued (a column past N reads column N - 1 and is never stored), with the chunk
  // count fixed at compile time, so that none waits for another.
  float v[kFinishTokens][S];
  const float* pc = p.skinny + min<int64_t>(n, p.N - 1);
#pragma unroll
  for (int i = 0; i < kFinishTokens; ++i) {
    const int64_t t = min<int64_t>(t0 + i, p.T - 1);
#pragma unroll
    for (int s = 0; s < S; ++s) v[i][s] = pc[(s * p.T + t) * npad];
  }
  for (int c = threadIdx.x; c < kFinishTokens * ldt; c += 256) {
    const int j = c / ldt, col = c - j * ldt;
    const int64_t t = min<int64_t>(t0 + j, p.T - 1);
    float v[S];
#pragma unroll
    for (int s = 0; s < S; ++s) v[s] = pt[(s * p.T + t) * ldt + col];
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) sum += v[s];
    int gi = 0;
    while (gi + 1 < p.n_groups && col >= p.g[gi + 1].t_col) ++gi;
    const float sc = p.g[gi].scale;
    if (sc != 1.0f) sum *= sc;
    tt[c] = AF32 ? sum : bf16_to_f32(f32_to_bf16_rne(sum));
  }
  __syncthreads();
  if (n >= p.N) return;
  float acc[kFinishTokens];
#pragma unroll
  for (int i = 0; i < kFinishTokens; ++i) {
    acc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) acc[i] += v[i][s];
  }
  for (int gi = 0; gi < p.n_groups; ++gi) {
    const GroupDev& g = p.g[gi];
    if (n < g.col_off || n >= g.col_off + g.n_cols) continue;
    const int64_t row = (n - g.col_off) * g.rank;
    const float* tg = tt + g.t_col;
    int qq = 0;
    // the row of B in 16-byte pieces when its start keeps that alignment (B itself is 16-byte aligned)
    constexpr int PE = AF32 ? 4 : 8;  // elements per piece
    if (g.rank % PE == 0) {
      for (; qq < g.rank; qq += PE) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const char*>(g.B) + (row + qq) * (AF32 ? 4 : 2));
        float bv[PE];
#pragma unroll
        for (int e = 0; e < PE; ++e)
          bv[e] = AF32 ? __uint_as_float(w[e]) : __uint_as_float(e & 1 ? w[e >> 1] & 0xffff0000u : w[e >> 1] << 16);
        // this piece's t~ of every token, read as 16-byte vectors before the FMAs (t_col and
        // ldt are multiples of the rank padding and qq of PE: 16-byte aligned)
        f32x4 tv[kFinishTokens][PE / 4];
#pragma unroll
        for (int i = 0; i < kFinishTokens; ++i)
#pragma unroll
          for (int h = 0; h < PE / 4; ++h) tv[i][h] = *reinterpret_cast<const f32x4*>(tg + i * ldt + qq + 4 * h);
#pragma unroll
        for (int e = 0; e < PE; ++e)
#pragma unroll
          for (int i = 0; i < kFinishTokens; ++i) acc[i] = fmaf(tv[i][e >> 2][e & 3], bv[e], acc[i]);
      }
    }
    for (; qq < g.rank; ++qq) {
      const float bv = AF32 ? static_cast<const float*>(g.B)[row + qq]
                            : bf16_to_f32(static_cast<const bf16_bits*>(g.B)[row + qq]);
#pragma unroll
      for (int i = 0; i < kFinishTokens; ++i) acc[i] = fmaf(tg[i * ldt + qq], bv, acc[i]);
    }
  }
  const bool has_bias = p.bias != nullptr || p.bias32 != nullptr;
  const float bias = p.bias32 != nullptr ? p.bias32[n]
                     : (p.bias != nullptr ? bf16_to_f32(static_cast<const bf16_bits*>(p.bias)[n]) : 0.f);
#pragma unroll
  for (int i = 0; i < kFinishTokens; ++i) {
    if (t0 + i < p.T)
      static_cast<bf16_bits*>(p.y)[(t0 + i) * p.ldy + n] = f32_to_bf16_rne(has_bias ? acc[i] + bias : acc[i]);
  }
}

// One instance of the finishing kernel per chunk count 1 .. kSkinnyMaxChunks; n selects it.
template <bool AF32, int TOK, int S = 1>
hipError_t launch_finish(const LinearProblem& p, hipStream_t s, dim3 grid, size_t shmem, int n, int64_t npad) {
  if constexpr (S > kSkinnyMaxChunks) {
    return hipErrorInvalidValue;
  } else {
    if (n != S) return launch_finish<AF32, TOK, S + 1>(p, s, grid, shmem, n, npad);
    hipLaunchKernelGGL((skinny_finish_kernel<AF32, TOK, S>), grid, dim3(256), shmem, s, p, npad);
    return hipGetLastError();
  }
}

template <bool NF4, bool AF32>
hipError_t launch_skinny_tb(const LinearProblem& p, hipStream_t s, dim3 grid, int nbw, int64_t kchunk,
                            int64_t npad) {
  // (token slices through LDS from 9 tokens on: below that they are at most 2 KB per group and
  // the per-group barrier costs about what the shared copy saves; the results are the same)
  switch ((p.T + 15) / 16) {
    case 1:
      if (p.T <= 8) hipLaunchKernelGGL((skinny_kernel<NF4, AF32, 1, false>), grid, dim3(256), 0, s, p, nbw, kchunk, npad);
      else hipLaunchKernelGGL((skinny_kernel<NF4, AF32, 1, true>), grid, dim3(256), 0, s, p, nbw, kchunk, npad);
      break;
    case 2: hipLaunchKernelGGL((skinny_kernel<NF4, AF32, 2, true>), grid, dim3(256), 0, s, p, nbw, kchunk, npad); break;
    case 3: hipLaunchKernelGGL((skinny_kernel<NF4, AF32, 3, true>), grid, dim3(256), 0, s, p, nbw, kchunk, npad); break;
    default: hipLaunchKernelGGL((skinny_kernel<NF4, AF32, 4, true>), grid, dim3(256), 0, s, p, nbw, kchunk, npad); break;
  }
  return hipGetLastError();
}

hipError_t launch_skinny(const LinearProblem& p, hipStream_t s) {
  int S;
  int64_t kchunk;
  skinny_plan(p.K, &S, &kchunk);
  const int nbw = static_cast<int>((p.N + kSkinnyRows - 1) / kSkinnyRows);
  const int nba = static_cast<int>(p.ldt / kSkinnyRows);
  const int64_t npad = skinny_npad(p.N);
  const bool af32 = p.n_groups > 0 && p.adapter == Elt::F32;
  const dim3 grid(static_cast<unsigned>(nbw + nba), static_cast<unsigned>(S));
  hipError_t e;
  if (p.nf4) e = af32 ? launch_skinny_tb<true, true>(p, s, grid, nbw, kchunk, npad)
                      : launch_skinny_tb<true, false>(p, s, grid, nbw, kchunk, npad);
  else e = af32 ? launch_skinny_tb<false, true>(p, s, grid, nbw, kchunk, npad)
                : launch_skinny_tb<false, false>(p, s, grid, nbw, kchunk, npad);
  if (e != hipSuccess) return e;
  // t~ of a block's tokens in LDS: 4 x ldt fp32, at most 64 KB (ldt <= 4096). (8 tokens per
  // block halves the re-reads of B but measured slower at every token count from 1 to 64:
  // half the blocks, and below 8 tokens duplicated work.)
  constexpr int tok = 4;
  const dim3 fgrid(static_cast<unsigned>((p.N + 255) / 256), static_cast<unsigned>((p.T + tok - 1) / tok));
  const size_t shmem = static_cast<size_t>(tok) * static_cast<size_t>(p.ldt) * 4;
  return af32 ? launch_finish<true, tok>(p, s, fgrid, shmem, S, npad)
              : launch_finish<false, tok>(p, s, fgrid, shmem, S, npad);
}

}  // namespace

// Split copies of an fp32 adapter (layout in GroupDev): hi(v) = RN_bf16(v) and
// lo(v) = RN_bf16(v - hi(v)), where v - hi(v) is exact in fp32, so hi + lo
// carries v to about 16 significant bits.
__global__ __launch_bounds__(256) void split_a_kernel(const float* __restrict__ A, int rank, int r_pad, int64_t K,
                                                      bf16_bits* __restrict__ A2) {
  const int64_t n = 2 * static_cast<int64_t>(r_pad) * K;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t row = i / K, k = i - row * K;
    const int q = static_cast<int>(row >> 1);
    const float v = q < rank ? A[q * K + k] : 0.f;
    const bf16_bits hi = f32_to_bf16_rne(v);
    A2[i] = (row & 1) ? f32_to_bf16_rne(v - bf16_to_f32(hi)) : hi;
  }
}

__global__ __launch_bounds__(256) void split_b_kernel(const float* __restrict__ B, int rank, int r_pad,
                                                      int64_t n_cols, bf16_bits* __restrict__ B2) {
  const int w = 3 * r_pad;
  const int64_t n = n_cols * w;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t row = i / w;
    const int c = static_cast<int>(i - row * w);
    const int seg = c / r_pad, q = c - seg * r_pad;
    const float v = q < rank ? B[row * rank + q] : 0.f;
    const bf16_bits hi = f32_to_bf16_rne(v);
    B2[i] = seg == 1 ? f32_to_bf16_rne(v - bf16_to_f32(hi)) : hi;
  }
}

// 4-bit weight, many tokens: the whole weight dequantized once into the bf16
// panel [N, K] (the same element value as inside the GEMM: RN_bf16 of the fp32
// product codebook[code] * absmax). Lane t of a wave writes the 16 output bytes
// at t * 16 + j * 1024 of the wave's 4 KB (2048 elements) for j = 0 .. 3, so
// every load and store instruction of the wave covers one contiguous range:
// 8 elements = one code dword, one absmax. Both nibbles of a code byte come from
// a 256-entry LDS table of codebook pairs in one 8-byte read.
constexpr int kPanelWaveElems = 2048;

__global__ __launch_bounds__(256) void nf4_panel_kernel(const uint8_t* __restrict__ codes,
                                                        const float* __restrict__ absmax,
                                                        const float* __restrict__ codebook, int64_t n_elems,
                                                        bf16_bits* __restrict__ panel) {
  __shared__ f32x2 pair[256];
  pair[threadIdx.x] = f32x2{codebook[threadIdx.x & 15], codebook[threadIdx.x >> 4]};
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t wstride = static_cast<int64_t>(gridDim.x) * 4;
  for (int64_t wv = wave0; wv * kPanelWaveElems < n_elems; wv += wstride) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t e0 = wv * kPanelWaveElems + j * 512 + lane * 8;  // first of this lane's 8 elements
      if (e0 >= n_elems) continue;  // n_elems is a multiple of 64: 8 elements are all in or all out
      const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + e0 / 2);
      const float a = absmax[e0 >> 6];
      u32x4 o;
#pragma unroll
      for (int b = 0; b < 4; ++b) {  // byte b holds elements e0 + 2b (bits 0-3) and e0 + 2b + 1 (bits 4-7)
        const f32x2 v = pair[(w >> (8 * b)) & 0xffu];
        o[b] = pack_bf16x2(v[0] * a, v[1] * a);
      }
      *reinterpret_cast<u32x4*>(panel + e0) = o;
    }
  }
}

hipError_t launch_nf4_panel(const LinearProblem& p, hipStream_t s) {
  const int64_t n = p.N * p.K;
  const int64_t waves = (n + kPanelWaveElems - 1) / kPanelWaveElems;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL(nf4_panel_kernel, dim3(static_cast<unsigned>(blocks < 8192 ? blocks : 8192)), dim3(256), 0, s,
                     p.codes, p.absmax, p.codebook, n, static_cast<bf16_bits*>(p.panel));
  return hipGetLastError();
}

// The split path's phase 1: split copies of every group, then the producer.
hipError_t split_producer(const LinearProblem& p, hipStream_t s) {
  for (int i = 0; i < p.n_groups; ++i) {
    const GroupDev& g = p.g[i];
    const int64_t na = 2 * static_cast<int64_t>(g.r_pad) * p.K, nb = g.n_cols * 3 * g.r_pad;
    const unsigned ga = static_cast<unsigned>((na + 255) / 256 < 4096 ? (na + 255) / 256 : 4096);
    const unsigned gb = static_cast<unsigned>((nb + 255) / 256 < 4096 ? (nb + 255) / 256 : 4096);
    hipLaunchKernelGGL(split_a_kernel, dim3(ga), dim3(256),
                       0, s, static_cast<const float*>(g.A), g.rank, g.r_pad, p.K, static_cast<bf16_bits*>(g.A2));
    hipLaunchKernelGGL(split_b_kernel, dim3(gb), dim3(256),
                       0, s, static_cast<const float*>(g.B), g.rank, g.r_pad, g.n_cols,
                       static_cast<bf16_bits*>(g.B2));
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return pipe::down::launch_split(p, s);
}

// The split path's phase 2: the hot GEMM over bf16 groups of rank 3 r_pad
// (t_hi | t_hi | t_lo against hi(B) | lo(B) | hi(B)).
hipError_t split_gemm(const LinearProblem& p, hipStream_t s) {
  LinearProblem q = p;
  q.adapter = Elt::BF16;
  q.ldt = 3 * p.ldt;
  for (int i = 0; i < q.n_groups; ++i) {
    GroupDev& g = q.g[i];
    g.B = g.B2;
    g.rank = 3 * g.r_pad;
    g.r_pad = 3 * g.r_pad;
    g.t_col = 3 * g.t_col;
  }
  return pipe::launch(q, s);
}

// b + sum_g u_g . c_g over the legacy lora_B biases, fp32, groups in order (one thread per column);
// u_g = strength_g . request_scale: the legacy vector takes the adapter strength, not alpha / rank.
__global__ __launch_bounds__(256) void bias32_kernel(LinearProblem p) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (n >= p.N) return;
  float v = 0.f;
  if (p.bias != nullptr)
    v = p.act == Elt::BF16 ? bf16_to_f32(static_cast<const bf16_bits*>(p.bias)[n]) : static_cast<const float*>(p.bias)[n];
  for (int gi = 0; gi < p.n_groups; ++gi) {
    const GroupDev& g = p.g[gi];
    if (g.Bb == nullptr || n < g.col_off || n >= g.col_off + g.n_cols) continue;
    const int64_t j = n - g.col_off;
    const float c = p.adapter == Elt::BF16 ? bf16_to_f32(static_cast<const bf16_bits*>(g.Bb)[j])
                                           : static_cast<const float*>(g.Bb)[j];
    v += g.bscale * c;
  }
  p.bias32[n] = v;
}

hipError_t launch_bias32(const LinearProblem& p, hipStream_t s) {
  hipLaunchKernelGGL(bias32_kernel, dim3(static_cast<unsigned>((p.N + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_lossless(const LinearProblem& p, hipStream_t s, int phase) {
  if (p.T == 0) return hipSuccess;
  // few tokens: the rank-wide product runs inside the same launches (phase 1 has nothing to do)
  if (p.skinny != nullptr) return phase == 1 ? hipSuccess : launch_skinny(p, s);
  if (p.nf4 && p.panel == nullptr) {
    // dequantized inside the hot GEMM (bf16 activations and adapter, one group whose rank is a
    // multiple of 8, K a multiple of 64)
    const bool ok = p.act == Elt::BF16 && p.adapter == Elt::BF16 && p.K % 64 == 0 &&
                    (p.n_groups == 0 || (p.n_groups == 1 && p.g[0].rank % 8 == 0));
    if (!ok) return hipErrorInvalidValue;
    if (p.n_groups > 0 && phase != 2) {
      const hipError_t e = pipe::down::launch(p, s);
      if (e != hipSuccess) return e;
    }
    return phase == 1 ? hipSuccess : pipe::launch(p, s);
  }
  if (p.nf4) {
    // the weight dequantized once into the panel, then the bf16 path over it
    if (phase != 2) {
      const hipError_t e = launch_nf4_panel(p, s);
      if (e != hipSuccess) return e;
    }
    LinearProblem q = p;
    q.nf4 = false;
    q.W = p.panel;
    q.codes = nullptr;
    q.absmax = nullptr;
    q.codebook = nullptr;
    q.panel = nullptr;
    return launch_lossless(q, s, phase);
  }
  const bool act_bf16 = p.act == Elt::BF16, ad_bf16 = p.adapter == Elt::BF16;
  // fp32 adapter on bf16 activations: the adapter products on bf16 MFMA over the hi / lo split
  if (split_fp32_adapter(p.act, p.adapter, p.nf4)) {
    if (p.n_groups > 0 && phase != 2) {
      const hipError_t e = split_producer(p, s);
      if (e != hipSuccess) return e;
    }
    return phase == 1 ? hipSuccess : split_gemm(p, s);
  }
  bool ranks_ok = true;
  for (int i = 0; i < p.n_groups; ++i) ranks_ok = ranks_ok && (p.g[i].rank % 8 == 0);
  // hot path: streaming rank-wide producer, then the pipelined fused GEMM
  if (act_bf16 && ad_bf16 && !p.nf4 && ranks_ok) {
    if (p.n_groups > 0 && phase != 2) {
      const hipError_t e = pipe::down::launch(p, s);
      if (e != hipSuccess) return e;
    }
    return phase == 1 ? hipSuccess : pipe::launch(p, s);
  }
  // other dtypes / 4-bit weight / ragged ranks: producer kernel, then the fused GEMM
  if (p.n_groups > 0 && phase != 2) {
    hipError_t e;
    if (act_bf16 && ad_bf16) e = launch_down<bf16_bits, bf16_bits>(p, s);
    else if (act_bf16) e = launch_down<bf16_bits, float>(p, s);
    else e = launch_down<float, float>(p, s);
    if (e != hipSuccess) return e;
  }
  if (phase == 1) return hipSuccess;
  // (a 4-bit weight took the few-token path or the panel, an fp32 adapter on bf16 activations the split path)
  if (act_bf16) return launch_fused<bf16_bits, bf16_bits>(p, s);
  return launch_fused<float, float>(p, s);
}

}  // namespace lora
