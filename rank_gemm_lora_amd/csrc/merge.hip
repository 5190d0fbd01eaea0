// Merge of an adapter into a plain dense weight, W <- RN_w(W + s . B.A), lossless
// tier (piper-offload README, "LoRA merge" and merge_lora: an in-place addmm_
// into a plain dense base; FastVideo lora_patch page, DenseLoRAPatch.apply_to:
// the sum is taken in fp32 and cast back once). s = (alpha / rank) . strength.
//
// The rank product is a dense contraction over the rank, so with a bf16
// adapter it runs on v_mfma_f32_16x16x32_bf16: a workgroup owns 64 weight rows
// x 128 columns; the A columns of its 128 k are staged transposed in LDS (k
// rows of 64 ranks, 16-byte chunks XOR-swizzled by row), the MFMA "A" operand
// is A^T (k), the "B" operand the rows of B (n), so each lane ends with 4
// consecutive k of one weight row and updates them in place: one fp32
// multiply-add with s and one rounding to the weight's dtype. The kernel is
// bound by the weight's read and write (about 32 FLOP per byte at rank 64).
// An fp32 adapter takes a plain fp32 FMA loop (same contract, one rounding).
#include "common.hpp"
#include "launch.hpp"

namespace lora {
namespace {

constexpr int kMergeRows = 64;   // weight rows per workgroup (4 waves of 16)
constexpr int kMergeCols = 128;  // weight columns per workgroup (8 blocks of 16)
constexpr int kMergeBlocks = kMergeCols / 16;
constexpr int kMergeQ = 64;      // ranks staged per pass (128-byte LDS rows)

__device__ __forceinline__ int mswz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

template <typename TW>
__device__ __forceinline__ float load_w(const TW* p) {
  if constexpr (sizeof(TW) == 2) return bf16_to_f32(*reinterpret_cast<const bf16_bits*>(p));
  else return *p;
}

// The weight tile (64 rows x 128 columns) travels in whole 256-byte (bf16) or
// 512-byte (fp32) row segments: its loads are issued first, it is parked in its own
// LDS region with the first ranks' A^T, updated there by the lanes and written
// back the same way. Ranks are staged 64 at a time, zero-padded to a multiple
// of 32 (one MFMA step); steps past the rank are skipped.
constexpr int kMergeAtBytes = kMergeCols * 128;  // A^T: 128 k rows x 64 ranks (bf16)

template <typename TW>
__global__ __launch_bounds__(256, 4) void merge_mfma_kernel(TW* __restrict__ W, int64_t N, int64_t K,
                                                         const bf16_bits* __restrict__ A,
                                                         const bf16_bits* __restrict__ B, int rank, float s) {
  constexpr int EW = sizeof(TW);
  __shared__ __attribute__((aligned(1024))) char lds[kMergeAtBytes + kMergeRows * kMergeCols * EW];
  char* const ldsw = lds + kMergeAtBytes;  // the weight tile
  constexpr int ROW_B = kMergeCols * EW;        // bytes of a tile row
  constexpr int PIECES = kMergeRows * ROW_B / 16 / 256;  // 16-byte pieces per thread (8 bf16, 16 fp32)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * kMergeCols;
  const int64_t nt0 = static_cast<int64_t>(blockIdx.y) * kMergeRows;
  const int64_t n = nt0 + wave * 16 + r;  // this lane's B row
  const bool vec_b = (rank % 8) == 0;

  // the weight tile, coalesced: piece p of the tile is row p / (ROW_B / 16), bytes 16 (p % (ROW_B / 16))
  const int64_t kcols = min<int64_t>(kMergeCols, K - k0);
  u32x4 wreg[PIECES];
#pragma unroll
  for (int it = 0; it < PIECES; ++it) {
    const int piece = it * 256 + static_cast<int>(threadIdx.x);
    const int row = piece / (ROW_B / 16), cb = (piece % (ROW_B / 16)) * 16;
    wreg[it] = u32x4{0u, 0u, 0u, 0u};
    if (nt0 + row < N && cb / EW < kcols)  // K is a multiple of 8: a piece is all in or all out
      wreg[it] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(W + (nt0 + row) * K + k0) + cb);
  }

  // weight tile in LDS: row-major, 16-byte pieces rotated by row against bank conflicts
  auto wpos = [&](int row, int cb) { return row * ROW_B + ((cb + row * 16) % ROW_B); };
  f32x4 acc[kMergeBlocks];
#pragma unroll
  for (int j = 0; j < kMergeBlocks; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int qc = 0; qc < rank; qc += kMergeQ) {
    const int qn = min(kMergeQ, (rank - qc + 31) / 32 * 32);  // ranks staged this pass (32 or 64)
    __syncthreads();  // every wave is done reading the previous ranks
    // A[qc + qq][k0 + kk .. + 8] -> A^T rows kk .. kk + 7, column qq; columns past the rank are zero
    for (int piece = static_cast<int>(threadIdx.x); piece < qn * (kMergeCols / 8); piece += 256) {
      const int qq = piece / (kMergeCols / 8), kk = (piece % (kMergeCols / 8)) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qc + qq < rank && k0 + kk < K)
        v = *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(qc + qq) * K + k0 + kk);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<bf16_bits*>(lds + mswz(kk + e, qq >> 3) * 16 + (qq & 7) * 2) =
            static_cast<bf16_bits>(v[e >> 1] >> (16 * (e & 1)));
    }
    if (qc == 0) {  // the weight tile into its LDS region (its registers are free from here on)
#pragma unroll
      for (int it = 0; it < PIECES; ++it) {
        const int piece = it * 256 + static_cast<int>(threadIdx.x);
        const int row = piece / (ROW_B / 16), cb = (piece % (ROW_B / 16)) * 16;
        *reinterpret_cast<u32x4*>(ldsw + wpos(row, cb)) = wreg[it];
      }
    }
    __syncthreads();
    for (int st = 0; st < qn / 32; ++st) {  // 32 ranks per MFMA step
      const int q8 = qc + st * 32 + 8 * q;  // this lane's 8 ranks of the step
      u32x4 bw = {0u, 0u, 0u, 0u};
      if (n < N) {
        if (vec_b && q8 < rank) {
          bw = *reinterpret_cast<const u32x4*>(B + n * rank + q8);
        } else if (!vec_b) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (q8 + e < rank) bw[e >> 1] |= static_cast<uint32_t>(B[n * rank + q8 + e]) << (16 * (e & 1));
        }
      }
      const bf16x8 bf = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
      for (int j = 0; j < kMergeBlocks; ++j) {
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(lds + mswz(j * 16 + r, st * 4 + q) * 16);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[j], 0, 0, 0);
      }
    }
  }

  // lane (r, q) of column block j holds (B.A)[n][k0 + 16 j + 4 q + e], e = 0..3: one fp32
  // multiply-add with s, one rounding, in place in LDS
  const int lrow = wave * 16 + r;
#pragma unroll
  for (int j = 0; j < kMergeBlocks; ++j) {
    char* wp = ldsw + wpos(lrow, (j * 16 + 4 * q) * EW);
    if constexpr (EW == 2) {
      const uint2 w = *reinterpret_cast<const uint2*>(wp);
      const float w4[4] = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                           __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
      uint2 o;
      o.x = pack_bf16x2(fmaf(s, acc[j][0], w4[0]), fmaf(s, acc[j][1], w4[1]));
      o.y = pack_bf16x2(fmaf(s, acc[j][2], w4[2]), fmaf(s, acc[j][3], w4[3]));
      *reinterpret_cast<uint2*>(wp) = o;
    } else {
      const f32x4 w = *reinterpret_cast<const f32x4*>(wp);
      *reinterpret_cast<f32x4*>(wp) = f32x4{fmaf(s, acc[j][0], w[0]), fmaf(s, acc[j][1], w[1]),
                                           fmaf(s, acc[j][2], w[2]), fmaf(s, acc[j][3], w[3])};
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < PIECES; ++it) {
    const int piece = it * 256 + static_cast<int>(threadIdx.x);
    const int row = piece / (ROW_B / 16), cb = (piece % (ROW_B / 16)) * 16;
    if (nt0 + row < N && cb / EW < kcols)
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(W + (nt0 + row) * K + k0) + cb) =
          *reinterpret_cast<const u32x4*>(ldsw + wpos(row, cb));
  }
}

// fp32 adapter: thread per 4 consecutive k of one row; sum over the rank in fp32 FMAs.
template <typename TW>
__global__ __launch_bounds__(256) void merge_f32_kernel(TW* __restrict__ W, int64_t N, int64_t K,
                                                        const float* __restrict__ A, const float* __restrict__ B,
                                                        int rank, float s) {
  const int64_t quads = K / 4;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= N * quads) return;
  const int64_t n = i / quads, k = (i - n * quads) * 4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < rank; ++q) {
    const float b = B[n * rank + q];
    const f32x4 a = *reinterpret_cast<const f32x4*>(A + static_cast<int64_t>(q) * K + k);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(b, a[e], acc[e]);
  }
  TW* w = W + n * K + k;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = fmaf(s, acc[e], load_w(w + e));
  if constexpr (sizeof(TW) == 2) {
    uint2 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(w) = o;
  } else {
    *reinterpret_cast<f32x4*>(w) = f32x4{v[0], v[1], v[2], v[3]};
  }
}

}  // namespace

hipError_t launch_merge(void* W, Elt wdt, int64_t N, int64_t K, const void* A, const void* B, int rank, Elt adt,
                        float s, hipStream_t st) {
  if (adt == Elt::BF16) {
    const dim3 grid(static_cast<unsigned>((K + kMergeCols - 1) / kMergeCols),
                    static_cast<unsigned>((N + kMergeRows - 1) / kMergeRows));
    if (wdt == Elt::BF16)
      hipLaunchKernelGGL(merge_mfma_kernel<bf16_bits>, grid, dim3(256), 0, st, static_cast<bf16_bits*>(W), N, K,
                         static_cast<const bf16_bits*>(A), static_cast<const bf16_bits*>(B), rank, s);
    else
      hipLaunchKernelGGL(merge_mfma_kernel<float>, grid, dim3(256), 0, st, static_cast<float*>(W), N, K,
                         static_cast<const bf16_bits*>(A), static_cast<const bf16_bits*>(B), rank, s);
  } else {
    const int64_t threads = N * (K / 4);
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
    if (wdt == Elt::BF16)
      hipLaunchKernelGGL(merge_f32_kernel<bf16_bits>, grid, dim3(256), 0, st, static_cast<bf16_bits*>(W), N, K,
                         static_cast<const float*>(A), static_cast<const float*>(B), rank, s);
    else
      hipLaunchKernelGGL(merge_f32_kernel<float>, grid, dim3(256), 0, st, static_cast<float*>(W), N, K,
                         static_cast<const float*>(A), static_cast<const float*>(B), rank, s);
  }
  return hipGetLastError();
}

}  // namespace lora
