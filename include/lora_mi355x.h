/*
 * lora_mi355x.h -- fused LoRA linear for AMD Instinct MI355X (gfx950).
 *
 * The layer computes
 *
 *     y = x . W^T + b + s . (x . A^T) . B^T,   s = (alpha / rank) . strength . request_scale
 *
 * (SGLang PR #43501 "[diffusion] Add the dynamic LoRA delta inside the second
 * GEMM", Motivation and Modifications; the delta is B @ A as on the FastVideo
 * lora_patch page). The rank-r update is added into the base GEMM's fp32
 * accumulator, the bias goes into the epilogue, and the [tokens, out] delta is
 * never materialized.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are row-major. x [T, K] with row stride ldx (elements), W [N, K]
 *   (row stride K), bias [N], A [r, K] (row stride K), B [N, r] (row stride r),
 *   y [T, N] with row stride ldy >= N, so a column view of a wider output is
 *   y + offset with the wider ldy.
 * - Every tensor pointer is DEVICE memory owned by the caller, unless a
 *   parameter says "host". The library never allocates device memory in a
 *   call; it uses the caller's workspace, sized by lora_linear_workspace_size().
 * - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL = the
 *   null stream); calls return without synchronizing.
 * - Status: 0 (LORA_OK) or a positive lora_status. Every argument is validated
 *   before anything is launched: on a nonzero status nothing has been written.
 *   A failed launch returns LORA_ERR_HIP; faults inside a kernel surface at the
 *   caller's next synchronization.
 * - Scales are plain per-call arguments: nothing is cached between calls (the
 *   request scale must be honoured per request -- SGLang PR #43501,
 *   Modifications, "Why not alpha").
 * - s == +-0, or A == B == NULL, leaves the adapter inactive: y is the base
 *   output (zero strengths are inactive -- piper-offload README, strengths; no
 *   adapter means plain X.W -- Unsloth fast-LoRA chapter, section 6).
 *   A non-finite alpha, strength or request_scale is LORA_ERR_NONFINITE
 *   (FastVideo DenseLoRAPatch rejects a non-finite strength).
 * - Calls on distinct streams with distinct output and workspace buffers may
 *   run concurrently; the library holds no mutable global state apart from
 *   the per-device scratch array of lora_linear_fwd_noalloc (see there).
 *
 * Quality tiers (SGLang PR #43501, Modifications):
 * - LORA_LOSSLESS (default): one fused pass. t~ = RN_adt(s . (x . A^T)) is
 *   formed in fp32 and rounded once to the adapter dtype, t~ . B^T is added to
 *   the base GEMM's fp32 accumulator, then y = RN_dt(acc + b).
 * - LORA_EXACT: the separate-pass chain, bit for bit: every GEMM sums products
 *   in fp64 with k ascending and rounds once to fp32; base = RN_dt(RN_f32(G +
 *   b)); t = RN_adt(G(x, A)); d = RN_adt(G(t, B)); d is multiplied by
 *   alpha/rank, strength and request_scale in turn (each rounded to fp32,
 *   skipped when exactly 1), rounding to adt after each; y = RN_dt(RN_f32(base
 *   + d)). Slow by design; kept for bitwise reproducibility.
 *
 * Alignment (LORA_ERR_ALIGN): in the lossless tier x, W, A, B, the 4-bit codes
 * and the workspace must be 16-byte aligned, and K and ldx must be multiples of
 * 16 bytes' worth of elements (8 for bf16, 4 for fp32); y, ldy and the bias
 * only need natural element alignment. The exact tier and dense_patch_apply
 * only need natural element alignment.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
typedef enum { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype;

/* Quality tier; LORA_LOSSLESS is the default (SGLang PR #43501, Modifications). */
typedef enum { LORA_LOSSLESS = 0, LORA_EXACT = 1 } lora_quality;

/* Where a lossless 4-bit call with more than 64 tokens dequantizes its weight
 * (lora_linear_nf4_fwd_ex): chosen from the shape, once per call into a bf16
 * panel, or inside the GEMM (Unsloth fast-LoRA chapter, section 3). */
typedef enum { LORA_NF4_AUTO = 0, LORA_NF4_PANEL = 1, LORA_NF4_IN_GEMM = 2 } lora_nf4_dequant;

/* Dense payloads (FastVideo lora_patch page):
 * LORA_PATCH_ADD     -- .diff / .diff_b  (DenseLoRAPatch.apply_to)
 * LORA_PATCH_REPLACE -- .set_weight      (DenseLoRAPatch.replacement_for) */
typedef enum { LORA_PATCH_ADD = 0, LORA_PATCH_REPLACE = 1 } lora_patch_mode;

typedef enum {
  LORA_OK = 0,
  LORA_ERR_NULL_PTR = 1,     /* a required pointer is NULL, or only one of A/B is given      */
  LORA_ERR_SHAPE = 2,        /* negative/zero size, ld too small, shape mismatch, bad groups */
  LORA_ERR_DTYPE = 3,        /* unsupported dtype or dtype combination                       */
  LORA_ERR_NONFINITE = 4,    /* alpha, strength or request_scale is NaN or infinite          */
  LORA_ERR_ALIGN = 5,        /* pointer or stride misaligned for the lossless kernels        */
  LORA_ERR_OVERLAP = 6,      /* output overlaps an input or the workspace                    */
  LORA_ERR_WORKSPACE = 7,    /* workspace NULL or smaller than lora_linear_workspace_size()  */
  LORA_ERR_UNSUPPORTED = 8,  /* device is not gfx950, or a limit below is exceeded           */
  LORA_ERR_HIP = 9           /* a HIP runtime call or kernel launch failed                   */
} lora_status;

/* Limits (LORA_ERR_UNSUPPORTED beyond them). */
#define LORA_MAX_GROUPS 8
#define LORA_MAX_RANK 1024

/*
 * One adapter of a stacked layer (q/k/v or gate/up), covering the output
 * columns [col_offset, col_offset + n_cols). A [rank, K] and B [n_cols, rank]
 * are device pointers in the adapter dtype; its combined scale is
 * (alpha / rank) . strength . request_scale. Groups must not overlap and must
 * lie inside [0, N_total). Columns outside every group get the base output.
 */
typedef struct lora_group {
  const void* A;
  const void* B;
  int32_t rank;
  int32_t reserved; /* set to 0 */
  double alpha;
  int64_t col_offset;
  int64_t n_cols;
} lora_group;

/*
 * lora_linear_fwd -- one LoRA linear layer.
 *
 *   x        [T, K] act_dtype, row stride ldx >= K
 *   W        [N, K] act_dtype
 *   bias     [N] act_dtype, or NULL
 *   A, B     [rank, K], [N, rank] adapter_dtype, or both NULL (base only)
 *   y        [T, N] act_dtype, row stride ldy >= N; must not overlap any input
 *   act_dtype     LORA_BF16 (adapter LORA_BF16 or LORA_F32), or LORA_F32 (adapter LORA_F32)
 *   quality       LORA_LOSSLESS or LORA_EXACT
 *   workspace     device scratch of at least lora_linear_workspace_size(T, K, N, &rank, 1, ...)
 *                 bytes (may be NULL when that size is 0); its contents are not
 *                 preserved between calls
 * T == 0 is a valid no-op.
 */
int lora_linear_fwd(const void* x, int64_t T, int64_t K, int64_t ldx,
                    const void* W, int64_t N, const void* bias,
                    const void* A, const void* B, int32_t rank, int32_t adapter_dtype,
                    double alpha, double strength, double request_scale,
                    void* y, int64_t ldy, int32_t act_dtype, int32_t quality,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * lora_linear_fwd_noalloc -- lora_linear_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and results (bit for bit), and no allocation of any kind. The
 * scratch those kernels need comes from one file-scope device array of
 * LORA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until the
 * process ends; its device address is looked up (hipGetSymbolAddress) on the
 * first call on each device.
 *   LORA_ERR_UNSUPPORTED when the call would need more scratch than that, i.e.
 *   when lora_linear_workspace_size(T, K, N, &rank, A || B ? 1 : 0,
 *   adapter_dtype, quality) > LORA_NOALLOC_SCRATCH_BYTES; otherwise the status
 *   of lora_linear_fwd.
 * Every call on one GPU shares that GPU's array and leaves its contents behind:
 * calls that can overlap in time on one GPU (different streams, or threads
 * without ordering) race on it and must not be mixed; calls ordered on one
 * stream are fine. No part of it needs to start at zero: each kernel writes
 * every scratch element it reads.
 */
#define LORA_NOALLOC_SCRATCH_BYTES (64ull * 1024ull * 1024ull)
int lora_linear_fwd_noalloc(const void* x, int64_t T, int64_t K, int64_t ldx,
                            const void* W, int64_t N, const void* bias,
                            const void* A, const void* B, int32_t rank, int32_t adapter_dtype,
                            double alpha, double strength, double request_scale,
                            void* y, int64_t ldy, int32_t act_dtype, int32_t quality, void* stream);

/*
 * lora_linear_fwd_phase -- lora_linear_fwd (lossless tier) with its two launches
 * selectable and the hot GEMM's output tile fixed by the caller, for callers
 * that schedule, time or compare the kernels of the path (SGLang PR #43501,
 * Modifications: the scale is applied to the rank-wide intermediate, then the
 * second LoRA product lands on the base output).
 *
 *   phase 0  the whole call, exactly lora_linear_fwd
 *   phase 1  writes the rank-wide intermediate RN_adt(s . x A^T) into the workspace
 *            (nothing when the adapter is inactive: s == 0 or A == B == NULL)
 *   phase 2  runs the fused GEMM y = RN(x W^T + t~ B^T + bias) reading that
 *            intermediate; the workspace must still hold what a phase-1 call with
 *            the same x, A, ranks and scales wrote (the library cannot check this)
 *   gemm_tile  0 picks the output tile from the layer's shape (128 x 128 when the
 *            256 x 256 tiles would fill less than three quarters of the compute
 *            units), 1 always 256 x 256, 2 always 128 x 128. Both tiles accumulate
 *            every output in the same order and give bitwise-identical results;
 *            only speed differs. Calls that do not reach the hot GEMM ignore it
 *            (64 tokens or fewer, fp32 activations, bf16 ranks not a multiple of 8).
 * Phase 1 then phase 2 on one stream gives exactly the output of lora_linear_fwd.
 * Arguments, validation and status codes as lora_linear_fwd; phase or gemm_tile
 * outside 0..2, or quality other than LORA_LOSSLESS, returns LORA_ERR_UNSUPPORTED.
 * Nothing is kept between calls.
 */
int lora_linear_fwd_phase(int32_t phase, int32_t gemm_tile, const void* x, int64_t T, int64_t K, int64_t ldx,
                          const void* W, int64_t N, const void* bias,
                          const void* A, const void* B, int32_t rank, int32_t adapter_dtype,
                          double alpha, double strength, double request_scale,
                          void* y, int64_t ldy, int32_t act_dtype, int32_t quality,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * lora_linear_stacked_fwd -- one base GEMM over W [N_total, K] with up to
 * LORA_MAX_GROUPS adapters, each added to its own column range of y
 * (SGLang PR #43501, Modifications: stacked q/k/v or gate/up adapters, one
 * update per group on column views of the output).
 * The result equals one lora_linear_fwd call per group on column views of y, bit
 * for bit, in the exact tier, at T <= 64, and wherever at most two groups meet any
 * 256-column block of y (groups of 256 columns or more, as q/k/v and gate/up have).
 * With more groups per block the lossless result meets the same accuracy bar but
 * may differ in the last bit (the extension is accumulated in another order).
 *
 *   groups    HOST array of n_groups lora_group (0 <= n_groups <= LORA_MAX_GROUPS);
 *             the A/B pointers inside are device pointers
 *   workspace at least lora_linear_workspace_size(T, K, N_total, ranks of the groups, n_groups, ...)
 *             bytes
 * Other arguments as lora_linear_fwd.
 */
int lora_linear_stacked_fwd(const void* x, int64_t T, int64_t K, int64_t ldx,
                            const void* W, int64_t N_total, const void* bias,
                            const lora_group* groups, int32_t n_groups, int32_t adapter_dtype,
                            double strength, double request_scale,
                            void* y, int64_t ldy, int32_t act_dtype, int32_t quality,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * One adapter of lora_linear_multi_fwd: like lora_group, plus its own strength
 * and the optional legacy lora_B bias of older adapters (piper-offload README,
 * LoRA resource: a <module>.lora_B.bias vector that merge mode adds to the
 * layer's bias with the same adapter strength). Its combined scale is
 * s = (alpha / rank) . strength . request_scale; its legacy vector takes
 * u = strength . request_scale (alpha / rank belongs to the factor pair).
 */
typedef struct lora_adapter {
  const void* A;       /* [rank, K] adapter dtype (device)                        */
  const void* B;       /* [n_cols, rank] adapter dtype (device)                   */
  const void* B_bias;  /* [n_cols] adapter dtype (device), or NULL                */
  int32_t rank;
  int32_t reserved;    /* set to 0 */
  double alpha;
  double strength;
  int64_t col_offset;  /* columns [col_offset, col_offset + n_cols) of y          */
  int64_t n_cols;
} lora_adapter;

/*
 * lora_linear_multi_fwd -- several adapters on one layer, summed independently
 * (piper-offload README, routed mode: y = base(x) + strength . (B.A.x + bias),
 * several LoRAs on one target summed independently; InvokeAI article,
 * section 3: a layer's list of (patch, weight) pairs):
 *
 *     y = x.W^T + b + sum_i [ s_i . (x.A_i^T).B_i^T + u_i . c_i ]   on adapter i's columns
 *
 * where c_i is adapter i's B_bias (0 when NULL), s_i its combined scale and
 * u_i = strength_i . request_scale. Column ranges may overlap; an adapter with
 * s_i == +-0 (or A = B = NULL) contributes nothing, its bias included.
 * Lossless tier: each t~_i = RN_adt(s_i . x.A_i^T) is a K-extension of the same
 * accumulator; b + sum_i u_i . c_i is formed in fp32 (u_i rounded to fp32 once)
 * and added in the epilogue before the one rounding. Exact tier: per adapter in
 * the order given, its delta chain and add (as lora_linear_fwd's), then its
 * legacy vector as its own payload: e = c_i multiplied by strength_i and then
 * request_scale (each rounded to fp32, skipped when exactly 1, rounding to the
 * adapter dtype after each), y = RN_dt(RN_f32(y + e)).
 *   adapters  HOST array of n_adapters (0 <= n_adapters <= LORA_MAX_GROUPS)
 *   workspace at least lora_linear_multi_workspace_size(...) bytes
 * Other arguments as lora_linear_fwd; B_bias must be naturally aligned and must
 * not overlap y. LORA_ERR_NONFINITE also when |u_i| of an active adapter with a
 * B_bias exceeds the fp32 range.
 */
int lora_linear_multi_fwd(const void* x, int64_t T, int64_t K, int64_t ldx,
                          const void* W, int64_t N, const void* bias,
                          const lora_adapter* adapters, int32_t n_adapters, int32_t adapter_dtype,
                          double request_scale, void* y, int64_t ldy, int32_t act_dtype, int32_t quality,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * lora_linear_nf4_fwd -- LoRA linear over a 4-bit codebook base weight,
 * dequantized inside the GEMM (Unsloth fast-LoRA chapter, section 3,
 * matmul_lora; 4-bit formats are blockwise -- piper-offload README
 * quantized-format table; InvokeAI article, NF4 section).
 *
 *   codes     uint8 [N, K/2]: row n, byte j holds element (n, 2j) in bits 0-3 and
 *             element (n, 2j+1) in bits 4-7
 *   absmax    fp32 [N*K/blocksize]: one scale per block of `blocksize` consecutive
 *             elements of the row-major [N, K] weight
 *   codebook  fp32 [16] (device)
 *   blocksize must be 64; K must be a multiple of 64
 * The weight element is W[n,k] = RN_bf16(RN_f32(codebook[code] * absmax[(n*K+k)/64]))
 * in both tiers. Activations, bias and y are bf16; the adapter is bf16 or fp32.
 *   workspace at least lora_linear_nf4_workspace_size(T, K, N, rank, adapter_dtype,
 *             quality) bytes. In the lossless tier with T > 64 it includes room for
 *             a bf16 copy of the dequantized weight ([N, K], rewritten by every
 *             call that uses it): above 256 tokens dequantizing once per call is
 *             cheaper than once per output tile. The weight is dequantized inside
 *             the kernel that reads it up to 64 tokens, up to 256 tokens with a
 *             bf16 adapter whose rank is a multiple of 8 (or no adapter), and in
 *             the exact tier; lora_linear_nf4_fwd_ex names the choice.
 */
int lora_linear_nf4_fwd(const void* x, int64_t T, int64_t K, int64_t ldx,
                        const uint8_t* codes, const float* absmax, const float* codebook,
                        int32_t blocksize, int64_t N, const void* bias,
                        const void* A, const void* B, int32_t rank, int32_t adapter_dtype,
                        double alpha, double strength, double request_scale,
                        void* y, int64_t ldy, int32_t quality,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * lora_linear_nf4_fwd_ex -- lora_linear_nf4_fwd with the place of the
 * dequantization named (Unsloth fast-LoRA chapter, section 3: dequantizing the
 * whole weight into a temporary per forward, against doing it where the GEMM
 * reads it). Lossless tier, T > 64 (below that the few-token kernel dequantizes
 * in registers whatever is asked; the exact tier ignores the argument):
 *   LORA_NF4_PANEL    once per call into a bf16 copy of the weight in the
 *                     workspace, then the bf16 GEMM over it
 *   LORA_NF4_IN_GEMM  inside the GEMM: each output tile of 128 tokens turns the
 *                     codes of its 128 weight rows into bf16 in registers and
 *                     LDS; needs a bf16 adapter whose rank is a multiple of 8
 *                     (or no adapter), LORA_ERR_UNSUPPORTED otherwise
 *   LORA_NF4_AUTO     what lora_linear_nf4_fwd does: the GEMM form up to 256
 *                     tokens (where it measured faster on MI355X) when it applies,
 *                     the panel otherwise
 * Both forms give the same weight, RN_bf16(RN_f32(codebook[code] * absmax)),
 * and the same output bits. Other values: LORA_ERR_UNSUPPORTED.
 * lora_linear_nf4_workspace_size covers every choice; the in-GEMM form needs only
 * lora_linear_workspace_size(T, K, N, &rank, 1, adapter_dtype, quality) bytes.
 */
int lora_linear_nf4_fwd_ex(const void* x, int64_t T, int64_t K, int64_t ldx,
                           const uint8_t* codes, const float* absmax, const float* codebook,
                           int32_t blocksize, int64_t N, const void* bias,
                           const void* A, const void* B, int32_t rank, int32_t adapter_dtype,
                           double alpha, double strength, double request_scale,
                           void* y, int64_t ldy, int32_t quality, int32_t dequant,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * dense_patch_apply -- dense payloads of an adapter, applied in place
 * (FastVideo lora_patch page, DenseLoRAPatch.apply_to / replacement_for):
 *
 *   LORA_PATCH_ADD:     dst = RN_dst( RN_f32( dst + RN_f32( src * RN_f32(strength) ) ) )
 *   LORA_PATCH_REPLACE: dst = RN_dst( RN_f32( src * RN_f32(strength) ) )
 *
 * The sum is taken in fp32 whatever the operand dtypes (a bf16 sum would
 * round away a delta three orders of magnitude below the weight); one
 * rounding back to dst's dtype; no fused multiply-add.
 *   dst_shape, src_shape  HOST arrays of dst_ndim / src_ndim sizes; the full shapes
 *                         must be equal (LORA_ERR_SHAPE otherwise), both tensors contiguous
 *   strength              finite (LORA_ERR_NONFINITE otherwise)
 * src must not overlap dst.
 */
int dense_patch_apply(void* dst, int32_t dst_dtype, const int64_t* dst_shape, int32_t dst_ndim,
                      const void* src, int32_t src_dtype, const int64_t* src_shape, int32_t src_ndim,
                      double strength, int32_t mode, void* stream);

/*
 * lora_merge_apply -- merge an adapter into a plain dense weight, in place
 * (piper-offload README, LoRA merge and merge_lora: an in-place addmm_ into a
 * plain dense base; FastVideo lora_patch page: the sum in fp32, one cast back):
 *
 *     W <- RN_w( W + s . B.A ),   s = (alpha / rank) . strength
 *
 *   W      [N, K] w_dtype (bf16 or fp32), row-major, updated in place
 *   A, B   [rank, K], [N, rank] adapter_dtype
 *   LORA_LOSSLESS  the rank product summed in fp32, s . (B.A) added to fp32(W)
 *                  in one multiply-add, one rounding to w_dtype; needs W, A, B
 *                  16-byte aligned and K a multiple of 8
 *   LORA_EXACT     G = RN_f32(sum over q ascending of B[n,q] A[q,k], in fp64),
 *                  d = RN_f32(G . RN_f32(s)) (skipped when RN_f32(s) == 1),
 *                  W <- RN_w(RN_f32(W + d)): the dense-payload chain with the
 *                  rank product as its delta
 * s == +-0 leaves W unchanged (nothing is launched); W must not overlap A or B.
 * A bf16 merge rounds away every part of the update below half a bf16 spacing
 * of the weight: the reason the SGLang PR keeps such adapters dynamic.
 */
int lora_merge_apply(void* W, int32_t w_dtype, int64_t N, int64_t K, const void* A, const void* B, int32_t rank,
                     int32_t adapter_dtype, double alpha, double strength, int32_t quality, void* stream);

/*
 * lora_linear_bwd -- gradients of the lossless bf16 LoRA linear for an output
 * gradient dy, the base weight frozen (Unsloth fast-LoRA chapter, sections 2
 * and 4: closed-form dX, dA, dB computed directly, the frozen weight needed
 * only for dX):
 *
 *     u = dy.B,  dx = dy.W + s.u.A,  dA = s.u^T.x,  dB = s.dy^T.(x.A^T),  db = sum over tokens of dy
 *
 * with s = (alpha / rank) . strength . request_scale.
 *   x [T, K] (ldx), W [N, K], A [rank, K], B [N, rank], dy [T, N] (lddy): bf16, 16-byte aligned,
 *   K, N, ldx and lddy multiples of 8
 *   dx [T, K] bf16 (row stride lddx), dA [rank, K], dB [N, rank], db [N] fp32: each optional (NULL = not
 *   computed); they must not overlap the inputs, the workspace or each other
 * Rounding: u~ = RN_bf16(s.u) and t~ = RN_bf16(s.x.A^T) as in the forward; dx = RN_bf16(dy.W + u~.A)
 * with one fp32 accumulator; dA = u~^T.x, dB = dy^T.t~ and db summed in fp32 over token chunks added in
 * a fixed order. T == 0 writes zero gradients.
 *   t_tilde   optional bf16 [T, ldt] (device): t~ of these x, A and s as the forward computed it, its
 *             first rank_pad(rank) columns read (rank_pad rounds the rank up to a multiple of 64;
 *             columns past the rank hold zeros). A lossless lora_linear_fwd call with bf16
 *             activations and adapter, T > 64 and this adapter alone leaves exactly that at the
 *             start of its workspace, ldt = rank_pad(rank); its workspace must then be kept
 *             unchanged until this call. Given, the backward does not read x a second time
 *             to recompute t~ (the gradients are the same bits). NULL: t~ is recomputed.
 *             ldt >= rank_pad(rank) when t_tilde is given (else LORA_ERR_SHAPE); t_tilde must not
 *             overlap the outputs or the workspace (LORA_ERR_OVERLAP).
 *   workspace at least lora_linear_bwd_workspace_size(T, K, N, rank, dx != NULL) bytes
 */
int lora_linear_bwd(const void* x, int64_t T, int64_t K, int64_t ldx, const void* W, int64_t N, const void* A,
                    const void* B, int32_t rank, double alpha, double strength, double request_scale, const void* dy,
                    int64_t lddy, void* dx, int64_t lddx, float* dA, float* dB, float* db, const void* t_tilde,
                    int64_t ldt, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of lora_linear_bwd (transposed copies, the rank-wide intermediates, partial sums). */
size_t lora_linear_bwd_workspace_size(int64_t T, int64_t K, int64_t N, int32_t rank, int32_t want_dx);

/*
 * Workspace bytes a call with T tokens, K inputs and N outputs needs for
 * adapters of the given ranks (`ranks` is a HOST array of n_ranks entries: one
 * for lora_linear_fwd and lora_linear_nf4_fwd, one per group for
 * lora_linear_stacked_fwd; n_ranks may be 0 for a call without adapters). It
 * holds the rank-wide intermediate [T, R] in the adapter dtype, R = the sum of
 * the ranks rounded up to multiples of 64. A lossless call with an fp32
 * adapter on bf16 activations runs the adapter products on bf16 MFMA over an
 * exact hi + lo split of each fp32 value, so its workspace holds the
 * intermediate as [T, 3 R] bf16 plus the split copies of A ([2 R, K]) and B (at
 * most [N, 3 R]), each region 256-byte aligned. A lossless call with at most 64
 * tokens on bf16 activations splits K into S chunks (S = ceil(K / c), c =
 * max(512, round_up(ceil(K / 32), 128))) and needs S fp32 partial sums of the
 * outputs and of x.A^T instead ([S, T, round_up(N, 64) + R] fp32);
 * for T <= 64 the larger of the layouts is returned. Returns 0 when T, K or
 * N <= 0, or when no rank is positive and T > 64.
 */
size_t lora_linear_workspace_size(int64_t T, int64_t K, int64_t N, const int32_t* ranks, int32_t n_ranks,
                                  int32_t adapter_dtype, int32_t quality);

/*
 * Workspace bytes of a lora_linear_nf4_fwd call: the adapter's share as
 * lora_linear_workspace_size (rank 0 = no adapter), plus, in the lossless tier
 * with T > 64, the dequantized weight panel (N * K * 2 bytes, 256-byte aligned
 * after the adapter's share). Returns 0 when T, K or N <= 0.
 */
size_t lora_linear_nf4_workspace_size(int64_t T, int64_t K, int64_t N, int32_t rank, int32_t adapter_dtype,
                                      int32_t quality);

/*
 * Workspace bytes of a lora_linear_multi_fwd call: as lora_linear_workspace_size
 * over the adapters' ranks, plus, in the lossless tier when an adapter with a
 * nonzero strength has a B_bias, an fp32 vector [N] at the front (256-byte
 * aligned). Returns 0 when T, K or N <= 0 (or as lora_linear_workspace_size).
 */
size_t lora_linear_multi_workspace_size(int64_t T, int64_t K, int64_t N, const lora_adapter* adapters,
                                        int32_t n_adapters, int32_t adapter_dtype, int32_t quality);

/* Static, human-readable text for a status code. */
const char* lora_status_string(int status);

/* LORA_OK when the current HIP device is a gfx950; LORA_ERR_UNSUPPORTED otherwise. */
int lora_device_check(void);

/*
 * lora_mfma_probe -- device measurement for reporting, not part of the layer.
 * Launches `blocks` workgroups of 8 waves, each issuing `iters` x 64 (8 chains of
 * 8) v_mfma_f32_16x16x32_bf16 back to back (no memory traffic in the loop): the
 * sustained matrix-core rate the device holds under a pure MFMA load, i.e. the
 * ceiling a GEMM reaches at the same clock (MI355X: 1024 dense bf16 FLOP per
 * SIMD per cycle). Per workgroup b, clocks[2b] receives the shader cycles of
 * its loop (s_memtime) and clocks[2b + 1] the 100 MHz real-time ticks
 * (s_memrealtime): their ratio times 100 MHz is the clock under that load.
 *   sink    float [blocks * 512] (device), written with sums that keep the loop
 *   clocks  uint64 [2 * blocks] (device)
 * FLOPs of one launch: blocks * 8 * iters * 64 * 16384. LORA_ERR_SHAPE for
 * iters or blocks < 1, LORA_ERR_NULL_PTR / LORA_ERR_ALIGN for the buffers.
 */
int lora_mfma_probe(int64_t iters, int32_t blocks, float* sink, uint64_t* clocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
