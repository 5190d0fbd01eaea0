"""Plain float64 definitions of the fused LoRA linear path (test infrastructure).

Each function is the definition written out with numpy float64 matrix products
(a library primitive); no blocking, fusion or reordering beyond the formula.
Inputs are the exact bf16/fp32 values of the tensors widened to float64.

Sources (web pages; the section named in each docstring):

* SGLang PR #43501, "[diffusion] Add the dynamic LoRA delta inside the second
  GEMM" -- Motivation and Modifications: the update is (x.A^T).B^T scaled by
  alpha/rank, the adapter strength and the request's LoRA scale; stacked
  q/k/v or gate/up adapters write column views of one output; FP32 adapters
  keep FP32 GEMMs.
* FastVideo ``lora_patch`` API page -- module text (the delta is B @ A) and
  ``DenseLoRAPatch.apply_to`` / ``replacement_for`` (dense payloads).
* Unsloth fast-LoRA chapter, section 3 (``matmul_lora``: 4-bit weight
  dequantized, then the base product plus the LoRA term).
* InvokeAI custom-modules article, NF4 section, and the piper-offload README
  quantized-format table (bitsandbytes NF4 is blockwise): the 4-bit weight is
  a 16-entry codebook value times a per-block absmax.
"""
from __future__ import annotations

import numpy as np

__all__ = ["f64", "combined_scale", "lora_linear", "lora_linear_stacked", "lora_linear_multi", "lora_linear_backward", "merged_weight",
           "nf4_unpack_codes", "nf4_dequant", "lora_linear_nf4", "dense_patch", "rel_rms"]


def f64(a) -> np.ndarray | None:
    """Exact widening of a torch tensor / numpy array of bf16, fp32 or fp64 to float64."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor
        return a.detach().cpu().double().numpy()
    return np.asarray(a, dtype=np.float64)


def combined_scale(alpha: float, rank: int, strength: float, request_scale: float) -> float:
    """s = (alpha / rank) * strength * request_scale, in float64, left to right.

    SGLang PR #43501, Modifications (quality="lossless"): the combined scale is
    alpha/rank times the adapter strength times the request scale. alpha/rank,
    not alpha/sqrt(rank).
    """
    return (float(alpha) / float(rank)) * float(strength) * float(request_scale)


def lora_linear(x, W, b, A, B, alpha, rank, strength, request_scale) -> np.ndarray:
    """y = x.W^T + b + s.(x.A^T).B^T in float64.

    x [T,K], W [N,K], b [N] or None, A [r,K], B [N,r]. The adapter is
    inactive (base output only) when A or B is None or when s is +-0: a zero
    strength is filtered out as inactive (piper-offload README, strengths), and
    a disabled adapter leaves the plain X.W (Unsloth chapter, section 6).
    """
    x, W, b, A, B = f64(x), f64(W), f64(b), f64(A), f64(B)
    y = x @ W.T
    if b is not None:
        y = y + b[None, :]
    s = combined_scale(alpha, rank, strength, request_scale)
    if A is not None and B is not None and s != 0.0:
        y = y + s * ((x @ A.T) @ B.T)
    return y


def lora_linear_stacked(x, W, b, groups, strength, request_scale) -> np.ndarray:
    """Stacked groups: y[:, o_g:o_g+N_g] += s_g.(x.A_g^T).B_g^T over one base product.

    SGLang PR #43501, Modifications: stacked q/k/v (or gate/up) adapters take
    one update per group on column views of the output. Each group has its own
    alpha_g / r_g; strength and request scale are shared. Columns outside every
    group get the base output only.
    """
    x, W, b = f64(x), f64(W), f64(b)
    y = x @ W.T
    if b is not None:
        y = y + b[None, :]
    for g in groups:
        s = combined_scale(g["alpha"], g["rank"], strength, request_scale)
        if g["A"] is None or g["B"] is None or s == 0.0:
            continue
        o, n = int(g["col_offset"]), int(g["n_cols"])
        y[:, o:o + n] += s * ((x @ f64(g["A"]).T) @ f64(g["B"]).T)
    return y


def lora_linear_multi(x, W, b, adapters, request_scale) -> np.ndarray:
    """Several adapters on one layer, each on its own columns:

        y = x.W^T + b + sum_i [ s_i.(x.A_i^T).B_i^T + u_i.c_i ]

    with s_i = (alpha_i / r_i) . strength_i . request_scale and u_i = strength_i . request_scale.

    piper-offload README, routed mode: the output residual is the strength
    times (B.A.x plus the legacy bias), and several LoRAs on one target are
    summed independently; its LoRA resource section: an older adapter may carry
    a lora_B.bias vector c_i, which merge mode adds to the layer's bias with the
    same adapter strength. InvokeAI article, section 3: a layer keeps a list of
    (patch, weight) pairs whose contributions add up. Reading: alpha_i / r_i
    belongs to the factor pair (SGLang PR #43501, Motivation), so the legacy
    vector takes the adapter strength and the request scale only. ``adapters``
    are dicts with A, B, c (or None), rank, alpha, strength, col_offset,
    n_cols; an adapter with A or B None or s_i == +-0 is inactive as a whole
    (its legacy vector included).
    """
    x, W, b = f64(x), f64(W), f64(b)
    y = x @ W.T
    if b is not None:
        y = y + b[None, :]
    for a in adapters:
        s = combined_scale(a["alpha"], a["rank"], a["strength"], request_scale)
        if a["A"] is None or a["B"] is None or s == 0.0:
            continue
        o, n = int(a["col_offset"]), int(a["n_cols"])
        y[:, o:o + n] += s * ((x @ f64(a["A"]).T) @ f64(a["B"]).T)
        if a.get("c") is not None:
            u = float(a["strength"]) * float(request_scale)
            y[:, o:o + n] += u * f64(a["c"])[None, :]
    return y


def lora_linear_backward(x, W, A, B, dy, alpha, rank, strength, request_scale):
    """Gradients of the LoRA linear y = x.W^T + b + s.(x.A^T).B^T for an output gradient dy
    (the base W frozen), in float64:

        u  = dy.B                       [T, r]
        dx = dy.W + s.u.A               [T, K]
        dA = s.u^T.x                    [r, K]
        dB = s.dy^T.(x.A^T)             [N, r]
        db = sum over tokens of dy      [N]

    Unsloth fast-LoRA chapter, sections 2 and 4: the backward of a LoRA layer has a closed form
    (dC/dA and dC/dB as products of X, the incoming gradient and the other factor), computed
    directly instead of through autograd, with the frozen weight only needed for dX. Written in
    this library's orientation (delta B @ A, FastVideo lora_patch page). Returns (dx, dA, dB, db).
    """
    x, W, A, B, dy = f64(x), f64(W), f64(A), f64(B), f64(dy)
    s = combined_scale(alpha, rank, strength, request_scale)
    u = dy @ B
    dx = dy @ W + s * (u @ A)
    dA = s * (u.T @ x)
    dB = s * (dy.T @ (x @ A.T))
    db = dy.sum(axis=0)
    return dx, dA, dB, db


def merged_weight(W, A, B, s) -> np.ndarray:
    """W + s.B.A: the merged weight whose linear equals the factored form.

    FastVideo lora_patch page, module text: a LoRA states the weight delta as
    B @ A.
    """
    return f64(W) + float(s) * (f64(B) @ f64(A))


def nf4_unpack_codes(codes, K: int) -> np.ndarray:
    """Packed uint8 [N, K/2] -> integer codes [N, K].

    Byte j of a row holds element 2j in its low nibble (bits 0-3) and element
    2j+1 in its high nibble (bits 4-7). The pages do not print a nibble order;
    this is the stated layout of the library's boundary.
    """
    c = np.asarray(codes.numpy() if hasattr(codes, "numpy") else codes, dtype=np.uint8)
    out = np.empty((c.shape[0], K), dtype=np.int64)
    out[:, 0::2] = c & 0x0F
    out[:, 1::2] = c >> 4
    return out


def nf4_dequant(codes, absmax, codebook, K: int, blocksize: int = 64) -> np.ndarray:
    """W[n,k] = codebook[code(n,k)] * absmax[(n*K + k) // blocksize], in float64 (exact).

    The weight is a 16-entry codebook value times an fp32 absmax per block of
    64 consecutive elements of the row-major [N, K] weight (blockwise 4-bit
    format: piper-offload README quantized-format table; InvokeAI article, NF4
    section). The product of two fp32 values is exact in float64.
    """
    c = nf4_unpack_codes(codes, K)
    N = c.shape[0]
    cb = f64(codebook)
    am = f64(absmax)
    flat_index = np.arange(N, dtype=np.int64)[:, None] * K + np.arange(K, dtype=np.int64)[None, :]
    return cb[c] * am[flat_index // blocksize]


def lora_linear_nf4(x, codes, absmax, codebook, blocksize, b, A, B, alpha, rank, strength,
                    request_scale) -> np.ndarray:
    """The LoRA linear of ``lora_linear`` over the dequantized 4-bit weight.

    Unsloth chapter, section 3 (``matmul_lora``): dequantize the 4-bit weight,
    take the base product, add the scaled low-rank term.
    """
    K = f64(x).shape[1]
    W = nf4_dequant(codes, absmax, codebook, K, blocksize)
    return lora_linear(x, W, b, A, B, alpha, rank, strength, request_scale)


def dense_patch(dst, src, strength, mode: str) -> np.ndarray:
    """Dense payloads in float64.

    FastVideo lora_patch page: ``apply_to`` (.diff/.diff_b) adds the delta times
    the strength to the parameter; ``replacement_for`` (.set_weight) returns the
    supplied value times the strength (the absent parameter counts as zero).
    """
    if mode == "add":
        return f64(dst) + float(strength) * f64(src)
    if mode == "replace":
        return float(strength) * f64(src)
    raise ValueError(mode)


def rel_rms(y, ref) -> float:
    """Relative RMS error ||y - ref||_2 / ||ref||_2 over all elements (float64)."""
    y, ref = f64(y), f64(ref)
    return float(np.linalg.norm((y - ref).ravel()) / np.linalg.norm(ref.ravel()))
