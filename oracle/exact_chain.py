"""The separate-pass chain that defines the exact tier, with explicit roundings.

SGLang PR #43501 describes the dynamic-LoRA path before the change (Motivation):
the [tokens, out] update is materialized, scaled by alpha/rank, by the adapter
strength and by the request's LoRA scale in one pass each, then added to the
base output. Its quality="exact" tier (Modifications) keeps that chain and only
skips multiplications by a unit scale, which are exact, so the output is bit
for bit the chain's. The pages do not print the GEMM's internals, so this file
*is* the definition the exact tier is held to (reading stated at the boundary):

E1  G(P, Q)[i, j] = RN_f32( sum_k P[i, k] * Q[j, k] ), the sum accumulated in
    float64 with k ascending from +0.0. Every product of bf16/fp32 inputs is
    exact in float64, so the only roundings are the fp64 adds and the final one.
E2  base = RN_dt( RN_f32( G(x, W) + b ) )   (without a bias: RN_dt(G(x, W)))
E3  t = RN_adt( G(x, A) ),  d = RN_adt( G(t, B) )
E4  for f in (alpha / rank, strength, request_scale), in that order, when
    RN_f32(f) != 1.0:  d = RN_adt( RN_f32( d * RN_f32(f) ) )
E5  y = RN_dt( RN_f32( base + d ) )
E6  4-bit weight: W = RN_bf16( RN_f32( codebook[c] * absmax ) ), then E2-E5
E7  dense payload (FastVideo DenseLoRAPatch.apply_to / replacement_for, the sum
    taken in float32 and cast back by the caller):
      add:     RN_dt( RN_f32( dst + RN_f32( diff * RN_f32(strength) ) ) )
      replace: RN_dt( RN_f32( value * RN_f32(strength) ) )

RN_* is IEEE round-to-nearest-even; dt is the activation dtype, adt the
adapter dtype. A combined scale of +-0 leaves the adapter inactive (base only).
Float64 holds the exact result of one fp32 add or multiply of fp32 values and
53 >= 2*24 + 2, so rounding that result to fp32 equals the fp32 operation.
"""
from __future__ import annotations

import numpy as np

from .lora_oracle import f64, nf4_unpack_codes

__all__ = ["rn_f32", "rn_bf16", "rn", "gemm_ordered", "chain_linear", "chain_stacked", "chain_multi",
           "chain_merge", "chain_nf4_weight", "chain_nf4", "chain_dense_patch"]


def rn_f32(a) -> np.ndarray:
    """Round float64 values to the nearest float32 (ties to even), returned as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def rn_bf16(a) -> np.ndarray:
    """Round float32-representable values to bfloat16 (ties to even), returned as float64.

    Integer rounding on the fp32 bit pattern: add 0x7FFF plus the lowest kept
    bit, drop 16 bits. Overflow carries into the exponent and gives +-inf as
    IEEE requires; NaN stays NaN (quiet).
    """
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(a, np.float64), equal_nan=True):
        raise ValueError("rn_bf16 expects float32-representable inputs")
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    nan = np.isnan(f)
    r = np.where(nan, ((u >> 16) | 0x40) & 0xFFFF, r)
    return (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rn(a, dtype: str) -> np.ndarray:
    """RN_dtype of float32-representable values: identity for 'f32', rn_bf16 for 'bf16'."""
    if dtype == "f32":
        return rn_f32(a)
    if dtype == "bf16":
        return rn_bf16(a)
    raise ValueError(dtype)


def gemm_ordered(P, Q) -> np.ndarray:
    """E1: RN_f32 of sum_k P[i,k]*Q[j,k], accumulated in float64 from +0.0, k ascending."""
    P, Q = f64(P), f64(Q)
    acc = np.zeros((P.shape[0], Q.shape[0]), dtype=np.float64)
    for k in range(P.shape[1]):
        acc += P[:, k, None] * Q[None, :, k]
    return rn_f32(acc)


def _scale_passes(d, factors, adt):
    """E4: one multiply pass per factor whose fp32 value is not exactly 1."""
    for f in factors:
        f32 = float(rn_f32(f))
        if f32 != 1.0:
            d = rn(rn_f32(d * f32), adt)
    return d


def _base(x, W, b, act):
    g = gemm_ordered(x, W)
    if b is None:
        return rn(g, act)
    return rn(rn_f32(g + f64(b)[None, :]), act)


def _delta(x, A, B, factors, adt):
    t = rn(gemm_ordered(x, A), adt)
    d = rn(gemm_ordered(t, B), adt)
    return _scale_passes(d, factors, adt)


def chain_linear(x, W, b, A, B, alpha, rank, strength, request_scale,
                 act: str = "bf16", adapter: str = "bf16") -> np.ndarray:
    """E1-E5 for one adapter; returns the exact-tier output as float64 values."""
    base = _base(x, W, b, act)
    factors = (float(alpha) / float(rank), float(strength), float(request_scale))
    if A is None or B is None or (factors[0] * factors[1] * factors[2]) == 0.0:
        return base
    d = _delta(x, A, B, factors, adapter)
    return rn(rn_f32(base + d), act)


def chain_stacked(x, W, b, groups, strength, request_scale, act: str = "bf16",
                  adapter: str = "bf16") -> np.ndarray:
    """E1-E5 per group on its column range of one base output."""
    y = _base(x, W, b, act).copy()
    for g in groups:
        factors = (float(g["alpha"]) / float(g["rank"]), float(strength), float(request_scale))
        if g["A"] is None or g["B"] is None or (factors[0] * factors[1] * factors[2]) == 0.0:
            continue
        o, n = int(g["col_offset"]), int(g["n_cols"])
        d = _delta(x, g["A"], g["B"], factors, adapter)
        y[:, o:o + n] = rn(rn_f32(y[:, o:o + n] + d), act)
    return y


def chain_multi(x, W, b, adapters, request_scale, act: str = "bf16", adapter: str = "bf16") -> np.ndarray:
    """E1-E5 per adapter, in the order given, on its column range of one base output.

    Each adapter has its own strength. Its legacy lora_B bias c (or None) is a
    dense payload of the adapter on its output columns, applied after the
    adapter's own delta: the scale passes of E4 over (strength, request_scale)
    only -- alpha / rank belongs to the factor pair -- then the add of E5:
    e = passes(c), y = RN_dt(RN_f32(y + e)). Adapters on the same columns add
    one after another.
    """
    y = _base(x, W, b, act).copy()
    for a in adapters:
        factors = (float(a["alpha"]) / float(a["rank"]), float(a["strength"]), float(request_scale))
        if a["A"] is None or a["B"] is None or (factors[0] * factors[1] * factors[2]) == 0.0:
            continue
        o, n = int(a["col_offset"]), int(a["n_cols"])
        d = _delta(x, a["A"], a["B"], factors, adapter)
        y[:, o:o + n] = rn(rn_f32(y[:, o:o + n] + d), act)
        if a.get("c") is not None:
            e = _scale_passes(f64(a["c"]), factors[1:], adapter)
            y[:, o:o + n] = rn(rn_f32(y[:, o:o + n] + e[None, :]), act)
    return y


def chain_merge(W, A, B, alpha, rank, strength, wdt: str = "bf16") -> np.ndarray:
    """Exact tier of the merge W <- W + s.B.A (piper-offload README, LoRA merge: an in-place
    addmm_ into a plain dense base), as the chain of a dense payload whose delta is the rank
    product: G = E1(B, A^T) (fp32, q ascending), then E7's add with s = RN_f32((alpha / rank) .
    strength): d = RN_f32(G . s) (skipped when s == 1), W' = RN_wdt(RN_f32(W + d))."""
    G = gemm_ordered(B, f64(A).T)
    s32 = float(rn_f32((float(alpha) / float(rank)) * float(strength)))
    d = G if s32 == 1.0 else rn_f32(G * s32)
    return rn(rn_f32(f64(W) + d), wdt)


def chain_nf4_weight(codes, absmax, codebook, K: int, blocksize: int = 64) -> np.ndarray:
    """E6: the bf16 weight the 4-bit path multiplies, RN_bf16(RN_f32(cb[c] * absmax))."""
    c = nf4_unpack_codes(codes, K)
    N = c.shape[0]
    cb = f64(codebook)
    am = f64(absmax)
    idx = (np.arange(N, dtype=np.int64)[:, None] * K + np.arange(K, dtype=np.int64)[None, :])
    return rn_bf16(rn_f32(cb[c] * am[idx // blocksize]))


def chain_nf4(x, codes, absmax, codebook, blocksize, b, A, B, alpha, rank, strength,
              request_scale, rows=None) -> np.ndarray:
    """E6 then E2-E5 (activations and adapter bf16). ``rows`` selects output rows."""
    K = f64(x).shape[1]
    W = chain_nf4_weight(codes, absmax, codebook, K, blocksize)
    xs = f64(x) if rows is None else f64(x)[rows]
    return chain_linear(xs, W, b, A, B, alpha, rank, strength, request_scale, "bf16", "bf16")


def chain_dense_patch(dst, src, strength, mode: str, dtype: str = "bf16") -> np.ndarray:
    """E7: the dense payload with the float32 roundings of the page's tensor ops."""
    s32 = float(rn_f32(strength))
    if mode == "add":
        return rn(rn_f32(f64(dst) + rn_f32(f64(src) * s32)), dtype)
    if mode == "replace":
        return rn(rn_f32(f64(src) * s32), dtype)
    raise ValueError(mode)
