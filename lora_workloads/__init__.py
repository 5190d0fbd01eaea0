"""Seeded synthetic inputs for the fused LoRA linear path.

This module only draws numbers. It holds none of the method's arithmetic: no
GEMM, no scale, no dequantization, no rounding rule of the method. Both the
oracle (under ``oracle/``) and the HIP path (``rank_gemm_lora_amd``) are fed
from here, and nothing else is shared between them.

Recipe (stated once, used everywhere):

* Generator: ``numpy.random.default_rng(seed)`` (PCG64). Every tensor is drawn
  as float64 standard normals, in the order the spec lists the tensors, and
  scaled by ``sqrt(v)`` where ``N(0, v)`` names the *variance* ``v``.
* Casting: float64 -> float32 (round to nearest even) -> bfloat16 (round to
  nearest even), both done by torch's CPU casts. The oracle widens the same
  bits back to float64, so both sides see identical values.
* Codes of the 4-bit weight are uniform bytes (two uniform nibbles each).
* The real models of the pages (Wan2.1 1.3B, Z-Image-Turbo, MiniMax-H3 with
  their adapters) are not available; these synthetic layers of the same
  shapes and ranks stand in for them.
"""
from __future__ import annotations

import math
import statistics
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = [
    "LinearSpec", "StackedSpec", "Nf4Spec", "PatchSpec", "MultiSpec", "MULTI_FFN_UP", "multi_inputs",
    "MergeSpec", "MERGE_WEIGHT", "MERGE_WEIGHT_SMALL", "merge_inputs",
    "TINY_FP32", "ATTN_PROJ", "FFN_UP", "FFN_DOWN", "QKV_STACKED", "NF4_LAYER",
    "PATCH_WEIGHT", "PATCH_NORM", "ZIMAGE_ATTN", "ZIMAGE_FFN_UP", "ZIMAGE_FFN_DOWN", "H3_FFN_UP",
    "H3_FFN_DOWN", "FEW_FFN_UP", "FEW_FFN_DOWN", "NF4_VECTOR",
    "linear_inputs", "ffn_pair_inputs", "stacked_inputs", "nf4_inputs", "patch_inputs",
    "nf4_style_codebook", "dyadic_linear_inputs", "to_dtype",
]

_CHUNK = 1 << 24  # draw at most 16 M float64 values at a time


def to_dtype(a64: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 numpy -> torch CPU tensor of ``dtype`` ('f32' or 'bf16'), via float32."""
    t = torch.from_numpy(np.ascontiguousarray(a64)).to(torch.float32)
    if dtype == "f32":
        return t
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(f"unknown dtype {dtype}")


def _normal(rng: np.random.Generator, shape, var: float, dtype: str,
            spread: str = "variance") -> torch.Tensor:
    """Draw N(0, var) in float64 (chunked, same stream as one draw) and cast."""
    n = int(np.prod(shape)) if len(shape) else 1
    scale = math.sqrt(var) if spread == "variance" else var
    out = torch.empty(n, dtype=torch.float32 if dtype == "f32" else torch.bfloat16)
    pos = 0
    while pos < n:
        m = min(_CHUNK, n - pos)
        out[pos:pos + m] = to_dtype(rng.standard_normal(m) * scale, dtype)
        pos += m
    return out.reshape(shape)


@dataclass(frozen=True)
class LinearSpec:
    """One LoRA linear layer: y[T,N] from x[T,K], W[N,K], A[r,K], B[N,r]."""
    name: str
    T: int
    K: int
    N: int
    rank: int
    alpha: float
    strength: float
    request_scale: float
    bias: bool
    seed: int
    act: str = "bf16"       # dtype of x, W, bias and y
    adapter: str = "bf16"   # dtype of A and B
    x_var: float = 1.0
    b_var: float = 0.02     # variance of B and of the bias
    B_zero: bool = False


@dataclass(frozen=True)
class StackedSpec:
    """q/k/v (or gate/up) groups: one W[sum N_g, K], one adapter per column range."""
    name: str
    T: int
    K: int
    n_cols: tuple
    ranks: tuple
    alphas: tuple
    strength: float
    request_scale: float
    bias: bool
    seed: int
    act: str = "bf16"
    adapter: str = "bf16"


@dataclass(frozen=True)
class Nf4Spec:
    """4-bit codebook base weight with fp32 absmax per 64-element block."""
    name: str
    T: int
    K: int
    N: int
    rank: int
    alpha: float
    strength: float
    request_scale: float
    bias: bool
    seed: int
    blocksize: int = 64
    absmax_var: float = 0.05


@dataclass(frozen=True)
class MultiSpec:
    """Several adapters on one layer: ``adapters`` holds (rank, alpha, strength, col_offset,
    n_cols, legacy lora_B bias present) per adapter; ranges may overlap."""
    name: str
    T: int
    K: int
    N: int
    adapters: tuple
    request_scale: float
    bias: bool
    seed: int
    adapter: str = "bf16"


@dataclass(frozen=True)
class MergeSpec:
    """An adapter merged into a dense weight: W [N, K], A [r, K], B [N, r]."""
    name: str
    N: int
    K: int
    rank: int
    alpha: float
    strength: float
    seed: int
    b_var: float = 0.02


@dataclass(frozen=True)
class PatchSpec:
    """Dense payload applied to a parameter of ``shape``."""
    name: str
    shape: tuple
    strength: float
    seed: int
    base_mean: float
    base_var: float
    diff_var: float
    dtype: str = "bf16"


# The workloads: shapes, ranks and scales of the synthetic video-DiT layers.
TINY_FP32 = LinearSpec("tiny_fp32", T=64, K=128, N=96, rank=8, alpha=16.0, strength=1.0,
                       request_scale=1.0, bias=True, seed=0, act="f32", adapter="f32")
ATTN_PROJ = LinearSpec("attn_proj", T=32760, K=1536, N=1536, rank=32, alpha=32.0, strength=0.8,
                       request_scale=1.0, bias=True, seed=2)
FFN_UP = LinearSpec("ffn_up", T=32760, K=1536, N=8960, rank=64, alpha=64.0, strength=1.0,
                    request_scale=0.7, bias=False, seed=3)
FFN_DOWN = LinearSpec("ffn_down", T=32760, K=8960, N=1536, rank=64, alpha=64.0, strength=1.0,
                      request_scale=0.7, bias=True, seed=3)
QKV_STACKED = StackedSpec("qkv_stacked", T=16384, K=3072, n_cols=(3072, 3072, 3072),
                          ranks=(128, 128, 128), alphas=(128.0, 128.0, 128.0), strength=1.0,
                          request_scale=1.0, bias=False, seed=4)
NF4_LAYER = Nf4Spec("nf4_layer", T=8192, K=4096, N=14336, rank=16, alpha=32.0, strength=1.0,
                    request_scale=1.0, bias=False, seed=5)
# The other token regimes of the pages' per-forward cost table (the table gives
# ranks and token counts, not layer dims: the 1536 / 8960 layers above are
# reused). Z-Image-Turbo at 1024^2: rank 32, 4352 tokens; MiniMax-H3 with
# Ulysses 2: rank 64, 18871 tokens per rank; and few tokens (the single-vector
# 4-bit case, a 64-token FFN pair).
ZIMAGE_ATTN = LinearSpec("zimage_attn", T=4352, K=1536, N=1536, rank=32, alpha=32.0, strength=0.8,
                         request_scale=1.0, bias=True, seed=8)
ZIMAGE_FFN_UP = LinearSpec("zimage_ffn_up", T=4352, K=1536, N=8960, rank=32, alpha=32.0, strength=1.0,
                           request_scale=0.7, bias=False, seed=9)
ZIMAGE_FFN_DOWN = LinearSpec("zimage_ffn_down", T=4352, K=8960, N=1536, rank=32, alpha=32.0, strength=1.0,
                             request_scale=0.7, bias=True, seed=9)
H3_FFN_UP = LinearSpec("h3_ffn_up", T=18871, K=1536, N=8960, rank=64, alpha=64.0, strength=1.0,
                       request_scale=0.7, bias=False, seed=10)
H3_FFN_DOWN = LinearSpec("h3_ffn_down", T=18871, K=8960, N=1536, rank=64, alpha=64.0, strength=1.0,
                         request_scale=0.7, bias=True, seed=10)
FEW_FFN_UP = LinearSpec("few_ffn_up", T=64, K=1536, N=8960, rank=64, alpha=64.0, strength=1.0,
                        request_scale=0.7, bias=False, seed=11)
FEW_FFN_DOWN = LinearSpec("few_ffn_down", T=64, K=8960, N=1536, rank=64, alpha=64.0, strength=1.0,
                          request_scale=0.7, bias=True, seed=11)
NF4_VECTOR = Nf4Spec("nf4_vector", T=1, K=4096, N=14336, rank=16, alpha=32.0, strength=1.0,
                     request_scale=1.0, bias=False, seed=12)

# Two adapters on the FFN up layer (piper-offload routed mode: several LoRAs on one target), the
# second an older adapter with a lora_B bias.
MULTI_FFN_UP = MultiSpec("multi_ffn_up", T=32760, K=1536, N=8960,
                         adapters=((64, 64.0, 1.0, 0, 8960, False), (32, 32.0, 0.5, 0, 8960, True)),
                         request_scale=0.7, bias=False, seed=13)

# The rank-16 adapter of the 4-bit layer's shape merged into a bf16 weight of that shape (merge mode);
# the second reads "N(0, 0.02)" of B as a standard deviation: the small update a bf16 merge loses.
MERGE_WEIGHT = MergeSpec("merge_weight", N=14336, K=4096, rank=16, alpha=32.0, strength=0.8, seed=14)
MERGE_WEIGHT_SMALL = MergeSpec("merge_weight_small_update", N=14336, K=4096, rank=16, alpha=32.0, strength=0.8,
                               seed=14, b_var=0.02 ** 2)

PATCH_WEIGHT = PatchSpec("patch_weight", shape=(14336, 4096), strength=0.8, seed=6,
                         base_mean=0.0, base_var=1.0 / 4096, diff_var=(1e-3) ** 2 / 4096)
PATCH_NORM = PatchSpec("patch_norm", shape=(3072,), strength=0.8, seed=7,
                       base_mean=1.0, base_var=0.1 ** 2, diff_var=1e-4)


def _linear_draw(rng, s: LinearSpec, spread: str) -> dict:
    x = _normal(rng, (s.T, s.K), s.x_var, s.act, spread)
    W = _normal(rng, (s.N, s.K), 1.0 / s.K, s.act, spread)
    A = _normal(rng, (s.rank, s.K), 1.0 / s.K, s.adapter, spread)
    B = _normal(rng, (s.N, s.rank), s.b_var, s.adapter, spread)
    b = _normal(rng, (s.N,), s.b_var, s.act, spread) if s.bias else None
    if s.B_zero:
        B = torch.zeros_like(B)
    return dict(x=x, W=W, b=b, A=A, B=B, rank=s.rank, alpha=s.alpha, strength=s.strength,
                request_scale=s.request_scale)


def linear_inputs(s: LinearSpec, spread: str = "variance", rng=None) -> dict:
    """x, W, b (or None), A, B as torch CPU tensors, plus the scalars of ``s``."""
    rng = np.random.default_rng(s.seed) if rng is None else rng
    return _linear_draw(rng, s, spread)


def ffn_pair_inputs(up: LinearSpec = FFN_UP, down: LinearSpec = FFN_DOWN,
                    spread: str = "variance"):
    """Up then down from one generator: the down layer continues up's stream.

    No activation sits between the two layers in the workload, so the down
    layer gets its own x ~ N(0, 1) of shape [T, 8960].
    """
    rng = np.random.default_rng(up.seed)
    u = _linear_draw(rng, up, spread)
    d = _linear_draw(rng, down, spread)
    return u, d


def stacked_inputs(s: StackedSpec, spread: str = "variance") -> dict:
    rng = np.random.default_rng(s.seed)
    n_total = sum(s.n_cols)
    x = _normal(rng, (s.T, s.K), 1.0, s.act, spread)
    W = _normal(rng, (n_total, s.K), 1.0 / s.K, s.act, spread)
    groups = []
    off = 0
    for n, r, a in zip(s.n_cols, s.ranks, s.alphas):
        A = _normal(rng, (r, s.K), 1.0 / s.K, s.adapter, spread)
        B = _normal(rng, (n, r), 0.02, s.adapter, spread)
        groups.append(dict(A=A, B=B, rank=r, alpha=a, col_offset=off, n_cols=n))
        off += n
    b = _normal(rng, (n_total,), 0.02, s.act, spread) if s.bias else None
    return dict(x=x, W=W, b=b, groups=groups, strength=s.strength, request_scale=s.request_scale)


def multi_inputs(s: MultiSpec, spread: str = "variance") -> dict:
    """x, W, b and one dict per adapter (A, B, c or None, rank, alpha, strength, col_offset, n_cols)."""
    rng = np.random.default_rng(s.seed)
    x = _normal(rng, (s.T, s.K), 1.0, "bf16", spread)
    W = _normal(rng, (s.N, s.K), 1.0 / s.K, "bf16", spread)
    b = _normal(rng, (s.N,), 0.02, "bf16", spread) if s.bias else None
    ads = []
    for r, a, st, o, n, has_c in s.adapters:
        A = _normal(rng, (r, s.K), 1.0 / s.K, s.adapter, spread)
        B = _normal(rng, (n, r), 0.02, s.adapter, spread)
        c = _normal(rng, (n,), 0.02, s.adapter, spread) if has_c else None
        ads.append(dict(A=A, B=B, c=c, rank=r, alpha=a, strength=st, col_offset=o, n_cols=n))
    return dict(x=x, W=W, b=b, adapters=ads, request_scale=s.request_scale)


def merge_inputs(s: MergeSpec) -> dict:
    """W, A, B (bf16) of a merge workload."""
    rng = np.random.default_rng(s.seed)
    W = _normal(rng, (s.N, s.K), 1.0 / s.K, "bf16")
    A = _normal(rng, (s.rank, s.K), 1.0 / s.K, "bf16")
    B = _normal(rng, (s.N, s.rank), s.b_var, "bf16")
    return dict(W=W, A=A, B=B, rank=s.rank, alpha=s.alpha, strength=s.strength)


def nf4_style_codebook() -> torch.Tensor:
    """A 16-entry "NF4-style" table: normal quantiles, ascending, max |v| = 1, exact 0.

    Stated construction (the pages print no table): 8 positive entries at the
    standard-normal quantiles of p = 0.5 + 0.47 * i / 8 (i = 1..8), 7 negative
    ones at -quantile(0.5 + 0.47 * i / 7) (i = 1..7), and 0. Each side is
    divided by its largest magnitude, then rounded to float32.
    """
    nd = statistics.NormalDist()
    pos = [nd.inv_cdf(0.5 + 0.47 * i / 8) for i in range(1, 9)]
    neg = [nd.inv_cdf(0.5 + 0.47 * i / 7) for i in range(1, 8)]
    vals = sorted([-v / neg[-1] for v in neg] + [0.0] + [v / pos[-1] for v in pos])
    return torch.tensor(vals, dtype=torch.float32)


def nf4_inputs(s: Nf4Spec, spread: str = "variance") -> dict:
    """x bf16, packed codes uint8 [N, K/2], absmax fp32 [N*K/64], codebook fp32 [16], A, B."""
    rng = np.random.default_rng(s.seed)
    x = _normal(rng, (s.T, s.K), 1.0, "bf16", spread)
    codes = torch.from_numpy(rng.integers(0, 256, size=(s.N, s.K // 2), dtype=np.uint8))
    nblk = s.N * s.K // s.blocksize
    scale = math.sqrt(s.absmax_var) if spread == "variance" else s.absmax_var
    absmax = torch.from_numpy(np.abs(rng.standard_normal(nblk)) * scale).to(torch.float32)
    A = _normal(rng, (s.rank, s.K), 1.0 / s.K, "bf16", spread)
    B = _normal(rng, (s.N, s.rank), 0.02, "bf16", spread)
    b = _normal(rng, (s.N,), 0.02, "bf16", spread) if s.bias else None
    return dict(x=x, codes=codes, absmax=absmax, codebook=nf4_style_codebook(),
                blocksize=s.blocksize, A=A, B=B, b=b, rank=s.rank, alpha=s.alpha,
                strength=s.strength, request_scale=s.request_scale)


def patch_inputs(s: PatchSpec, spread: str = "variance") -> dict:
    rng = np.random.default_rng(s.seed)
    n = int(np.prod(s.shape))
    base = torch.empty(n, dtype=torch.bfloat16 if s.dtype == "bf16" else torch.float32)
    pos = 0
    sd = math.sqrt(s.base_var) if spread == "variance" else s.base_var
    while pos < n:
        m = min(_CHUNK, n - pos)
        base[pos:pos + m] = to_dtype(s.base_mean + rng.standard_normal(m) * sd, s.dtype)
        pos += m
    diff = _normal(rng, (n,), s.diff_var, s.dtype, spread)
    return dict(dst=base.reshape(s.shape), diff=diff.reshape(s.shape), strength=s.strength)


def small_linear_inputs(T, K, N, rank, seed, act="bf16", adapter="bf16", bias=True,
                        alpha=None, strength=1.0, request_scale=1.0, b_var=0.02) -> dict:
    """Generic seeded case for parity tests at sizes the oracle finishes quickly."""
    s = LinearSpec("small", T=T, K=K, N=N, rank=rank,
                   alpha=float(rank if alpha is None else alpha), strength=strength,
                   request_scale=request_scale, bias=bias, seed=seed, act=act, adapter=adapter,
                   b_var=b_var)
    return linear_inputs(s)


def dyadic_linear_inputs(T, K, N, rank, seed, act="bf16", adapter="bf16", bias=True,
                         density=0.15) -> dict:
    """Sparse small-integer inputs scaled by powers of two.

    Every product and partial sum of such inputs is a small multiple of a power
    of two, so (when the test confirms it) all intermediates are exactly
    representable and every rounding step is the identity.
    """
    rng = np.random.default_rng(seed)

    def draw(shape, scale):
        v = rng.integers(-3, 4, size=shape).astype(np.float64)
        v *= rng.random(shape) < density
        return v * scale

    x = draw((T, K), 1.0)
    W = draw((N, K), 0.25)
    A = draw((rank, K), 0.5)
    B = draw((N, rank), 0.125)
    b = draw((N,), 0.5) if bias else None
    return dict(x=to_dtype(x, act), W=to_dtype(W, act), A=to_dtype(A, adapter),
                B=to_dtype(B, adapter), b=None if b is None else to_dtype(b, act))
