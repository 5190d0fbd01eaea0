"""Python binding of liblora_mi355x.so, the fused LoRA linear for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C-ABI declared in ``include/lora_mi355x.h``. PyTorch is used
for device memory and streams (tensor ``data_ptr()`` and the current HIP
stream), nothing else. There is no CPU fallback: importing this package
without the built library raises.

Low-level functions carry the C names and take plain integers for pointers:
``lora_linear_fwd``, ``lora_linear_stacked_fwd``, ``lora_linear_nf4_fwd`` (and
``lora_linear_nf4_fwd_ex``, which names where the 4-bit weight is dequantized),
``dense_patch_apply``, ``lora_linear_workspace_size``, ``lora_status_string``,
``lora_device_check``. Tensor-level helpers (``lora_linear``,
``lora_linear_stacked``, ``lora_linear_nf4``, ``dense_patch``) check that the
tensors sit on one device, allocate the output and workspace with torch when
not given, and call the C functions on the current stream.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime this library binds to (one runtime per process)

__all__ = [
    "LIB_PATH", "LoraError", "LORA_F32", "LORA_BF16", "LORA_LOSSLESS", "LORA_EXACT",
    "LORA_PATCH_ADD", "LORA_PATCH_REPLACE", "lora_linear_fwd", "lora_linear_stacked_fwd",
    "lora_linear_nf4_fwd", "lora_linear_nf4_fwd_ex", "LORA_NF4_AUTO", "LORA_NF4_PANEL", "LORA_NF4_IN_GEMM",
    "dense_patch_apply", "lora_linear_fwd_phase", "lora_linear_workspace_size",
    "lora_linear_nf4_workspace_size", "lora_linear_multi_fwd", "lora_linear_multi_workspace_size",
    "lora_linear_multi", "LoraAdapter", "lora_merge_apply", "lora_merge", "lora_linear_bwd",
    "lora_linear_bwd_workspace_size", "lora_linear_backward",
    "lora_status_string",
    "lora_device_check", "lora_mfma_probe", "lora_linear_fwd_noalloc", "LORA_NOALLOC_SCRATCH_BYTES", "lora_linear", "lora_linear_stacked", "lora_linear_nf4", "dense_patch",
    "LoraGroup", "hip_runtimes_mapped",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblora_mi355x.so")

LORA_F32, LORA_BF16 = 0, 1
LORA_LOSSLESS, LORA_EXACT = 0, 1
LORA_PATCH_ADD, LORA_PATCH_REPLACE = 0, 1
LORA_NF4_AUTO, LORA_NF4_PANEL, LORA_NF4_IN_GEMM = 0, 1, 2
_DEQUANT = {"auto": LORA_NF4_AUTO, "panel": LORA_NF4_PANEL, "in_gemm": LORA_NF4_IN_GEMM}
_QUALITY = {"lossless": LORA_LOSSLESS, "exact": LORA_EXACT}
_MODE = {"add": LORA_PATCH_ADD, "replace": LORA_PATCH_REPLACE}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python rank_gemm_lora_amd/_build.py` "
                      "(or __graft_entry__.build()); there is no fallback path")
_lib = ctypes.CDLL(LIB_PATH)

_p, _i64, _i32, _f64, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_size_t


class LoraGroup(ctypes.Structure):
    """C ``lora_group``: one adapter of a stacked layer."""
    _fields_ = [("A", _p), ("B", _p), ("rank", _i32), ("reserved", _i32), ("alpha", _f64),
                ("col_offset", _i64), ("n_cols", _i64)]


class LoraAdapter(ctypes.Structure):
    """C ``lora_adapter``: one of several adapters on one layer."""
    _fields_ = [("A", _p), ("B", _p), ("B_bias", _p), ("rank", _i32), ("reserved", _i32), ("alpha", _f64),
                ("strength", _f64), ("col_offset", _i64), ("n_cols", _i64)]


_lib.lora_linear_fwd.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _p, _p, _i32, _i32, _f64, _f64, _f64,
                                 _p, _i64, _i32, _i32, _p, _sz, _p]
_lib.lora_linear_fwd.restype = ctypes.c_int
_lib.lora_linear_fwd_noalloc.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _p, _p, _i32, _i32, _f64, _f64, _f64,
                                         _p, _i64, _i32, _i32, _p]
_lib.lora_linear_fwd_noalloc.restype = ctypes.c_int
LORA_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024
_lib.lora_mfma_probe.argtypes = [_i64, _i32, _p, _p, _p]
_lib.lora_mfma_probe.restype = ctypes.c_int
_lib.lora_linear_fwd_phase.argtypes = [_i32, _i32, _p, _i64, _i64, _i64, _p, _i64, _p, _p, _p, _i32, _i32, _f64,
                                       _f64, _f64, _p, _i64, _i32, _i32, _p, _sz, _p]
_lib.lora_linear_fwd_phase.restype = ctypes.c_int
_lib.lora_linear_stacked_fwd.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, ctypes.POINTER(LoraGroup), _i32,
                                         _i32, _f64, _f64, _p, _i64, _i32, _i32, _p, _sz, _p]
_lib.lora_linear_stacked_fwd.restype = ctypes.c_int
_lib.lora_linear_nf4_fwd.argtypes = [_p, _i64, _i64, _i64, _p, _p, _p, _i32, _i64, _p, _p, _p, _i32, _i32,
                                     _f64, _f64, _f64, _p, _i64, _i32, _p, _sz, _p]
_lib.lora_linear_nf4_fwd.restype = ctypes.c_int
_lib.lora_linear_nf4_fwd_ex.argtypes = [_p, _i64, _i64, _i64, _p, _p, _p, _i32, _i64, _p, _p, _p, _i32, _i32,
                                        _f64, _f64, _f64, _p, _i64, _i32, _i32, _p, _sz, _p]
_lib.lora_linear_nf4_fwd_ex.restype = ctypes.c_int
_lib.dense_patch_apply.argtypes = [_p, _i32, ctypes.POINTER(_i64), _i32, _p, _i32, ctypes.POINTER(_i64), _i32,
                                   _f64, _i32, _p]
_lib.dense_patch_apply.restype = ctypes.c_int
_lib.lora_linear_workspace_size.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_i32), _i32, _i32, _i32]
_lib.lora_linear_workspace_size.restype = _sz
_lib.lora_linear_multi_fwd.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, ctypes.POINTER(LoraAdapter), _i32, _i32,
                                       _f64, _p, _i64, _i32, _i32, _p, _sz, _p]
_lib.lora_linear_multi_fwd.restype = ctypes.c_int
_lib.lora_linear_multi_workspace_size.argtypes = [_i64, _i64, _i64, ctypes.POINTER(LoraAdapter), _i32, _i32, _i32]
_lib.lora_linear_multi_workspace_size.restype = _sz
_lib.lora_linear_bwd.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _p, _i32, _f64, _f64, _f64, _p, _i64, _p, _i64,
                                 _p, _p, _p, _p, _i64, _p, _sz, _p]
_lib.lora_linear_bwd.restype = ctypes.c_int
_lib.lora_linear_bwd_workspace_size.argtypes = [_i64, _i64, _i64, _i32, _i32]
_lib.lora_linear_bwd_workspace_size.restype = _sz
_lib.lora_merge_apply.argtypes = [_p, _i32, _i64, _i64, _p, _p, _i32, _i32, _f64, _f64, _i32, _p]
_lib.lora_merge_apply.restype = ctypes.c_int
_lib.lora_linear_nf4_workspace_size.argtypes = [_i64, _i64, _i64, _i32, _i32, _i32]
_lib.lora_linear_nf4_workspace_size.restype = _sz
_lib.lora_status_string.argtypes = [ctypes.c_int]
_lib.lora_status_string.restype = ctypes.c_char_p
_lib.lora_device_check.argtypes = []
_lib.lora_device_check.restype = ctypes.c_int


class LoraError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: status {status} ({lora_status_string(status)})")


def _check(status: int, fn: str) -> int:
    if status != 0:
        raise LoraError(status, fn)
    return status


# ----------------------------------------------------------------- C names, plain integers

def lora_linear_fwd(x, T, K, ldx, W, N, bias, A, B, rank, adapter_dtype, alpha, strength, request_scale,
                    y, ldy, act_dtype, quality, workspace, workspace_bytes, stream):
    return _check(_lib.lora_linear_fwd(x, T, K, ldx, W, N, bias, A, B, rank, adapter_dtype, alpha, strength,
                                       request_scale, y, ldy, act_dtype, quality, workspace, workspace_bytes,
                                       stream), "lora_linear_fwd")


def lora_linear_fwd_noalloc(x, T, K, ldx, W, N, bias, A, B, rank, adapter_dtype, alpha, strength, request_scale,
                            y, ldy, act_dtype, quality, stream):
    return _check(_lib.lora_linear_fwd_noalloc(x, T, K, ldx, W, N, bias, A, B, rank, adapter_dtype, alpha, strength,
                                               request_scale, y, ldy, act_dtype, quality, stream),
                  "lora_linear_fwd_noalloc")


def lora_linear_fwd_phase(phase, gemm_tile, x, T, K, ldx, W, N, bias, A, B, rank, adapter_dtype, alpha, strength,
                          request_scale, y, ldy, act_dtype, quality, workspace, workspace_bytes, stream):
    return _check(_lib.lora_linear_fwd_phase(phase, gemm_tile, x, T, K, ldx, W, N, bias, A, B, rank, adapter_dtype,
                                             alpha, strength, request_scale, y, ldy, act_dtype, quality, workspace,
                                             workspace_bytes, stream), "lora_linear_fwd_phase")


def lora_linear_stacked_fwd(x, T, K, ldx, W, N_total, bias, groups, n_groups, adapter_dtype, strength,
                            request_scale, y, ldy, act_dtype, quality, workspace, workspace_bytes, stream):
    arr = (LoraGroup * max(1, n_groups))(*groups)
    return _check(_lib.lora_linear_stacked_fwd(x, T, K, ldx, W, N_total, bias, arr, n_groups, adapter_dtype,
                                               strength, request_scale, y, ldy, act_dtype, quality, workspace,
                                               workspace_bytes, stream), "lora_linear_stacked_fwd")


def lora_linear_multi_fwd(x, T, K, ldx, W, N, bias, adapters, n_adapters, adapter_dtype, request_scale, y, ldy,
                          act_dtype, quality, workspace, workspace_bytes, stream):
    arr = (LoraAdapter * max(1, n_adapters))(*adapters)
    return _check(_lib.lora_linear_multi_fwd(x, T, K, ldx, W, N, bias, arr, n_adapters, adapter_dtype, request_scale,
                                             y, ldy, act_dtype, quality, workspace, workspace_bytes, stream),
                  "lora_linear_multi_fwd")


def lora_linear_bwd(x, T, K, ldx, W, N, A, B, rank, alpha, strength, request_scale, dy, lddy, dx, lddx, dA, dB, db,
                    t_tilde, ldt, workspace, workspace_bytes, stream):
    return _check(_lib.lora_linear_bwd(x, T, K, ldx, W, N, A, B, rank, alpha, strength, request_scale, dy, lddy, dx,
                                       lddx, dA, dB, db, t_tilde, ldt, workspace, workspace_bytes, stream),
                  "lora_linear_bwd")


def lora_linear_bwd_workspace_size(T, K, N, rank, want_dx=True) -> int:
    return int(_lib.lora_linear_bwd_workspace_size(T, K, N, rank, 1 if want_dx else 0))


def lora_merge_apply(W, w_dtype, N, K, A, B, rank, adapter_dtype, alpha, strength, quality, stream):
    return _check(_lib.lora_merge_apply(W, w_dtype, N, K, A, B, rank, adapter_dtype, alpha, strength, quality, stream),
                  "lora_merge_apply")


def lora_linear_multi_workspace_size(T, K, N, adapters, adapter_dtype, quality=LORA_LOSSLESS) -> int:
    arr = (LoraAdapter * max(1, len(adapters)))(*adapters)
    return int(_lib.lora_linear_multi_workspace_size(T, K, N, arr, len(adapters), adapter_dtype, quality))


def lora_linear_nf4_fwd(x, T, K, ldx, codes, absmax, codebook, blocksize, N, bias, A, B, rank, adapter_dtype,
                        alpha, strength, request_scale, y, ldy, quality, workspace, workspace_bytes, stream):
    return _check(_lib.lora_linear_nf4_fwd(x, T, K, ldx, codes, absmax, codebook, blocksize, N, bias, A, B, rank,
                                           adapter_dtype, alpha, strength, request_scale, y, ldy, quality,
                                           workspace, workspace_bytes, stream), "lora_linear_nf4_fwd")


def lora_linear_nf4_fwd_ex(x, T, K, ldx, codes, absmax, codebook, blocksize, N, bias, A, B, rank, adapter_dtype,
                           alpha, strength, request_scale, y, ldy, quality, dequant, workspace, workspace_bytes,
                           stream):
    return _check(_lib.lora_linear_nf4_fwd_ex(x, T, K, ldx, codes, absmax, codebook, blocksize, N, bias, A, B, rank,
                                              adapter_dtype, alpha, strength, request_scale, y, ldy, quality,
                                              dequant, workspace, workspace_bytes, stream), "lora_linear_nf4_fwd_ex")


def dense_patch_apply(dst, dst_dtype, dst_shape, src, src_dtype, src_shape, strength, mode, stream):
    ds = (_i64 * max(1, len(dst_shape)))(*dst_shape)
    ss = (_i64 * max(1, len(src_shape)))(*src_shape)
    return _check(_lib.dense_patch_apply(dst, dst_dtype, ds, len(dst_shape), src, src_dtype, ss, len(src_shape),
                                         strength, mode, stream), "dense_patch_apply")


def lora_linear_workspace_size(T, K, N, ranks, adapter_dtype, quality=LORA_LOSSLESS) -> int:
    arr = (_i32 * max(1, len(ranks)))(*ranks)
    return int(_lib.lora_linear_workspace_size(T, K, N, arr, len(ranks), adapter_dtype, quality))


def lora_linear_nf4_workspace_size(T, K, N, rank, adapter_dtype, quality=LORA_LOSSLESS) -> int:
    return int(_lib.lora_linear_nf4_workspace_size(T, K, N, rank, adapter_dtype, quality))


def lora_status_string(status: int) -> str:
    return _lib.lora_status_string(status).decode()


def lora_device_check() -> int:
    return int(_lib.lora_device_check())


def lora_mfma_probe(iters, blocks, sink, clocks, stream):
    return _check(_lib.lora_mfma_probe(iters, blocks, sink, clocks, stream), "lora_mfma_probe")


def hip_runtimes_mapped() -> list:
    """Distinct libamdhip64 files mapped into this process (exactly one is expected)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(os.path.realpath(line.split()[-1]))
    return sorted(paths)


# ----------------------------------------------------------------- tensor-level helpers

def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LORA_BF16
    if t.dtype == torch.float32:
        return LORA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _row_major(t: torch.Tensor, name: str):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    return t.stride(0)


def _workspace(T, K, N, ranks, adapter_dtype, quality, workspace, device):
    need = lora_linear_workspace_size(T, K, N, list(ranks), adapter_dtype, quality)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace, need


def lora_linear(x, W, b, A, B, alpha, strength=1.0, request_scale=1.0, out=None, quality="lossless",
                workspace=None, stream=None, gemm_tile=None):
    """y = x.W^T + b + s.(x.A^T).B^T on the GPU; returns ``out`` (allocated when None).

    ``gemm_tile`` (lossless only): None or 0 lets the library pick the hot GEMM's output
    tile, 1 fixes 256 x 256, 2 fixes 128 x 128 (same bits, different speed)."""
    T, K = x.shape
    N = W.shape[0]
    ldx = _row_major(x, "x")
    if out is None:
        out = torch.empty((T, N), dtype=x.dtype, device=x.device)
    ldy = _row_major(out, "out")
    rank = 0 if A is None else A.shape[0]
    adt = _dt(A) if A is not None else _dt(x)
    q = _QUALITY[quality]
    ws, need = _workspace(T, K, N, [rank] if rank else [], adt, q, workspace, x.device)
    args = (x.data_ptr(), T, K, ldx, W.data_ptr(), N, _ptr(b), _ptr(A), _ptr(B), rank, adt, float(alpha),
            float(strength), float(request_scale), out.data_ptr(), ldy, _dt(x), q, ws.data_ptr(), ws.numel(),
            _stream(stream))
    if gemm_tile:
        lora_linear_fwd_phase(0, int(gemm_tile), *args)
    else:
        lora_linear_fwd(*args)
    return out


def lora_linear_stacked(x, W, b, groups, strength=1.0, request_scale=1.0, out=None, quality="lossless",
                        workspace=None, stream=None):
    """Stacked groups: ``groups`` is a list of dicts with A, B, alpha, col_offset, n_cols."""
    T, K = x.shape
    N = W.shape[0]
    ldx = _row_major(x, "x")
    if out is None:
        out = torch.empty((T, N), dtype=x.dtype, device=x.device)
    ldy = _row_major(out, "out")
    adt = _dt(groups[0]["A"]) if groups else _dt(x)
    cg = [LoraGroup(_ptr(g["A"]), _ptr(g["B"]), 0 if g["A"] is None else g["A"].shape[0], 0, float(g["alpha"]),
                    int(g["col_offset"]), int(g["n_cols"])) for g in groups]
    q = _QUALITY[quality]
    ws, need = _workspace(T, K, N, [g.rank for g in cg if g.rank > 0], adt, q, workspace, x.device)
    lora_linear_stacked_fwd(x.data_ptr(), T, K, ldx, W.data_ptr(), N, _ptr(b), cg, len(cg), adt, float(strength),
                            float(request_scale), out.data_ptr(), ldy, _dt(x), q, ws.data_ptr(), ws.numel(),
                            _stream(stream))
    return out


def lora_linear_multi(x, W, b, adapters, request_scale=1.0, out=None, quality="lossless", workspace=None,
                      stream=None):
    """Several adapters on one layer: ``adapters`` is a list of dicts with A, B, c (legacy
    lora_B bias or None), alpha, strength, col_offset, n_cols; column ranges may overlap."""
    T, K = x.shape
    N = W.shape[0]
    ldx = _row_major(x, "x")
    if out is None:
        out = torch.empty((T, N), dtype=x.dtype, device=x.device)
    ldy = _row_major(out, "out")
    adt = _dt(adapters[0]["A"]) if adapters else _dt(x)
    ca = [LoraAdapter(_ptr(a["A"]), _ptr(a["B"]), _ptr(a.get("c")), 0 if a["A"] is None else a["A"].shape[0], 0,
                      float(a["alpha"]), float(a["strength"]), int(a["col_offset"]), int(a["n_cols"]))
          for a in adapters]
    q = _QUALITY[quality]
    need = lora_linear_multi_workspace_size(T, K, N, ca, adt, q)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    lora_linear_multi_fwd(x.data_ptr(), T, K, ldx, W.data_ptr(), N, _ptr(b), ca, len(ca), adt, float(request_scale),
                          out.data_ptr(), ldy, _dt(x), q, ws.data_ptr(), ws.numel(), _stream(stream))
    return out


def lora_linear_nf4(x, codes, absmax, codebook, N, b, A, B, alpha, strength=1.0, request_scale=1.0,
                    blocksize=64, out=None, quality="lossless", workspace=None, stream=None, dequant="auto"):
    """``dequant``: "auto", "panel" or "in_gemm" (where a lossless call with more than 64 tokens
    dequantizes the 4-bit weight; the same output bits either way)."""
    T, K = x.shape
    ldx = _row_major(x, "x")
    if out is None:
        out = torch.empty((T, N), dtype=x.dtype, device=x.device)
    ldy = _row_major(out, "out")
    rank = 0 if A is None else A.shape[0]
    adt = _dt(A) if A is not None else LORA_BF16
    q = _QUALITY[quality]
    need = lora_linear_nf4_workspace_size(T, K, N, rank, adt, q)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    lora_linear_nf4_fwd_ex(x.data_ptr(), T, K, ldx, codes.data_ptr(), absmax.data_ptr(), codebook.data_ptr(),
                           blocksize, N, _ptr(b), _ptr(A), _ptr(B), rank, adt, float(alpha), float(strength),
                           float(request_scale), out.data_ptr(), ldy, q, _DEQUANT[dequant], ws.data_ptr(),
                           ws.numel(), _stream(stream))
    return out


def lora_merge(W, A, B, alpha, strength=1.0, quality="lossless", stream=None):
    """W <- RN(W + (alpha / rank) . strength . B.A) in place on the GPU; returns ``W``."""
    N, K = W.shape
    if not (W.is_contiguous() and A.is_contiguous() and B.is_contiguous()):
        raise ValueError("lora_merge needs contiguous tensors")
    lora_merge_apply(W.data_ptr(), _dt(W), N, K, A.data_ptr(), B.data_ptr(), A.shape[0], _dt(A), float(alpha),
                     float(strength), _QUALITY[quality], _stream(stream))
    return W


def lora_linear_backward(x, W, A, B, dy, alpha, strength=1.0, request_scale=1.0, want=("dx", "dA", "dB", "db"),
                         workspace=None, stream=None, t_tilde=None):
    """Gradients of the LoRA linear for the output gradient ``dy``: returns (dx, dA, dB, db),
    each None unless named in ``want`` (dx bf16; dA, dB, db fp32). ``t_tilde``: optional bf16
    [T, ldt] tensor holding the forward's t~ (for instance a view of the forward call's
    workspace), so that x is not read again to recompute it."""
    T, K = x.shape
    N = W.shape[0]
    r = A.shape[0]
    ldx, lddy = _row_major(x, "x"), _row_major(dy, "dy")
    dev = x.device
    dx = torch.empty((T, K), dtype=torch.bfloat16, device=dev) if "dx" in want else None
    dA = torch.empty((r, K), dtype=torch.float32, device=dev) if "dA" in want else None
    dB = torch.empty((N, r), dtype=torch.float32, device=dev) if "dB" in want else None
    db = torch.empty((N,), dtype=torch.float32, device=dev) if "db" in want else None
    need = lora_linear_bwd_workspace_size(T, K, N, r, dx is not None)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ldt = _row_major(t_tilde, "t_tilde") if t_tilde is not None else 0
    lora_linear_bwd(x.data_ptr(), T, K, ldx, W.data_ptr(), N, A.data_ptr(), B.data_ptr(), r, float(alpha),
                    float(strength), float(request_scale), dy.data_ptr(), lddy, _ptr(dx), K, _ptr(dA), _ptr(dB),
                    _ptr(db), _ptr(t_tilde), ldt, ws.data_ptr(), ws.numel(), _stream(stream))
    return dx, dA, dB, db


def dense_patch(dst, src, strength, mode="add", stream=None):
    """Apply a dense payload to ``dst`` in place; returns ``dst``."""
    if not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("dense_patch needs contiguous tensors")
    dense_patch_apply(dst.data_ptr(), _dt(dst), list(dst.shape), src.data_ptr(), _dt(src), list(src.shape),
                      float(strength), _MODE[mode], _stream(stream))
    return dst
