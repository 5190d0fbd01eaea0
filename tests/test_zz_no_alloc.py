"""lora_linear_fwd_noalloc (the entry point for callers that cannot allocate) against
lora_linear_fwd through the C-ABI: the same kernels, so the same bits, on two calls in a
row (the second smaller, after the first has left its data in the shared scratch array),
over the paths that use scratch: the rank-wide intermediate, the producer's K-split
partial sums, the few-token partial sums, the fp32-adapter split copies, the exact tier.
A call that would need more than the array holds is rejected before anything runs."""
import numpy as np
import pytest
import torch

import lora_workloads as lw
import rank_gemm_lora_amd as rg
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _args(d, y, adt, act, q):
    T, K = d["x"].shape
    N = d["W"].shape[0]
    A, B = d["A"], d["B"]
    return (d["x"].data_ptr(), T, K, K, d["W"].data_ptr(), N, None if d["b"] is None else d["b"].data_ptr(),
            None if A is None else A.data_ptr(), None if B is None else B.data_ptr(), 0 if A is None else A.shape[0],
            adt, d["alpha"], d["strength"], d["request_scale"], y.data_ptr(), N, act, q)


def _pair(shape, seed, adapter="bf16", act="bf16", quality="lossless", inactive=False):
    T, K, N, r = shape
    h = lw.small_linear_inputs(T, K, N, r, seed, act=act, adapter=adapter, bias=True, alpha=2.0 * r, strength=0.8,
                               request_scale=0.7)
    d = {k: (dev(v) if hasattr(v, "to") else v) for k, v in h.items()}
    if inactive:
        d["A"], d["B"] = None, None
    adt = rg.LORA_F32 if adapter == "f32" else rg.LORA_BF16
    actc = rg.LORA_F32 if act == "f32" else rg.LORA_BF16
    q = rg.LORA_EXACT if quality == "exact" else rg.LORA_LOSSLESS
    dt = torch.float32 if act == "f32" else torch.bfloat16
    y_ref = torch.full((T, N), float("nan"), dtype=dt, device="cuda:0")
    y_na = torch.full((T, N), float("nan"), dtype=dt, device="cuda:0")
    ranks = [] if inactive else [r]
    ws = torch.empty(max(1, rg.lora_linear_workspace_size(T, K, N, ranks, adt, q)), dtype=torch.uint8,
                     device="cuda:0")
    s = torch.cuda.current_stream().cuda_stream
    return d, (y_ref, y_na), (adt, actc, q), ws, s


CASES = [  # (first call, second call smaller), options
    (((300, 512, 520, 24), (130, 256, 300, 24)), {}),
    (((4352, 1536, 1536, 32), (2000, 1536, 700, 32)), {}),                 # producer K split
    (((64, 8960, 1536, 64), (20, 1536, 520, 16)), {}),                     # few tokens
    (((64, 8960, 8960, 64), (16, 4096, 3000, 32)), {}),                    # few tokens, 41.6 MB of scratch
    (((300, 512, 520, 24), (100, 256, 200, 8)), {"adapter": "f32"}),       # hi/lo split copies
    (((200, 256, 300, 24), (50, 128, 96, 8)), {"quality": "exact"}),
    (((64, 128, 96, 8), (33, 128, 40, 8)), {"act": "f32", "adapter": "f32"}),
    (((300, 512, 520, 24), (100, 256, 200, 24)), {"inactive": True}),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_equals_fwd_on_two_calls(case):
    shapes, opt = CASES[case]
    for i, shape in enumerate(shapes):
        say(f"case noalloc {case} call {i}: T,K,N,r={shape} {opt}")
        d, (y_ref, y_na), (adt, act, q), ws, s = _pair(shape, 70 + 3 * case + i, **opt)
        rg.lora_linear_fwd(*_args(d, y_ref, adt, act, q), ws.data_ptr(), ws.numel(), s)
        rg.lora_linear_fwd_noalloc(*_args(d, y_na, adt, act, q), s)
        torch.cuda.synchronize()
        assert not bool(torch.isnan(y_na).any()), "output not completely written"
        assert torch.equal(y_ref, y_na), f"{(y_ref != y_na).sum().item()} outputs differ"


def test_noalloc_rejects_calls_beyond_its_scratch():
    T, K, N, r = 4096, 8192, 8192, 1024   # fp32 adapter split layout: far beyond 32 MiB
    need = rg.lora_linear_workspace_size(T, K, N, [r], rg.LORA_F32, rg.LORA_LOSSLESS)
    assert need > rg.LORA_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda:0")  # never read: the call stops before any launch
    st = rg._lib.lora_linear_fwd_noalloc(x.data_ptr(), T, K, K, x.data_ptr(), N, None, x.data_ptr(), x.data_ptr(), r,
                                         rg.LORA_F32, 1.0, 1.0, 1.0, x.data_ptr(), N, rg.LORA_BF16,
                                         rg.LORA_LOSSLESS, None)
    assert st == 8  # LORA_ERR_UNSUPPORTED
    assert rg._lib.lora_linear_fwd_noalloc(None, 0, K, K, x.data_ptr(), N, None, None, None, 0, rg.LORA_BF16, 1.0,
                                           1.0, 1.0, None, N, rg.LORA_BF16, rg.LORA_LOSSLESS, None) == 0  # T == 0
