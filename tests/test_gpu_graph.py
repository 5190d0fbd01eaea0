"""The library's calls captured in a HIP graph: every replay gives the eager call's bits.

Callers that capture (serving loops, the few-token regimes replayed per step) need every launch of
a call to be capturable and to give the same result on every replay. Covered: the hot path (one
adapter and two per tile), the rank-wide producer's K split with its finishing kernel, the
few-token path, the fp32-adapter split, the 4-bit panel and the 4-bit weight dequantized inside the
GEMM, the no-allocation entry point and the
backward, including its empty batch, which writes zero gradients by kernel. Each graph is replayed
several times with eager work between the replays (the output is overwritten before each one),
and each replay is compared with the eager result bit for bit.
"""
import numpy as np
import pytest
import torch

import lora_workloads as lw
import rank_gemm_lora_amd as rg
from tests.gpu_util import DEV, dev, say

pytestmark = pytest.mark.gpu


def _replays_equal(fn, outs, n_replays=4):
    """Run fn eagerly, capture it, replay it n_replays times with the outputs overwritten and eager
    work in between, and check every replay against the eager outputs."""
    fn()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # (a warm call on the capture stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    scratch = torch.empty(1 << 20, device=DEV)
    for k in range(n_replays):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else 7)
        scratch.normal_()  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o, r), f"replay {k}, output {i}"


@pytest.mark.parametrize("T,K,N,r,adapter", [(300, 256, 520, 24, "bf16"), (300, 2048, 520, 32, "bf16"),
                                              (20, 512, 300, 64, "bf16"), (300, 384, 520, 64, "f32")])
def test_linear_in_a_graph(T, K, N, r, adapter):
    d = lw.small_linear_inputs(T, K, N, r, 11 + r, adapter=adapter, bias=True, alpha=2.0 * r, strength=0.8,
                               request_scale=0.7)
    say(f"case graph linear T={T} K={K} N={N} r={r} adapter={adapter}")
    x, W, b, A, B = dev(d["x"]), dev(d["W"]), dev(d["b"]), dev(d["A"]), dev(d["B"])
    adt = rg.LORA_F32 if adapter == "f32" else rg.LORA_BF16
    ws = torch.empty(max(1, rg.lora_linear_workspace_size(T, K, N, [r], adt)), dtype=torch.uint8, device=DEV)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    _replays_equal(lambda: rg.lora_linear(x, W, b, A, B, d["alpha"], 0.8, 0.7, out=y, workspace=ws), [y])


def test_stacked_two_groups_per_tile_in_a_graph():
    rng = np.random.default_rng(5)
    T, K, Nt = 300, 256, 700
    specs = [(24, 48.0, 0, 200), (16, 8.0, 248, 300), (64, 64.0, 560, 140)]
    x = dev(lw.to_dtype(rng.standard_normal((T, K)), "bf16"))
    W = dev(lw.to_dtype(rng.standard_normal((Nt, K)) / np.sqrt(K), "bf16"))
    groups = [dict(A=dev(lw.to_dtype(rng.standard_normal((r, K)) / np.sqrt(K), "bf16")),
                   B=dev(lw.to_dtype(rng.standard_normal((n, r)) * np.sqrt(0.02), "bf16")),
                   rank=r, alpha=a, col_offset=o, n_cols=n) for r, a, o, n in specs]
    say("case graph stacked")
    ws = torch.empty(max(1, rg.lora_linear_workspace_size(T, K, Nt, [g["rank"] for g in groups], rg.LORA_BF16)),
                     dtype=torch.uint8, device=DEV)
    y = torch.empty((T, Nt), dtype=torch.bfloat16, device=DEV)
    _replays_equal(lambda: rg.lora_linear_stacked(x, W, None, groups, 0.9, 0.8, out=y, workspace=ws), [y])


def test_nf4_panel_in_a_graph():
    rng = np.random.default_rng(41)
    T, K, N, r = 130, 256, 300, 16
    x = dev(lw.to_dtype(rng.standard_normal((T, K)), "bf16"))
    codes = dev(torch.from_numpy(rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)))
    absmax = dev(torch.from_numpy(np.abs(rng.standard_normal(N * K // 64)) * np.sqrt(0.05)).float())
    cb = dev(lw.nf4_style_codebook())
    A = dev(lw.to_dtype(rng.standard_normal((r, K)) / np.sqrt(K), "bf16"))
    B = dev(lw.to_dtype(rng.standard_normal((N, r)) * np.sqrt(0.02), "bf16"))
    say("case graph 4-bit panel")
    ws = torch.empty(max(1, rg.lora_linear_nf4_workspace_size(T, K, N, r, rg.LORA_BF16)), dtype=torch.uint8,
                     device=DEV)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    _replays_equal(lambda: rg.lora_linear_nf4(x, codes, absmax, cb, N, None, A, B, 32.0, 1.0, 1.0, out=y,
                                              workspace=ws), [y])


def test_nf4_in_gemm_in_a_graph():
    rng = np.random.default_rng(43)
    T, K, N, r = 300, 256, 300, 16
    x = dev(lw.to_dtype(rng.standard_normal((T, K)), "bf16"))
    codes = dev(torch.from_numpy(rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)))
    absmax = dev(torch.from_numpy(np.abs(rng.standard_normal(N * K // 64)) * np.sqrt(0.05)).float())
    cb = dev(lw.nf4_style_codebook())
    A = dev(lw.to_dtype(rng.standard_normal((r, K)) / np.sqrt(K), "bf16"))
    B = dev(lw.to_dtype(rng.standard_normal((N, r)) * np.sqrt(0.02), "bf16"))
    say("case graph 4-bit in-GEMM")
    ws = torch.empty(max(1, rg.lora_linear_workspace_size(T, K, N, [r], rg.LORA_BF16)), dtype=torch.uint8,
                     device=DEV)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    _replays_equal(lambda: rg.lora_linear_nf4(x, codes, absmax, cb, N, None, A, B, 32.0, 1.0, 1.0, out=y,
                                              workspace=ws, dequant="in_gemm"), [y])


def test_noalloc_in_a_graph():
    d = lw.small_linear_inputs(300, 2048, 520, 32, 3, bias=True, alpha=64.0, strength=0.8, request_scale=0.7)
    x, W, b, A, B = dev(d["x"]), dev(d["W"]), dev(d["b"]), dev(d["A"]), dev(d["B"])
    y = torch.empty((300, 520), dtype=torch.bfloat16, device=DEV)
    say("case graph no-allocation entry point")

    def call():
        rg.lora_linear_fwd_noalloc(x.data_ptr(), 300, 2048, 2048, W.data_ptr(), 520, b.data_ptr(), A.data_ptr(),
                                   B.data_ptr(), 32, rg.LORA_BF16, d["alpha"], 0.8, 0.7, y.data_ptr(), 520,
                                   rg.LORA_BF16, rg.LORA_LOSSLESS, torch.cuda.current_stream().cuda_stream)
    _replays_equal(call, [y])


@pytest.mark.parametrize("T", [300, 0])
def test_backward_in_a_graph(T):
    K, N, r = 256, 520, 24
    d = lw.small_linear_inputs(max(T, 1), K, N, r, 7, bias=False, alpha=48.0)
    rng = np.random.default_rng(8)
    x = dev(d["x"])[:T]
    dy = dev(lw.to_dtype(rng.standard_normal((max(T, 1), N)), "bf16"))[:T]
    W, A, B = dev(d["W"]), dev(d["A"]), dev(d["B"])
    say(f"case graph backward T={T}")
    ws = torch.empty(max(1, rg.lora_linear_bwd_workspace_size(T, K, N, r, True)), dtype=torch.uint8, device=DEV)
    dx = torch.empty((T, K), dtype=torch.bfloat16, device=DEV)
    dA = torch.empty((r, K), device=DEV)
    dB = torch.empty((N, r), device=DEV)
    db = torch.empty((N,), device=DEV)

    def call():
        rg.lora_linear_bwd(x.data_ptr(), T, K, K, W.data_ptr(), N, A.data_ptr(), B.data_ptr(), r, 48.0, 1.0, 1.0,
                           dy.data_ptr(), N, dx.data_ptr() if T else None, K, dA.data_ptr(), dB.data_ptr(),
                           db.data_ptr(), None, 0, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    outs = ([dx] if T else []) + [dA, dB, db]
    _replays_equal(call, outs)
    if T == 0:
        assert not dA.any() and not dB.any() and not db.any()
