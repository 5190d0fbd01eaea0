"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle, at sizes
the oracle finishes in seconds that still span several tiles and ragged tails.

Exact tier: bit-identical to the separate-pass chain. Lossless tier: relative
RMS <= 4e-3 against fp64 (1e-6 for fp32 outputs) and no larger than the chain's
error; bit-identical to the exact result on dyadic inputs where every rounding
is the identity. Each GPU step prints its case first.
"""
import json
import os

import numpy as np
import pytest
import torch

import lora_workloads as lw
import rank_gemm_lora_amd as rg
from oracle import exact_chain as ec
from oracle import lora_oracle as lo
from tests.gpu_util import (DEV, LOSSLESS_F32_GATE, assert_bitwise, assert_gate, dev, host64, say)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_exact_chain.json")


def run_linear(d, quality, act="bf16", adapter="bf16", strength=None, request_scale=None, A="A", B="B"):
    x, W, b = dev(d["x"]), dev(d["W"]), dev(d["b"])
    Ad = dev(d[A]) if A else None
    Bd = dev(d[B]) if B else None
    y = rg.lora_linear(x, W, b, Ad, Bd, d["alpha"], d["strength"] if strength is None else strength,
                       d["request_scale"] if request_scale is None else request_scale, quality=quality)
    torch.cuda.synchronize()
    return y


def oracle_pair(d, act="bf16", adapter="bf16", strength=None, request_scale=None):
    st = d["strength"] if strength is None else strength
    rs = d["request_scale"] if request_scale is None else request_scale
    args = (d["x"], d["W"], d["b"], d["A"], d["B"], d["alpha"], d["rank"], st, rs)
    return lo.lora_linear(*args), ec.chain_linear(*args, act, adapter)


def test_device_is_gfx950_and_one_runtime():
    assert rg.lora_device_check() == 0
    assert len(rg.hip_runtimes_mapped()) == 1, rg.hip_runtimes_mapped()


# ------------------------------------------------------------------ fp32 tiny layer

@pytest.mark.parametrize("variant", ["base", "strength_half", "B_zero"])
def test_tiny_fp32(variant):
    s = lw.TINY_FP32
    d = lw.linear_inputs(s)
    strength = 0.5 if variant == "strength_half" else 1.0
    if variant == "B_zero":
        d["B"] = torch.zeros_like(d["B"])
    say(f"case tiny_fp32 {variant}")
    y64, yc = oracle_pair(d, "f32", "f32", strength=strength)
    y = run_linear(d, "lossless", strength=strength)
    e = lo.rel_rms(host64(y), y64)
    say(f"  lossless rel_rms {e:.3e}")
    assert e <= LOSSLESS_F32_GATE
    ye = run_linear(d, "exact", strength=strength)
    assert_bitwise(ye, yc, "tiny fp32 exact")
    if variant == "B_zero":  # base only, bitwise, in both tiers
        yb = rg.lora_linear(dev(d["x"]), dev(d["W"]), dev(d["b"]), None, None, d["alpha"], quality="exact")
        assert torch.equal(ye, yb)


def test_tiny_fp32_half_strength_equals_unit_scale():
    # alpha/rank = 2 and strength 0.5: combined s = 1 (skipped); the chain multiplies
    # by 2 then 0.5, both exact, so all three outputs agree bit for bit.
    d = lw.linear_inputs(lw.TINY_FP32)
    say("case tiny_fp32 half strength == unit")
    y_half = run_linear(d, "exact", strength=0.5)
    y_unit = rg.lora_linear(dev(d["x"]), dev(d["W"]), dev(d["b"]), dev(d["A"]), dev(d["B"]), 8.0, 1.0, 1.0,
                            quality="exact")
    assert torch.equal(y_half, y_unit)
    yl_half = run_linear(d, "lossless", strength=0.5)
    yl_unit = rg.lora_linear(dev(d["x"]), dev(d["W"]), dev(d["b"]), dev(d["A"]), dev(d["B"]), 8.0, 1.0, 1.0)
    assert torch.equal(yl_half, yl_unit)


# ------------------------------------------------------------------ bf16, several tiles, ragged tails

CASES = [
    # T, K, N, rank, bias, seed   (tiles are 256 x 256 with 64-wide K steps)
    (300, 200, 520, 24, True, 1),     # ragged T, K, N; rank padded to 64
    (513, 384, 768, 64, False, 2),    # one-row M tail
    (64, 136, 96, 5, True, 3),        # rank not a multiple of 8
    (257, 1536, 300, 32, True, 4),    # long K
    (40, 64, 1000, 128, True, 5),     # two K-extension steps
]


@pytest.mark.parametrize("T,K,N,r,bias,seed", CASES)
def test_bf16_linear(T, K, N, r, bias, seed):
    d = lw.small_linear_inputs(T, K, N, r, seed, bias=bias, alpha=2.0 * r, strength=0.8, request_scale=0.7)
    say(f"case bf16 T={T} K={K} N={N} r={r} bias={bias}")
    y64, yc = oracle_pair(d)
    y = run_linear(d, "lossless")
    assert_gate(y, y64, yc, what="lossless")
    ye = run_linear(d, "exact")
    assert_bitwise(ye, yc, "exact")


@pytest.mark.parametrize("T,K,N,r", [(300, 256, 520, 24), (70, 64, 40, 8)])
def test_bf16_std_spread_variant(T, K, N, r):
    # second accuracy case: the std reading of N(0, v) (delta ~ 0.1 of base)
    s = lw.LinearSpec("std", T=T, K=K, N=N, rank=r, alpha=r, strength=1.0, request_scale=0.7, bias=True, seed=9)
    d = lw.linear_inputs(s, spread="std")
    say(f"case bf16 std-spread T={T} K={K} N={N} r={r}")
    y64, yc = oracle_pair(d)
    assert_gate(run_linear(d, "lossless"), y64, yc, what="lossless std")
    assert_bitwise(run_linear(d, "exact"), yc, "exact std")


@pytest.mark.parametrize("T,seed", [(290, 0), (290, 1), (50, 2), (1, 3)])
def test_dyadic_inputs_lossless_is_exact(T, seed):
    K, N, r = 192, 300, 16
    d = lw.dyadic_linear_inputs(T, K, N, r, seed, bias=True, density=0.08)
    say(f"case dyadic T={T} seed={seed}")
    xd, Wd, bd, Ad, Bd = (lo.f64(d[k]) for k in ("x", "W", "b", "A", "B"))
    y64 = lo.lora_linear(d["x"], d["W"], d["b"], d["A"], d["B"], 16.0, r, 1.0, 1.0)
    # every intermediate exactly representable: t in bf16, the result in bf16
    t = xd @ Ad.T
    assert np.array_equal(ec.rn_bf16(ec.rn_f32(t)), t)
    assert np.array_equal(ec.rn_bf16(ec.rn_f32(y64)), y64)
    y = rg.lora_linear(dev(d["x"]), dev(d["W"]), dev(d["b"]), dev(d["A"]), dev(d["B"]), 16.0, 1.0, 1.0)
    torch.cuda.synchronize()
    assert_bitwise(y, y64, "lossless dyadic")
    ye = rg.lora_linear(dev(d["x"]), dev(d["W"]), dev(d["b"]), dev(d["A"]), dev(d["B"]), 16.0, 1.0, 1.0,
                        quality="exact")
    torch.cuda.synchronize()
    assert_bitwise(ye, y64, "exact dyadic")


@pytest.mark.parametrize("T", [300, 33])
def test_inactive_adapter_is_base_only_bitwise(T):
    d = lw.small_linear_inputs(T, 200, 520, 24, 7, bias=True, alpha=24.0)
    x, W, b, A, B = (dev(d[k]) for k in ("x", "W", "b", "A", "B"))
    say(f"case inactive adapter T={T}")
    for q in ("lossless", "exact"):
        y_none = rg.lora_linear(x, W, b, None, None, 24.0, quality=q)
        y_s0 = rg.lora_linear(x, W, b, A, B, 24.0, 0.0, 1.0, quality=q)
        y_neg0 = rg.lora_linear(x, W, b, A, B, 24.0, -0.0, 1.0, quality=q)
        y_B0 = rg.lora_linear(x, W, b, A, torch.zeros_like(B), 24.0, 1.0, 1.0, quality=q)
        torch.cuda.synchronize()
        assert torch.equal(y_none, y_s0) and torch.equal(y_none, y_neg0)
        assert not bool((y_none == 0).any())
        assert torch.equal(y_none, y_B0)
    base_chain = ec.chain_linear(d["x"], d["W"], d["b"], None, None, 24.0, 24, 1.0, 1.0)
    assert_bitwise(rg.lora_linear(x, W, b, None, None, 24.0, quality="exact"), base_chain, "base exact")


def test_request_scale_is_read_per_call():
    d = lw.small_linear_inputs(300, 128, 260, 16, 8, bias=True, alpha=16.0)
    say("case request scale per call")
    outs = []
    for rs in (0.7, 0.3, 0.7):
        y = run_linear(d, "lossless", request_scale=rs)
        y64, yc = oracle_pair(d, request_scale=rs)
        assert_gate(y, y64, yc, what=f"rs={rs}")
        outs.append(y.clone())
    assert not torch.equal(outs[0], outs[1])
    assert torch.equal(outs[0], outs[2])


def test_default_quality_is_lossless_and_deterministic():
    d = lw.small_linear_inputs(300, 200, 520, 24, 11, bias=True, alpha=48.0, strength=0.8, request_scale=0.7)
    say("case default quality + determinism")
    x, W, b, A, B = (dev(d[k]) for k in ("x", "W", "b", "A", "B"))
    y_default = rg.lora_linear(x, W, b, A, B, 48.0, 0.8, 0.7)
    y_lossless = rg.lora_linear(x, W, b, A, B, 48.0, 0.8, 0.7, quality="lossless")
    y_again = rg.lora_linear(x, W, b, A, B, 48.0, 0.8, 0.7)
    torch.cuda.synchronize()
    assert torch.equal(y_default, y_lossless) and torch.equal(y_default, y_again)


@pytest.mark.parametrize("T,K,N,r,adapter", [(300, 200, 520, 24, "bf16"), (513, 384, 768, 64, "bf16"),
                                              (257, 512, 300, 64, "f32"), (64, 136, 96, 5, "bf16"),
                                              (300, 2048, 520, 32, "bf16")])  # the last: producer K split
def test_phases_compose_to_the_fused_call(T, K, N, r, adapter):
    """Phase 1 (rank-wide producer) then phase 2 (fused GEMM) equal lora_linear_fwd bit for bit."""
    d = lw.small_linear_inputs(T, K, N, r, 21, bias=True, alpha=2.0 * r, strength=0.8, request_scale=0.7)
    say(f"case phases T={T} K={K} N={N} r={r} adapter={adapter}")
    x, W, b = dev(d["x"]), dev(d["W"]), dev(d["b"])
    adt = rg.LORA_F32 if adapter == "f32" else rg.LORA_BF16
    tdt = torch.float32 if adapter == "f32" else torch.bfloat16
    A, B = dev(d["A"]).to(tdt).contiguous(), dev(d["B"]).to(tdt).contiguous()
    ws = torch.empty(max(1, rg.lora_linear_workspace_size(T, K, N, [r], adt)), dtype=torch.uint8, device=DEV)
    y_one = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    y_two = torch.full((T, N), 3.0, dtype=torch.bfloat16, device=DEV)
    sp = torch.cuda.current_stream().cuda_stream
    args = (x.data_ptr(), T, K, K, W.data_ptr(), N, b.data_ptr(), A.data_ptr(), B.data_ptr(), r, adt,
            d["alpha"], 0.8, 0.7)
    tail = (rg.LORA_BF16, rg.LORA_LOSSLESS, ws.data_ptr(), ws.numel(), sp)
    rg.lora_linear_fwd(*args, y_one.data_ptr(), N, *tail)
    ws.zero_()
    rg.lora_linear_fwd_phase(1, 0, *args, y_two.data_ptr(), N, *tail)
    torch.cuda.synchronize()
    assert bool((y_two == 3.0).all())      # phase 1 writes only the workspace
    rg.lora_linear_fwd_phase(2, 0, *args, y_two.data_ptr(), N, *tail)
    torch.cuda.synchronize()
    assert torch.equal(y_one, y_two)


def test_column_view_output_with_wider_ldy():
    d = lw.small_linear_inputs(130, 128, 200, 16, 12, bias=True, alpha=16.0, strength=0.9)
    say("case column view")
    x, W, b, A, B = (dev(d[k]) for k in ("x", "W", "b", "A", "B"))
    for q in ("lossless", "exact"):
        wide = torch.full((130, 328), 7.0, dtype=torch.bfloat16, device=DEV)
        view = wide[:, 64:264]
        rg.lora_linear(x, W, b, A, B, 16.0, 0.9, 1.0, out=view, quality=q)
        ref = rg.lora_linear(x, W, b, A, B, 16.0, 0.9, 1.0, quality=q)
        torch.cuda.synchronize()
        assert torch.equal(view, ref)
        assert bool((wide[:, :64] == 7.0).all()) and bool((wide[:, 264:] == 7.0).all())


# ------------------------------------------------------------------ more tiles than compute units
# Launches of several waves of output tiles (one adapter over all columns, or
# none), against launches small enough for one wave, bitwise, and against the
# oracle. Ragged T and N, K tails, 1, 2 and 4 K-extension stages.

@pytest.mark.parametrize("T,K,N,r,bias", [(2600, 200, 13000, 24, True), (2600, 512, 6000, 100, False),
                                          (1100, 256, 16000, 200, True), (2600, 320, 6000, 0, True)])
def test_more_tiles_than_compute_units(T, K, N, r, bias):
    rank = max(r, 1)
    d = lw.small_linear_inputs(T, K, N, rank, 40 + r, bias=bias, alpha=2.0 * rank, strength=0.9,
                               request_scale=0.7)
    say(f"case many tiles T={T} K={K} N={N} r={r} bias={bias}")
    x, W, b = dev(d["x"]), dev(d["W"]), dev(d["b"])
    A, B = (dev(d["A"]), dev(d["B"])) if r else (None, None)
    y = rg.lora_linear(x, W, b, A, B, d["alpha"], 0.9, 0.7)
    torch.cuda.synchronize()
    rows = min(T, 256 * (256 // -(-N // 256)))  # whole tile rows of a launch with at most 256 tiles
    y_few = rg.lora_linear(x[:rows].contiguous(), W, b, A, B, d["alpha"], 0.9, 0.7)
    torch.cuda.synchronize()
    assert torch.equal(y[:rows], y_few), "a launch of several tile waves and one of a single wave differ"
    if r:
        y64, yc = oracle_pair(d, strength=0.9, request_scale=0.7)
    else:
        y64 = lo.lora_linear(d["x"], d["W"], d["b"], None, None, d["alpha"], rank, 0.9, 0.7)
        yc = None
    assert_gate(y, y64, yc, what="many tiles")


def test_many_tiles_unaligned_column_view():
    d = lw.small_linear_inputs(2600, 192, 6000, 64, 47, bias=True, alpha=64.0)
    say("case many tiles, unaligned column view")
    x, W, b, A, B = (dev(d[k]) for k in ("x", "W", "b", "A", "B"))
    wide = torch.full((2600, 6011), 5.0, dtype=torch.bfloat16, device=DEV)
    view = wide[:, 3:6003]
    rg.lora_linear(x, W, b, A, B, 64.0, out=view)
    ref = rg.lora_linear(x, W, b, A, B, 64.0)
    torch.cuda.synchronize()
    assert torch.equal(view, ref)
    assert bool((wide[:, :3] == 5.0).all()) and bool((wide[:, 6003:] == 5.0).all())


# ------------------------------------------------------------------ goldens through the exact tier

def _hex(v):
    return float.fromhex(v) if isinstance(v, str) else float(v)


def test_handworked_goldens_exact_tier():
    cases = json.load(open(GOLDEN))["linear"]
    for c in cases:
        act, adt = c["act"], c["adapter"]
        say(f"case golden {c['name']}")
        mat = lambda rows, dt: None if rows is None else lw.to_dtype(
            np.array([[_hex(v) for v in r] for r in rows]), dt)
        x, W, A, B = mat(c["x"], act), mat(c["W"], act), mat(c["A"], adt), mat(c["B"], adt)
        b = None if c["b"] is None else lw.to_dtype(np.array([_hex(v) for v in c["b"]]), act)
        y = rg.lora_linear(dev(x), dev(W), dev(b), dev(A), dev(B), c["alpha"], c["strength"],
                           _hex(c["request_scale"]), quality="exact")
        torch.cuda.synchronize()
        want = np.array([[_hex(v) for v in r] for r in c["expected"]])
        assert_bitwise(y, want, c["name"])


# ------------------------------------------------------------------ fp32 adapter on bf16 activations

# ------------------------------------------------------------------ the hot GEMM's two output tiles
# 256 x 256 (one workgroup per CU) and 128 x 128 (two per CU, chosen when the large tiles would
# leave compute units idle) accumulate every output in the same order: same bits.

@pytest.mark.parametrize("case", ["ragged_bias", "tail_row", "two_ext_stages", "four_ext_stages", "no_adapter",
                                  "f32_adapter", "nf4_sized", "many_tiles"])
def test_gemm_tiles_bitwise_equal(case):
    """The tile is a per-call argument (lora_linear_fwd_phase, phase 0): 256 x 256 against 128 x 128."""
    say(f"case gemm tiles {case}")
    shapes = {"ragged_bias": (300, 200, 520, 24, True), "tail_row": (513, 384, 768, 64, False),
              "two_ext_stages": (257, 1536, 300, 128, True), "four_ext_stages": (300, 256, 700, 200, True),
              "no_adapter": (300, 200, 520, 24, True), "f32_adapter": (300, 200, 520, 24, True),
              "nf4_sized": (130, 4096, 600, 16, False), "many_tiles": (2600, 512, 6000, 96, False)}
    T, K, N, r, bias = shapes[case]
    d = lw.small_linear_inputs(T, K, N, r, 61, adapter="f32" if case == "f32_adapter" else "bf16", bias=bias,
                               alpha=2.0 * r, strength=0.8, request_scale=0.7)
    A, B = (None, None) if case == "no_adapter" else (dev(d["A"]), dev(d["B"]))
    outs = []
    for tile in (1, 2):
        outs.append(rg.lora_linear(dev(d["x"]), dev(d["W"]), dev(d["b"]), A, B, d["alpha"], d["strength"],
                                   d["request_scale"], gemm_tile=tile))
        torch.cuda.synchronize()
    y256, y128 = outs
    assert torch.equal(y256, y128), f"{case}: {(y256 != y128).sum().item()} outputs differ"
    if case != "no_adapter":
        assert torch.equal(y256, run_linear(d, "lossless")), f"{case}: the automatic choice differs"


@pytest.mark.parametrize("T,K,S", [(129, 512, 2), (129, 768, 3), (129, 1024, 4), (6529, 2048, 5), (5377, 2048, 6),
                                   (4609, 2048, 7), (129, 2048, 8)])
def test_producer_k_split_counts(T, K, S):
    """Fewer than 128 tiles of 128 tokens: the rank-wide producer splits K into S parts (chosen by T
    and K alone) whose partial sums a finishing kernel adds, one kernel instance per S. Each S from
    2 to 8 against the oracle."""
    N, r = 96, 16
    d = lw.small_linear_inputs(T, K, N, r, 500 + S, bias=True, alpha=2.0 * r, strength=0.8, request_scale=0.7)
    say(f"case producer split S={S} T={T} K={K}")
    y64, yc = oracle_pair(d)
    assert_gate(run_linear(d, "lossless"), y64, yc, what=f"lossless, producer split {S}")


@pytest.mark.parametrize("T,K,N,r", [(300, 200, 520, 24), (257, 512, 300, 64)])
def test_fp32_adapter_on_bf16(T, K, N, r):
    d = lw.small_linear_inputs(T, K, N, r, 21, adapter="f32", bias=True, alpha=2.0 * r, strength=0.8,
                               request_scale=0.7)
    say(f"case fp32 adapter T={T} K={K} N={N} r={r}")
    y64, yc = oracle_pair(d, "bf16", "f32")
    assert_gate(run_linear(d, "lossless"), y64, yc, what="lossless f32-adapter")
    assert_bitwise(run_linear(d, "exact"), yc, "exact f32-adapter")


# ------------------------------------------------------------------ few tokens (T <= 64)
# The weight read is the whole cost: K is split into chunks whose fp32 partial
# sums a second kernel adds. Ragged K (not a multiple of 64), ragged N, ranks
# that are not multiples of 8, tokens from 1 to 64.

@pytest.mark.parametrize("T,K,N,r,bias", [(1, 328, 300, 16, True), (7, 1536, 300, 70, False),
                                          (16, 328, 1000, 8, True), (33, 64, 96, 128, True),
                                          (64, 2056, 520, 24, False),
                                          # the most K chunks: 32 of 512, and 32 of 640 with a ragged last
                                          (16, 16384, 300, 16, True), (5, 20000, 260, 24, False)])
def test_few_tokens_linear(T, K, N, r, bias):
    d = lw.small_linear_inputs(T, K, N, r, 60 + T, bias=bias, alpha=2.0 * r, strength=0.8, request_scale=0.7)
    say(f"case few tokens T={T} K={K} N={N} r={r} bias={bias}")
    y64, yc = oracle_pair(d)
    assert_gate(run_linear(d, "lossless"), y64, yc, what="few-token lossless")
    assert_bitwise(run_linear(d, "exact"), yc, "few-token exact")


@pytest.mark.parametrize("adapter", ["bf16", "f32"])
def test_few_tokens_rows_do_not_depend_on_the_batch(adapter):
    """Up to 8 tokens each wave loads its token fragments itself; from 9 on the workgroup shares
    them through LDS. Every token is computed on its own (K chunks fixed by K alone), so the
    rows of a 9-, 33- or 64-token call equal the same rows in 1-, 4- and 8-token calls bit for bit."""
    T, K, N, r = 64, 2056, 520, 24
    d = lw.small_linear_inputs(T, K, N, r, 91, adapter=adapter, bias=True, alpha=2.0 * r, strength=0.8,
                               request_scale=0.7)
    say(f"case few tokens rows vs batch adapter={adapter}")
    x, W, b, A, B = dev(d["x"]), dev(d["W"]), dev(d["b"]), dev(d["A"]), dev(d["B"])
    call = lambda xs: rg.lora_linear(xs, W, b, A, B, d["alpha"], 0.8, 0.7)
    big = {t: call(x[:t]) for t in (9, 33, 64)}
    small = {t: call(x[:t]) for t in (1, 4, 8)}
    torch.cuda.synchronize()
    for tb, yb in big.items():
        for ts, ys in small.items():
            assert torch.equal(yb[:ts], ys), (tb, ts)


@pytest.mark.parametrize("T,K,N,r", [(40, 256, 520, 24), (3, 512, 300, 64), (9, 16384, 260, 16)])
def test_few_tokens_fp32_adapter(T, K, N, r):
    d = lw.small_linear_inputs(T, K, N, r, 70 + T, adapter="f32", bias=True, alpha=2.0 * r, strength=0.8,
                               request_scale=0.7)
    say(f"case few tokens fp32 adapter T={T} K={K} N={N} r={r}")
    y64, yc = oracle_pair(d, "bf16", "f32")
    assert_gate(run_linear(d, "lossless"), y64, yc, what="few-token lossless f32-adapter")


@pytest.mark.parametrize("T,K,N,r", [(300, 200, 520, 24), (129, 264, 300, 64), (513, 64, 1000, 128)])
def test_fp32_layer_multi_tile(T, K, N, r):
    """fp32 activations and adapter over several ragged output tiles (the tiny fp32 layer is one
    tile): fp32 output within 1e-6 relative RMS of fp64 (fp32 accumulation over K <= 264 terms
    stays under it), exact tier bit for bit with the chain."""
    d = lw.small_linear_inputs(T, K, N, r, 31 + r, act="f32", adapter="f32", bias=True, alpha=2.0 * r,
                               strength=0.8, request_scale=0.7)
    say(f"case fp32 layer T={T} K={K} N={N} r={r}")
    y64, yc = oracle_pair(d, "f32", "f32")
    y = run_linear(d, "lossless")
    e = lo.rel_rms(host64(y), y64)
    say(f"  lossless rel_rms {e:.3e}")
    assert y.dtype == torch.float32 and e <= LOSSLESS_F32_GATE
    ye = run_linear(d, "exact")
    assert_bitwise(ye, yc, "fp32 layer exact")


@pytest.mark.parametrize("T,K,N,r", [(300, 200, 520, 24), (20, 512, 300, 64), (300, 2048, 520, 32)])
def test_strided_input_rows_equal_contiguous(T, K, N, r):
    """x as a column view of a wider tensor (row stride ldx > K, 16-byte aligned start): the same
    bits as the contiguous input, in both tiers (hot kernel; few-token path; producer K split)."""
    d = lw.small_linear_inputs(T, K, N, r, 51 + r, bias=True, alpha=2.0 * r, strength=0.8, request_scale=0.7)
    say(f"case strided x T={T} K={K} N={N} r={r}")
    x = dev(d["x"])
    wide = torch.full((T, K + 40), float("nan"), dtype=torch.bfloat16, device=DEV)
    wide[:, 16:16 + K] = x
    xv = wide[:, 16:16 + K]
    assert xv.stride(0) == K + 40 and xv.data_ptr() % 16 == 0
    W, b, A, B = dev(d["W"]), dev(d["b"]), dev(d["A"]), dev(d["B"])
    for q in ("lossless", "exact"):
        want = rg.lora_linear(x, W, b, A, B, d["alpha"], 0.8, 0.7, quality=q)
        got = rg.lora_linear(xv, W, b, A, B, d["alpha"], 0.8, 0.7, quality=q)
        torch.cuda.synchronize()
        assert torch.equal(got, want), q


# ------------------------------------------------------------------ stacked groups

def _stacked_inputs(seed, adapter="bf16", bias=True, T=300):
    rng = np.random.default_rng(seed)
    K, Nt = 256, 700
    specs = [(24, 48.0, 0, 200), (16, 8.0, 248, 300), (64, 64.0, 560, 140)]  # rank, alpha, offset, n_cols
    x = lw.to_dtype(rng.standard_normal((T, K)), "bf16")
    W = lw.to_dtype(rng.standard_normal((Nt, K)) / np.sqrt(K), "bf16")
    b = lw.to_dtype(rng.standard_normal(Nt) * np.sqrt(0.02), "bf16") if bias else None
    groups = [dict(A=lw.to_dtype(rng.standard_normal((r, K)) / np.sqrt(K), adapter),
                   B=lw.to_dtype(rng.standard_normal((n, r)) * np.sqrt(0.02), adapter),
                   rank=r, alpha=a, col_offset=o, n_cols=n) for r, a, o, n in specs]
    return x, W, b, groups


@pytest.mark.parametrize("T", [300, 20])
@pytest.mark.parametrize("adapter", ["bf16", "f32"])
def test_stacked_groups(adapter, T):
    x, W, b, groups = _stacked_inputs(31, adapter, T=T)
    say(f"case stacked adapter={adapter} T={T}")
    y64 = lo.lora_linear_stacked(x, W, b, groups, 0.9, 0.8)
    yc = ec.chain_stacked(x, W, b, groups, 0.9, 0.8, "bf16", adapter)
    gg = [dict(g, A=dev(g["A"]), B=dev(g["B"])) for g in groups]
    y = rg.lora_linear_stacked(dev(x), dev(W), dev(b), gg, 0.9, 0.8)
    torch.cuda.synchronize()
    assert_gate(y, y64, yc, what="stacked lossless")
    ye = rg.lora_linear_stacked(dev(x), dev(W), dev(b), gg, 0.9, 0.8, quality="exact")
    torch.cuda.synchronize()
    assert_bitwise(ye, yc, "stacked exact")
    # stacked == one call per group into column views of the same output
    for q, ys in (("lossless", y), ("exact", ye)):
        sep = rg.lora_linear(dev(x), dev(W), dev(b), None, None, 1.0, quality=q)
        for g in gg:
            o, n = g["col_offset"], g["n_cols"]
            rg.lora_linear(dev(x), dev(W)[o:o + n], dev(b)[o:o + n], g["A"], g["B"], g["alpha"], 0.9, 0.8,
                           out=sep[:, o:o + n], quality=q)
        torch.cuda.synchronize()
        assert torch.equal(sep, ys), q


# ------------------------------------------------------------------ 4-bit base weight

def _nf4_small(T=130, K=256, N=300, r=16, seed=41, bias=True, adapter="bf16"):
    rng = np.random.default_rng(seed)
    x = lw.to_dtype(rng.standard_normal((T, K)), "bf16")
    codes = torch.from_numpy(rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8))
    absmax = torch.from_numpy(np.abs(rng.standard_normal(N * K // 64)) * np.sqrt(0.05)).float()
    A = lw.to_dtype(rng.standard_normal((r, K)) / np.sqrt(K), adapter)
    B = lw.to_dtype(rng.standard_normal((N, r)) * np.sqrt(0.02), adapter)
    b = lw.to_dtype(rng.standard_normal(N) * np.sqrt(0.02), "bf16") if bias else None
    return dict(x=x, codes=codes, absmax=absmax, codebook=lw.nf4_style_codebook(), A=A, B=B, b=b, rank=r,
                alpha=32.0, N=N)


# T <= 64: the few-token kernel dequantizes weight fragments in registers;
# T = 130 and 600: the weight is dequantized once into a bf16 panel in the
# workspace, then the bf16 GEMM runs over it (ragged tails).
@pytest.mark.parametrize("T", [1, 64, 130, 600])
@pytest.mark.parametrize("adapter", ["bf16", "f32"])
def test_nf4_linear(adapter, T):
    d = _nf4_small(T=T, adapter=adapter)
    say(f"case nf4 adapter={adapter} T={T}")
    y64 = lo.lora_linear_nf4(d["x"], d["codes"], d["absmax"], d["codebook"], 64, d["b"], d["A"], d["B"],
                             d["alpha"], d["rank"], 1.0, 0.9)
    yc = ec.chain_nf4(d["x"], d["codes"], d["absmax"], d["codebook"], 64, d["b"], d["A"], d["B"], d["alpha"],
                      d["rank"], 1.0, 0.9) if adapter == "bf16" else None
    args = (dev(d["x"]), dev(d["codes"]), dev(d["absmax"]), dev(d["codebook"]), d["N"], dev(d["b"]),
            dev(d["A"]), dev(d["B"]), d["alpha"], 1.0, 0.9)
    y = rg.lora_linear_nf4(*args)
    torch.cuda.synchronize()
    if adapter == "f32":
        W = ec.chain_nf4_weight(d["codes"], d["absmax"], d["codebook"], 256)
        yc = ec.chain_linear(d["x"], W, d["b"], d["A"], d["B"], d["alpha"], d["rank"], 1.0, 0.9, "bf16", "f32")
    assert_gate(y, y64, yc, what="nf4 lossless")
    ye = rg.lora_linear_nf4(*args, quality="exact")
    torch.cuda.synchronize()
    assert_bitwise(ye, yc, "nf4 exact")


@pytest.mark.parametrize("T", [64, 256])
def test_nf4_one_hot_returns_dequantized_columns(T):
    d = _nf4_small(T=T, K=256, N=300, bias=False)
    say(f"case nf4 one-hot T={T}")
    x = torch.zeros((T, 256), dtype=torch.bfloat16)
    x[torch.arange(T), torch.arange(T) % 256] = 1.0  # row m selects k = m mod 256
    Wq = ec.chain_nf4_weight(d["codes"], d["absmax"], d["codebook"], 256)  # [N, K]
    want = Wq.T[np.arange(T) % 256].copy()
    for q in ("lossless", "exact"):
        y = rg.lora_linear_nf4(dev(x), dev(d["codes"]), dev(d["absmax"]), dev(d["codebook"]), 300, None, None,
                               None, 32.0, quality=q)
        torch.cuda.synchronize()
        assert_bitwise(y, want, f"one-hot {q}")


# The 4-bit weight dequantized inside the hot GEMM (128-token tiles) against the panel path: the
# same weight bits (one table of RN_bf16(RN_f32(codebook[c] . absmax)) per 64-element block, built
# with the panel kernel's arithmetic) and the same accumulation order, so the same output bits.
# The cases walk the kernel's stage plans: no adapter; one K-extension stage (rank <= 64); two
# (<= 128); four (rank 200: the codes of the first main stage are loaded by the prologue ahead of
# the extension stages); K of one and of two 64-element stages; ragged tiles both ways; a strided
# input and a column view of a wider output; with and without bias.
# The last two shapes have enough output tiles that the 256 x 256 tile is chosen on MI355X's 256
# compute units (one row of weight per thread, eight code words per stage); the others take the
# 128 x 128 tile.
@pytest.mark.parametrize("T,K,N,r,bias", [
    (65, 256, 300, 16, True), (130, 256, 300, 0, False), (300, 64, 260, 8, True), (257, 128, 520, 128, True),
    (600, 448, 1000, 200, False), (1000, 1024, 700, 64, True), (1790, 128, 9100, 200, True),
    (1000, 64, 16384, 16, False)])
def test_nf4_in_gemm_equals_panel(T, K, N, r, bias):
    d = _nf4_small(T=T, K=K, N=N, r=max(r, 8), bias=bias, seed=60 + T)
    say(f"case nf4 in-GEMM vs panel T={T} K={K} N={N} r={r} bias={bias}")
    A, B = (dev(d["A"]), dev(d["B"])) if r else (None, None)
    xs = torch.zeros((T, K + 64), dtype=torch.bfloat16)
    xs[:, :K] = d["x"]
    xv = dev(xs)[:, :K]  # row stride K + 64
    args = (xv, dev(d["codes"]), dev(d["absmax"]), dev(d["codebook"]), N, dev(d["b"]), A, B, d["alpha"], 0.8, 0.9)
    outs = {}
    for mode in ("panel", "in_gemm"):
        wide = torch.full((T, N + 40), float("nan"), dtype=torch.bfloat16, device=DEV)
        outs[mode] = wide
        rg.lora_linear_nf4(*args, out=wide[:, 24:24 + N], dequant=mode)
    torch.cuda.synchronize()
    y = outs["in_gemm"][:, 24:24 + N]
    assert torch.equal(outs["panel"][:, 24:24 + N], y), "in-GEMM dequantization differs from the panel"
    assert torch.isnan(outs["in_gemm"][:, :24]).all(), "wrote left of the column view"
    assert torch.isnan(outs["in_gemm"][:, 24 + N:]).all(), "wrote right of the column view"
    y64 = lo.lora_linear_nf4(d["x"], d["codes"], d["absmax"], d["codebook"], 64, d["b"],
                             d["A"] if r else None, d["B"] if r else None, d["alpha"], max(r, 8), 0.8, 0.9)
    yc = None  # (without an adapter the chain is the base GEMM summed exactly: only the gate applies)
    if r and T * K * N <= 300 * 256 * 520:
        yc = ec.chain_nf4(d["x"], d["codes"], d["absmax"], d["codebook"], 64, d["b"], d["A"] if r else None,
                          d["B"] if r else None, d["alpha"], max(r, 8), 0.8, 0.9)
    assert_gate(y, y64, yc, what="nf4 in-GEMM lossless")


def test_nf4_in_gemm_workspace_and_choice():
    """The in-GEMM form needs no panel in the workspace (the panel path refuses that size), and an
    fp32 adapter or a rank that is not a multiple of 8 is refused for it."""
    d = _nf4_small(T=300, K=256, N=300, r=16, bias=False, seed=9)
    say("case nf4 in-GEMM workspace")
    x, codes, am, cb = dev(d["x"]), dev(d["codes"]), dev(d["absmax"]), dev(d["codebook"])
    A, B = dev(d["A"]), dev(d["B"])
    small = rg.lora_linear_workspace_size(300, 256, 300, [16], rg.LORA_BF16)
    assert small < rg.lora_linear_nf4_workspace_size(300, 256, 300, 16, rg.LORA_BF16)
    ws = torch.empty(small, dtype=torch.uint8, device=DEV)
    yp = rg.lora_linear_nf4(x, codes, am, cb, 300, None, A, B, 32.0, dequant="panel")
    yg = rg.lora_linear_nf4(x, codes, am, cb, 300, None, A, B, 32.0, dequant="in_gemm", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(yp, yg)
    WORKSPACE, UNSUPPORTED = 7, 8
    with pytest.raises(rg.LoraError) as e:
        rg.lora_linear_nf4(x, codes, am, cb, 300, None, A, B, 32.0, dequant="panel", workspace=ws)
    assert e.value.status == WORKSPACE
    with pytest.raises(rg.LoraError) as e:
        rg.lora_linear_nf4(x, codes, am, cb, 300, None, A.float(), B.float(), 32.0, dequant="in_gemm")
    assert e.value.status == UNSUPPORTED
    with pytest.raises(rg.LoraError) as e:
        rg.lora_linear_nf4(x, codes, am, cb, 300, None, A[:12].contiguous(), B[:, :12].contiguous(), 32.0,
                           dequant="in_gemm")
    assert e.value.status == UNSUPPORTED


# ------------------------------------------------------------------ dense patches

@pytest.mark.parametrize("shape,dt_dst,dt_src,mode", [
    ((1031, 77), "bf16", "bf16", "add"), ((3072 + 5,), "bf16", "bf16", "add"), ((513, 64), "f32", "bf16", "add"),
    ((300, 40), "bf16", "f32", "add"), ((333,), "f32", "f32", "replace"), ((1031, 77), "bf16", "bf16", "replace"),
])
def test_dense_patch(shape, dt_dst, dt_src, mode):
    rng = np.random.default_rng(51)
    n = int(np.prod(shape))
    dst = lw.to_dtype(rng.standard_normal(n) * 0.02, dt_dst).reshape(shape)
    src = lw.to_dtype(rng.standard_normal(n) * 2e-5, dt_src).reshape(shape)
    say(f"case dense patch {shape} {dt_dst}<-{dt_src} {mode}")
    want = ec.chain_dense_patch(dst, src, 0.8, mode, dt_dst)
    g = dev(dst)
    rg.dense_patch(g, dev(src), 0.8, mode)
    torch.cuda.synchronize()
    assert_bitwise(g, want.reshape(shape), "patch")


def test_dense_patch_unaligned_and_goldens():
    rng = np.random.default_rng(52)
    base = lw.to_dtype(rng.standard_normal(1001) * 0.02, "bf16")
    diff = lw.to_dtype(rng.standard_normal(1001) * 2e-5, "bf16")
    say("case dense patch unaligned")
    g = dev(base)
    gs = dev(diff)
    rg.dense_patch(g[1:], gs[:1000], 0.8)  # dst starts 2 bytes into its allocation
    torch.cuda.synchronize()
    want = ec.chain_dense_patch(base[1:], diff[:1000], 0.8, "add", "bf16")
    assert_bitwise(g[1:], want, "unaligned patch")
    for c in json.load(open(GOLDEN))["patch"]:
        say(f"case golden {c['name']}")
        dst = lw.to_dtype(np.array([_hex(c["dst"])] * 19), c["dtype"])
        src = lw.to_dtype(np.array([_hex(c["src"])] * 19), "bf16")
        gd = dev(dst)
        rg.dense_patch(gd, dev(src), _hex(c["strength"]), c["mode"])
        torch.cuda.synchronize()
        assert bool((host64(gd) == _hex(c["expected"])).all()), c["name"]


# ------------------------------------------------------------------ several adapters on one layer

def _multi_inputs(seed, T, adapter="bf16", n_ads=3, K=256, N=520):
    rng = np.random.default_rng(seed)
    x = lw.to_dtype(rng.standard_normal((T, K)), "bf16")
    W = lw.to_dtype(rng.standard_normal((N, K)) / np.sqrt(K), "bf16")
    b = lw.to_dtype(rng.standard_normal(N) * np.sqrt(0.02), "bf16")
    # rank, alpha, strength, column range, legacy lora_B bias: overlapping ranges, ragged edges
    specs = [(16, 32.0, 1.0, 0, N, True), (24, 24.0, 0.6, 130, 300, False), (64, 16.0, -0.8, 200, 320, True),
             (8, 8.0, 0.9, 0, 257, True)][:n_ads]
    ads = [dict(A=lw.to_dtype(rng.standard_normal((r, K)) / np.sqrt(K), adapter),
                B=lw.to_dtype(rng.standard_normal((n, r)) * np.sqrt(0.02), adapter),
                c=lw.to_dtype(rng.standard_normal(n) * np.sqrt(0.02), adapter) if has_c else None,
                rank=r, alpha=a, strength=st, col_offset=o, n_cols=n) for r, a, st, o, n, has_c in specs]
    return x, W, b, ads


@pytest.mark.parametrize("T,adapter,n_ads", [(300, "bf16", 2), (300, "bf16", 3), (300, "f32", 3), (20, "bf16", 4),
                                             (20, "f32", 2)])
def test_multi_adapters(T, adapter, n_ads):
    """Overlapping adapters with their own strengths and legacy lora_B biases (2 per tile: the hot
    kernel; 3: the general pipelined kernel; 20 tokens: the few-token path)."""
    x, W, b, ads = _multi_inputs(81 + n_ads, T, adapter, n_ads)
    say(f"case multi T={T} adapter={adapter} n={n_ads}")
    y64 = lo.lora_linear_multi(x, W, b, ads, 0.7)
    yc = ec.chain_multi(x, W, b, ads, 0.7, "bf16", adapter)
    gg = [dict(a, A=dev(a["A"]), B=dev(a["B"]), c=dev(a["c"])) for a in ads]
    y = rg.lora_linear_multi(dev(x), dev(W), dev(b), gg, 0.7)
    torch.cuda.synchronize()
    assert_gate(y, y64, yc, what="multi lossless")
    ye = rg.lora_linear_multi(dev(x), dev(W), dev(b), gg, 0.7, quality="exact")
    torch.cuda.synchronize()
    assert_bitwise(ye, yc, "multi exact")


@pytest.mark.parametrize("T", [300, 20])
def test_multi_disjoint_equals_stacked(T):
    """Disjoint adapters, one strength, no legacy bias: the multi call is the stacked call, bit for bit."""
    x, W, b, groups = _stacked_inputs(33, "bf16", T=T)
    gg = [dict(g, A=dev(g["A"]), B=dev(g["B"])) for g in groups]
    say(f"case multi == stacked T={T}")
    for q in ("lossless", "exact"):
        ys = rg.lora_linear_stacked(dev(x), dev(W), dev(b), gg, 0.9, 0.8, quality=q)
        ym = rg.lora_linear_multi(dev(x), dev(W), dev(b), [dict(g, c=None, strength=0.9) for g in gg], 0.8,
                                  quality=q)
        torch.cuda.synchronize()
        assert torch.equal(ys, ym), q


# ------------------------------------------------------------------ merge W <- W + s.B.A

def _ulp_bf16(v):
    """Spacing of bf16 values at |v| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("N,K,r,wdt,adt", [(300, 520, 64, "bf16", "bf16"), (257, 1000, 100, "bf16", "bf16"),
                                           (130, 264, 5, "bf16", "bf16"), (300, 520, 24, "f32", "bf16"),
                                           (300, 520, 24, "bf16", "f32"), (64, 136, 8, "f32", "f32")])
def test_merge(N, K, r, wdt, adt):
    rng = np.random.default_rng(90 + r)
    W = lw.to_dtype(rng.standard_normal((N, K)) / np.sqrt(K), wdt)
    A = lw.to_dtype(rng.standard_normal((r, K)) / np.sqrt(K), adt)
    B = lw.to_dtype(rng.standard_normal((N, r)) * np.sqrt(0.02), adt)
    alpha, strength = 2.0 * r, 0.7
    say(f"case merge N={N} K={K} r={r} w={wdt} adapter={adt}")
    W64 = lo.merged_weight(W, A, B, lo.combined_scale(alpha, r, strength, 1.0))
    g = dev(W)
    rg.lora_merge(g, dev(A), dev(B), alpha, strength)
    torch.cuda.synchronize()
    got = host64(g)
    if wdt == "bf16":
        # one rounding of the fp32 sum: the correctly rounded merge, except where the fp32 sum sits
        # within its own rounding of a bf16 tie (then one bf16 spacing away)
        want = ec.rn(ec.rn_f32(W64), "bf16")  # (through fp32: a double-rounding tie is within the allowance)
        diff = np.abs(got - want)
        # the fp32 sum of r products and the fp32 add err by at most r 2^-23 |s| (|B| |A|) + 2^-23 |W'|
        # (standard summation bound), which can cross one bf16 rounding boundary
        sc = lo.combined_scale(alpha, r, strength, 1.0)
        fp32_err = r * 2.0 ** -23 * abs(sc) * (np.abs(lo.f64(B)) @ np.abs(lo.f64(A))) + 2.0 ** -23 * np.abs(W64)
        assert (diff <= _ulp_bf16(want) * 1.0001 + 2 * fp32_err).all()
        assert (diff > 0).mean() < 1e-3
    else:
        assert lo.rel_rms(got, W64) <= 1e-6
    ge = dev(W)
    rg.lora_merge(ge, dev(A), dev(B), alpha, strength, quality="exact")
    torch.cuda.synchronize()
    assert_bitwise(ge, ec.chain_merge(W, A, B, alpha, r, strength, wdt), "merge exact")


def test_merge_zero_strength_and_merged_layer():
    d = lw.small_linear_inputs(300, 256, 520, 32, 95, bias=True, alpha=32.0, strength=0.8, request_scale=1.0)
    say("case merge: zero strength, merged layer vs dynamic layer")
    g = dev(d["W"])
    rg.lora_merge(g, dev(d["A"]), dev(d["B"]), 32.0, 0.0)
    rg.lora_merge(g, dev(d["A"]), dev(d["B"]), 32.0, -0.0, quality="exact")
    torch.cuda.synchronize()
    assert torch.equal(g, dev(d["W"]))
    # the layer over the merged bf16 weight loses what the merge rounded away; the fused dynamic
    # layer keeps it (its error is no larger than the merged layer's against fp64)
    rg.lora_merge(g, dev(d["A"]), dev(d["B"]), 32.0, 0.8)
    y_merged = rg.lora_linear(dev(d["x"]), g, dev(d["b"]), None, None, 1.0)
    y_dyn = rg.lora_linear(dev(d["x"]), dev(d["W"]), dev(d["b"]), dev(d["A"]), dev(d["B"]), 32.0, 0.8, 1.0)
    torch.cuda.synchronize()
    y64 = lo.lora_linear(d["x"], d["W"], d["b"], d["A"], d["B"], 32.0, 32, 0.8, 1.0)
    e_m, e_d = lo.rel_rms(host64(y_merged), y64), lo.rel_rms(host64(y_dyn), y64)
    say(f"  merged-weight layer rel_rms {e_m:.3e}, dynamic {e_d:.3e}")
    assert e_d <= e_m and e_m <= 4e-3


# ------------------------------------------------------------------ backward

@pytest.mark.parametrize("T,K,N,r", [(300, 256, 520, 24), (513, 384, 768, 64), (100, 136, 96, 5), (40, 64, 1000, 128),
                                     (700, 512, 392, 200)])
def test_backward(T, K, N, r):
    d = lw.small_linear_inputs(T, K, N, r, 100 + r, bias=False, alpha=2.0 * r, strength=0.8, request_scale=0.7)
    rng = np.random.default_rng(200 + r)
    dy = lw.to_dtype(rng.standard_normal((T, N)), "bf16")
    say(f"case backward T={T} K={K} N={N} r={r}")
    dx, dA, dB, db = rg.lora_linear_backward(dev(d["x"]), dev(d["W"]), dev(d["A"]), dev(d["B"]), dev(dy), d["alpha"],
                                             0.8, 0.7)
    torch.cuda.synchronize()
    o = lo.lora_linear_backward(d["x"], d["W"], d["A"], d["B"], dy, d["alpha"], r, 0.8, 0.7)
    for name, got, want, gate in (("dx", dx, o[0], 4e-3), ("dA", dA, o[1], 4e-3), ("dB", dB, o[2], 4e-3),
                                  ("db", db, o[3], 1e-5)):
        e = lo.rel_rms(host64(got), want)
        say(f"  {name} rel_rms {e:.3e}")
        assert e <= gate, (name, e)
    # dx is the forward layer of dy over W^T with the adapter (B^T, A^T), bit for bit
    Wt, Bt, At = dev(d["W"]).t().contiguous(), dev(d["B"]).t().contiguous(), dev(d["A"]).t().contiguous()
    y = rg.lora_linear(dev(dy), Wt, None, Bt, At, d["alpha"], 0.8, 0.7)
    torch.cuda.synchronize()
    assert torch.equal(y, dx)


@pytest.mark.parametrize("T,K,N,r", [(300, 256, 520, 24), (513, 384, 768, 64), (700, 512, 392, 200)])
def test_backward_with_the_forward_t_is_the_same_bits(T, K, N, r):
    """t~ handed over from the forward call's workspace gives the gradients the backward computes
    when it recomputes t~ itself, bit for bit."""
    d = lw.small_linear_inputs(T, K, N, r, 300 + r, bias=True, alpha=2.0 * r, strength=0.8, request_scale=0.7)
    rng = np.random.default_rng(400 + r)
    dy = dev(lw.to_dtype(rng.standard_normal((T, N)), "bf16"))
    x, W, A, B = dev(d["x"]), dev(d["W"]), dev(d["A"]), dev(d["B"])
    say(f"case backward with the forward t~ T={T} K={K} N={N} r={r}")
    rp = -(-r // 64) * 64
    ws = torch.empty(rg.lora_linear_workspace_size(T, K, N, [r], rg.LORA_BF16), dtype=torch.uint8, device=DEV)
    rg.lora_linear(x, W, dev(d["b"]), A, B, d["alpha"], 0.8, 0.7, workspace=ws)
    tt = ws[:T * rp * 2].view(torch.bfloat16).view(T, rp)
    got = rg.lora_linear_backward(x, W, A, B, dy, d["alpha"], 0.8, 0.7, t_tilde=tt)
    want = rg.lora_linear_backward(x, W, A, B, dy, d["alpha"], 0.8, 0.7)
    # the same t~ at a row stride of rp + 3 elements from a start that is only 2-byte aligned
    # (its transposed copy then takes the element-wise transpose instead of 16-byte pieces)
    wide = torch.full((T, rp + 4), float("nan"), dtype=torch.bfloat16, device=DEV)
    odd = wide.view(-1)[1:1 + (T - 1) * (rp + 3) + rp].as_strided((T, rp), (rp + 3, 1))
    odd.copy_(tt)
    assert odd.stride(0) == rp + 3 and odd.data_ptr() % 16 != 0
    got_odd = rg.lora_linear_backward(x, W, A, B, dy, d["alpha"], 0.8, 0.7, t_tilde=odd)
    torch.cuda.synchronize()
    for name, g, g2, w in zip(("dx", "dA", "dB", "db"), got, got_odd, want):
        assert torch.equal(g, w), name
        assert torch.equal(g2, w), name + " (t~ at an odd stride)"


def test_backward_partial_outputs_and_empty_batch():
    d = lw.small_linear_inputs(300, 256, 520, 24, 150, bias=False, alpha=48.0)
    rng = np.random.default_rng(151)
    dy = dev(lw.to_dtype(rng.standard_normal((300, 520)), "bf16"))
    say("case backward partial outputs")
    full = rg.lora_linear_backward(dev(d["x"]), dev(d["W"]), dev(d["A"]), dev(d["B"]), dy, 48.0)
    only_db = rg.lora_linear_backward(dev(d["x"]), dev(d["W"]), dev(d["A"]), dev(d["B"]), dy, 48.0, want=("db",))
    only_dA = rg.lora_linear_backward(dev(d["x"]), dev(d["W"]), dev(d["A"]), dev(d["B"]), dy, 48.0, want=("dA",))
    torch.cuda.synchronize()
    assert torch.equal(full[3], only_db[3]) and torch.equal(full[1], only_dA[1])
    assert only_db[0] is None and only_db[1] is None and only_db[2] is None
    e = rg.lora_linear_backward(dev(d["x"])[:0], dev(d["W"]), dev(d["A"]), dev(d["B"]), dy[:0], 48.0)
    torch.cuda.synchronize()
    assert e[0].numel() == 0 and not e[1].any() and not e[2].any() and not e[3].any()
