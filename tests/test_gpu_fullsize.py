"""GPU parity at the workloads' full sizes, in the launch configuration bench.py
uses (same entry points, lossless default).

Every output buffer starts as NaN, so "no NaN afterwards" proves that every
element was written (a tile the grid mapping skipped would stay NaN).

Lossless: relative RMS <= 4e-3 against the fp64 plain definition over the
WHOLE output (numpy float64 BLAS on the host), and, on at least 256 rows (the
first rows, every row of the ragged last 256-token tile, random rows), no
larger than the separate-pass chain's error on the same rows. Exact tier:
bit-identical to the chain on those rows. Dense patches: bit-identical over the
whole tensor.
"""
import numpy as np
import pytest
import torch

import lora_workloads as lw
import rank_gemm_lora_amd as rg
from oracle import exact_chain as ec
from oracle import lora_oracle as lo
from tests.gpu_util import assert_bitwise, assert_gate, dev, host64, nan_out, sample_rows, say
from tests.oracle_pool import rows_parallel

pytestmark = pytest.mark.gpu


def _check(name, y, ye, y64, rows, chain, what_rows):
    """y, ye: GPU outputs (lossless, exact); y64: fp64 plain definition of every output; chain: the
    chain's values on ``rows``."""
    assert not bool(torch.isnan(y).any()), f"{name}: lossless output not completely written"
    assert not bool(torch.isnan(ye).any()), f"{name}: exact-tier output not completely written"
    T, N = y64.shape
    assert_gate(y, y64, None, what=f"{name} lossless, all {T} x {N} outputs")
    idx = torch.from_numpy(rows).to(y.device)
    assert_gate(y[idx], y64[rows], chain, what=f"{name} lossless vs chain, {what_rows}")
    assert_bitwise(ye[idx], chain, f"{name} exact, {what_rows}")


def _linear_case(d, name, act="bf16", adapter="bf16"):
    T, K = d["x"].shape
    N = d["W"].shape[0]
    rows = sample_rows(T, seed=1)
    say(f"case full-size {name}: T={T} K={K} N={N} r={d['rank']} sampled rows={len(rows)}")
    args = (dev(d["x"]), dev(d["W"]), dev(d["b"]), dev(d["A"]), dev(d["B"]), d["alpha"], d["strength"],
            d["request_scale"])
    y = rg.lora_linear(*args, out=nan_out(T, N))
    ye = rg.lora_linear(*args, quality="exact", out=nan_out(T, N))
    torch.cuda.synchronize()
    oargs = (d["W"], d["b"], d["A"], d["B"], d["alpha"], d["rank"], d["strength"], d["request_scale"])
    y64 = lo.lora_linear(d["x"], *oargs)
    yc = rows_parallel(ec.chain_linear, d["x"], rows, (*oargs, act, adapter))
    _check(name, y, ye, y64, rows, yc, f"{len(rows)} rows")


def test_attention_projection_full():
    _linear_case(lw.linear_inputs(lw.ATTN_PROJ), "attn_proj")


def test_ffn_pair_full():
    up, down = lw.ffn_pair_inputs()
    _linear_case(up, "ffn_up")
    _linear_case(down, "ffn_down")


@pytest.mark.parametrize("pair", ["zimage", "h3", "few"])
def test_other_token_regimes_full(pair):
    """Z-Image-Turbo (4352 tokens, rank 32), MiniMax-H3 per rank (18871, rank 64), 64 tokens."""
    up, down = {"zimage": (lw.ZIMAGE_FFN_UP, lw.ZIMAGE_FFN_DOWN), "h3": (lw.H3_FFN_UP, lw.H3_FFN_DOWN),
                "few": (lw.FEW_FFN_UP, lw.FEW_FFN_DOWN)}[pair]
    u, d = lw.ffn_pair_inputs(up, down)
    _linear_case(u, up.name)
    _linear_case(d, down.name)
    if pair == "zimage":
        _linear_case(lw.linear_inputs(lw.ZIMAGE_ATTN), lw.ZIMAGE_ATTN.name)


def test_multi_adapters_full():
    s = lw.MULTI_FFN_UP
    d = lw.multi_inputs(s)
    rows = sample_rows(s.T, seed=4)
    say(f"case full-size two adapters on FFN up T={s.T} sampled rows={len(rows)}")
    gg = [dict(a, A=dev(a["A"]), B=dev(a["B"]), c=dev(a["c"])) for a in d["adapters"]]
    y = rg.lora_linear_multi(dev(d["x"]), dev(d["W"]), dev(d["b"]), gg, s.request_scale, out=nan_out(s.T, s.N))
    ye = rg.lora_linear_multi(dev(d["x"]), dev(d["W"]), dev(d["b"]), gg, s.request_scale, quality="exact",
                              out=nan_out(s.T, s.N))
    torch.cuda.synchronize()
    y64 = lo.lora_linear_multi(d["x"], d["W"], d["b"], d["adapters"], s.request_scale)
    yc = rows_parallel(ec.chain_multi, d["x"], rows, (d["W"], d["b"], d["adapters"], s.request_scale))
    _check("multi", y, ye, y64, rows, yc, f"{len(rows)} rows")


@pytest.mark.parametrize("adapter", ["bf16", "f32"])
def test_qkv_stacked_full(adapter):
    spec = lw.QKV_STACKED if adapter == "bf16" else lw.StackedSpec(
        **{**lw.QKV_STACKED.__dict__, "name": "qkv_stacked_f32", "adapter": "f32"})
    d = lw.stacked_inputs(spec)
    T, N = spec.T, d["W"].shape[0]
    rows = sample_rows(T, seed=2)
    say(f"case full-size qkv stacked adapter={adapter} sampled rows={len(rows)}")
    gg = [dict(g, A=dev(g["A"]), B=dev(g["B"])) for g in d["groups"]]
    y = rg.lora_linear_stacked(dev(d["x"]), dev(d["W"]), dev(d["b"]), gg, d["strength"], d["request_scale"],
                               out=nan_out(T, N))
    ye = rg.lora_linear_stacked(dev(d["x"]), dev(d["W"]), dev(d["b"]), gg, d["strength"], d["request_scale"],
                                quality="exact", out=nan_out(T, N))
    torch.cuda.synchronize()
    y64 = lo.lora_linear_stacked(d["x"], d["W"], d["b"], d["groups"], d["strength"], d["request_scale"])
    yc = rows_parallel(ec.chain_stacked, d["x"], rows,
                       (d["W"], d["b"], d["groups"], d["strength"], d["request_scale"], "bf16", adapter))
    _check(f"stacked {adapter}", y, ye, y64, rows, yc, f"{len(rows)} rows")


@pytest.mark.parametrize("s", [lw.NF4_LAYER, lw.NF4_VECTOR], ids=["tokens8192", "single_vector"])
def test_nf4_layer_full(s):
    d = lw.nf4_inputs(s)
    rows = sample_rows(s.T, seed=3, min_rows=72)
    say(f"case full-size nf4 T={s.T} K={s.K} N={s.N} r={s.rank} sampled rows={len(rows)}")
    args = (dev(d["x"]), dev(d["codes"]), dev(d["absmax"]), dev(d["codebook"]), s.N, dev(d["b"]), dev(d["A"]),
            dev(d["B"]), d["alpha"], d["strength"], d["request_scale"])
    y = rg.lora_linear_nf4(*args, out=nan_out(s.T, s.N), dequant="panel")
    ye = rg.lora_linear_nf4(*args, quality="exact", out=nan_out(s.T, s.N))
    # the weight dequantized inside the GEMM instead: the same bits at full size
    yg = rg.lora_linear_nf4(*args, out=nan_out(s.T, s.N), dequant="in_gemm")
    torch.cuda.synchronize()
    assert torch.equal(y, yg), "4-bit weight dequantized in the GEMM differs from the panel path"
    del yg
    # fp64 over every output with the bf16 weight both tiers multiply (E6), and with the exact
    # codebook x absmax product
    W = ec.chain_nf4_weight(d["codes"], d["absmax"], d["codebook"], s.K, 64)
    oargs = (d["b"], d["A"], d["B"], d["alpha"], d["rank"], d["strength"], d["request_scale"])
    y64 = lo.lora_linear(d["x"], W, *oargs)
    y64_exact_w = lo.lora_linear_nf4(d["x"], d["codes"], d["absmax"], d["codebook"], 64, *oargs)
    yc = rows_parallel(ec.chain_linear, d["x"], rows, (W, *oargs))
    _check("nf4", y, ye, y64, rows, yc, f"{len(rows)} rows")
    assert_gate(y, y64_exact_w, None, what="nf4 lossless vs exact-weight fp64, all outputs")


@pytest.mark.parametrize("spec", [lw.PATCH_WEIGHT, lw.PATCH_NORM], ids=["weight_14336x4096", "rmsnorm_3072"])
def test_dense_patch_full(spec):
    d = lw.patch_inputs(spec)
    say(f"case full-size dense patch {spec.shape}")
    want = ec.chain_dense_patch(d["dst"], d["diff"], spec.strength, "add", "bf16")
    g = dev(d["dst"])
    rg.dense_patch(g, dev(d["diff"]), spec.strength, "add")
    torch.cuda.synchronize()
    assert_bitwise(g, want.reshape(spec.shape), "dense patch add")
    # the page's point: the delta survives because the sum is taken in fp32
    changed = float((host64(g) != lo.f64(d["dst"])).mean())
    say(f"  fraction of elements changed by the patch: {changed:.3f}")
    assert changed > 0.01
    want_r = ec.chain_dense_patch(d["dst"], d["diff"], spec.strength, "replace", "bf16")
    g2 = dev(d["dst"])
    rg.dense_patch(g2, dev(d["diff"]), spec.strength, "replace")
    torch.cuda.synchronize()
    assert_bitwise(g2, want_r.reshape(spec.shape), "dense patch replace")


@pytest.mark.parametrize("spec", [lw.MERGE_WEIGHT, lw.MERGE_WEIGHT_SMALL], ids=["variance", "small_update"])
def test_merge_full(spec):
    d = lw.merge_inputs(spec)
    rows = sample_rows(spec.N, seed=5)
    say(f"case full-size merge {spec.N}x{spec.K} r={spec.rank} rows={len(rows)}")
    g = dev(d["W"])
    rg.lora_merge(g, dev(d["A"]), dev(d["B"]), spec.alpha, spec.strength)
    ge = dev(d["W"])
    rg.lora_merge(ge, dev(d["A"]), dev(d["B"]), spec.alpha, spec.strength, quality="exact")
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).to(g.device)
    want = ec.chain_merge(d["W"][rows], d["A"], d["B"][rows], spec.alpha, spec.rank, spec.strength)
    assert_bitwise(ge[idx], want, "merge exact (sampled rows)")
    # lossless: the exact tier's value, or one bf16 spacing away where the fp32 sums round differently
    got, ref = host64(g[idx]), want
    assert (got != ref).mean() < 1e-3
    assert (np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7 + 2.0 ** -20).all()


def test_backward_ffn_up_full():
    """Backward of the 32760-token FFN up layer (r 64) against the fp64 oracle over every token."""
    up, _ = lw.ffn_pair_inputs()
    rng = np.random.default_rng(16)
    T, N = up["x"].shape[0], up["W"].shape[0]
    dy = lw.to_dtype(rng.standard_normal((T, N)), "bf16")
    say(f"case full-size backward FFN up T={T} N={N}")
    g = rg.lora_linear_backward(dev(up["x"]), dev(up["W"]), dev(up["A"]), dev(up["B"]), dev(dy), up["alpha"],
                                up["strength"], up["request_scale"])
    torch.cuda.synchronize()
    o = lo.lora_linear_backward(up["x"], up["W"], up["A"], up["B"], dy, up["alpha"], up["rank"], up["strength"],
                                up["request_scale"])
    for name, got, want, gate in (("dx", g[0], o[0], 4e-3), ("dA", g[1], o[1], 4e-3), ("dB", g[2], o[2], 4e-3),
                                  ("db", g[3], o[3], 1e-5)):
        e = lo.rel_rms(host64(got), want)
        say(f"  {name} rel_rms {e:.3e}")
        assert e <= gate, (name, e)
