"""GPU parity at the workloads' full sizes, in the launch configuration bench.py
uses (same entry points, lossless default), on rows the CPU oracle can afford:
the first rows, the rows of the ragged last 256-token tile and random rows in
between. Lossless: relative RMS <= 4e-3 against fp64 and no larger than the
separate-pass chain's error on the same rows. Exact tier: bit-identical to the
chain on the same rows. Dense patches: bit-identical over the whole tensor.
"""
import numpy as np
import pytest
import torch

import lora_workloads as lw
import rank_gemm_lora_amd as rg
from oracle import exact_chain as ec
from oracle import lora_oracle as lo
from tests.gpu_util import assert_bitwise, assert_gate, dev, host64, sample_rows, say

pytestmark = pytest.mark.gpu


def _linear_case(d, name, act="bf16", adapter="bf16"):
    T = d["x"].shape[0]
    rows = sample_rows(T, n_each=32, seed=1)
    say(f"case full-size {name}: T={T} K={d['x'].shape[1]} N={d['W'].shape[0]} r={d['rank']} rows={len(rows)}")
    args = (dev(d["x"]), dev(d["W"]), dev(d["b"]), dev(d["A"]), dev(d["B"]), d["alpha"], d["strength"],
            d["request_scale"])
    y = rg.lora_linear(*args)
    torch.cuda.synchronize()
    xs = d["x"][rows]
    oargs = (xs, d["W"], d["b"], d["A"], d["B"], d["alpha"], d["rank"], d["strength"], d["request_scale"])
    y64 = lo.lora_linear(*oargs)
    yc = ec.chain_linear(*oargs, act, adapter)
    assert_gate(y[torch.from_numpy(rows).to(y.device)], y64, yc, what=f"{name} lossless (sampled rows)")
    ye = rg.lora_linear(*args, quality="exact")
    torch.cuda.synchronize()
    assert_bitwise(ye[torch.from_numpy(rows).to(ye.device)], yc, f"{name} exact (sampled rows)")
    assert not bool(torch.isnan(y).any())


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
    rows = sample_rows(s.T, n_each=24, seed=4)
    say(f"case full-size two adapters on FFN up T={s.T} rows={len(rows)}")
    gg = [dict(a, A=dev(a["A"]), B=dev(a["B"]), c=dev(a["c"])) for a in d["adapters"]]
    y = rg.lora_linear_multi(dev(d["x"]), dev(d["W"]), dev(d["b"]), gg, s.request_scale)
    torch.cuda.synchronize()
    xs = d["x"][rows]
    y64 = lo.lora_linear_multi(xs, d["W"], d["b"], d["adapters"], s.request_scale)
    yc = ec.chain_multi(xs, d["W"], d["b"], d["adapters"], s.request_scale)
    idx = torch.from_numpy(rows).to(y.device)
    assert_gate(y[idx], y64, yc, what="multi lossless (sampled rows)")
    ye = rg.lora_linear_multi(dev(d["x"]), dev(d["W"]), dev(d["b"]), gg, s.request_scale, quality="exact")
    torch.cuda.synchronize()
    assert_bitwise(ye[idx], yc, "multi exact (sampled rows)")


@pytest.mark.parametrize("adapter", ["bf16", "f32"])
def test_qkv_stacked_full(adapter):
    spec = lw.QKV_STACKED if adapter == "bf16" else lw.StackedSpec(
        **{**lw.QKV_STACKED.__dict__, "name": "qkv_stacked_f32", "adapter": "f32"})
    d = lw.stacked_inputs(spec)
    T = spec.T
    rows = sample_rows(T, n_each=24, seed=2)
    say(f"case full-size qkv stacked adapter={adapter} rows={len(rows)}")
    gg = [dict(g, A=dev(g["A"]), B=dev(g["B"])) for g in d["groups"]]
    y = rg.lora_linear_stacked(dev(d["x"]), dev(d["W"]), dev(d["b"]), gg, d["strength"], d["request_scale"])
    torch.cuda.synchronize()
    xs = d["x"][rows]
    y64 = lo.lora_linear_stacked(xs, d["W"], d["b"], d["groups"], d["strength"], d["request_scale"])
    yc = ec.chain_stacked(xs, d["W"], d["b"], d["groups"], d["strength"], d["request_scale"], "bf16", adapter)
    idx = torch.from_numpy(rows).to(y.device)
    assert_gate(y[idx], y64, yc, what=f"stacked {adapter} lossless (sampled rows)")
    ye = rg.lora_linear_stacked(dev(d["x"]), dev(d["W"]), dev(d["b"]), gg, d["strength"], d["request_scale"],
                                quality="exact")
    torch.cuda.synchronize()
    assert_bitwise(ye[idx], yc, f"stacked {adapter} exact (sampled rows)")


@pytest.mark.parametrize("s", [lw.NF4_LAYER, lw.NF4_VECTOR], ids=["tokens8192", "single_vector"])
def test_nf4_layer_full(s):
    d = lw.nf4_inputs(s)
    # (8 rows per region: the fp64 references of the 4-bit layer take about a second per row on the host)
    rows = sample_rows(s.T, n_each=8, seed=3)
    say(f"case full-size nf4 T={s.T} K={s.K} N={s.N} r={s.rank} rows={len(rows)}")
    args = (dev(d["x"]), dev(d["codes"]), dev(d["absmax"]), dev(d["codebook"]), s.N, dev(d["b"]), dev(d["A"]),
            dev(d["B"]), d["alpha"], d["strength"], d["request_scale"])
    y = rg.lora_linear_nf4(*args)
    torch.cuda.synchronize()
    xs = d["x"][rows]
    W = ec.chain_nf4_weight(d["codes"], d["absmax"], d["codebook"], s.K, 64)
    say("  dequantized weight ready")
    y64 = lo.lora_linear(xs, W, d["b"], d["A"], d["B"], d["alpha"], d["rank"], d["strength"], d["request_scale"])
    yc = ec.chain_linear(xs, W, d["b"], d["A"], d["B"], d["alpha"], d["rank"], d["strength"], d["request_scale"])
    say("  rounding chain ready")
    # the fp64 reference of the 4-bit layer uses the exact codebook x absmax product
    y64_exact_w = lo.lora_linear_nf4(xs, d["codes"], d["absmax"], d["codebook"], 64, d["b"], d["A"], d["B"],
                                     d["alpha"], d["rank"], d["strength"], d["request_scale"])
    idx = torch.from_numpy(rows).to(y.device)
    assert_gate(y[idx], y64, yc, what="nf4 lossless vs bf16-weight fp64 (sampled rows)")
    assert_gate(y[idx], y64_exact_w, None, what="nf4 lossless vs exact-weight fp64 (sampled rows)")
    ye = rg.lora_linear_nf4(*args, quality="exact")
    torch.cuda.synchronize()
    assert_bitwise(ye[idx], yc, "nf4 exact (sampled rows)")


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
    rows = sample_rows(spec.N, n_each=24, seed=5)
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
