"""Pins for the CPU oracle: each check compares it with something other than itself.

* exact rational arithmetic (fractions.Fraction) and IEEE rounding written
  from the standard's rules (tests/fraction_ref.py);
* hand-worked scalar cases (tests/golden/handworked_exact_chain.json);
* algebraic identities (merged == factored, stacked == per-group layers);
* special cases that reduce to a library routine (torch F.linear in float64);
* exhaustive indexing of the 4-bit codes.

A plausible slip in the oracle -- a dropped term, a wrong sign, a transposed
operand, a wrong nibble or block index, a missing or extra rounding, the wrong
summation order -- fails at least one of these.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import exact_chain as ec
from oracle import lora_oracle as lo
from tests.fraction_ref import exact, round_fraction, dot_exact
import lora_workloads as lw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_exact_chain.json")


def _hex(v):
    return float.fromhex(v) if isinstance(v, str) else float(v)


def _mat(rows, dtype):
    if rows is None:
        return None
    a = np.array([[_hex(v) for v in r] for r in rows], dtype=np.float64)
    return lw.to_dtype(a, dtype)


def _vec(vals, dtype):
    if vals is None:
        return None
    return lw.to_dtype(np.array([_hex(v) for v in vals], dtype=np.float64), dtype)


# ---------------------------------------------------------------- rounding primitives

def _edge_f32_values():
    rng = np.random.default_rng(11)
    vals = list((rng.standard_normal(400) * np.exp2(rng.integers(-140, 126, 400))).astype(np.float32))
    # ties and near-ties at bf16 granularity, subnormals, extremes
    for base in (1.0, 1.5, 2.0 ** -130, 3.0e38, 2.0 ** -126):
        b = np.float32(base)
        u = np.array([b], np.float32).view(np.uint32)[0]
        for off in (0x7FFF, 0x8000, 0x8001, 0x17FFF, 0x18000, 0x18001, 0xFFFF):
            vals.append(np.array([u + off], np.uint32).view(np.float32)[0])
            vals.append(-np.array([u + off], np.uint32).view(np.float32)[0])
    vals += [np.float32(3.3895314e38), np.float32(np.finfo(np.float32).max), np.float32(1e-45)]
    return np.array(vals, dtype=np.float32)


def test_rn_bf16_matches_exact_rounding():
    vals = _edge_f32_values()
    got = ec.rn_bf16(vals.astype(np.float64))
    assert np.all(np.isfinite(vals))
    for v, g in zip(vals, got):
        want = round_fraction(exact(float(v)), "bf16")
        if float(v) < 0 and want == 0.0:
            want = -0.0
        assert g == want or (math.isinf(g) and math.isinf(want) and (g > 0) == (want > 0)), (v, g, want)


def test_rn_bf16_signed_zero_and_nan():
    assert math.copysign(1.0, ec.rn_bf16(np.array([-0.0]))[0]) == -1.0
    assert np.isnan(ec.rn_bf16(np.array([np.nan]))[0])
    with pytest.raises(ValueError):
        ec.rn_bf16(np.array([1.0 + 2.0 ** -40]))  # not an fp32 value


def test_rn_f32_matches_exact_rounding():
    rng = np.random.default_rng(12)
    vals = rng.standard_normal(300) * np.exp2(rng.integers(-150, 128, 300))
    vals = np.concatenate([vals, [1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, 1 + 2.0 ** -24 + 2.0 ** -50,
                                  2.0 ** -149 * 1.5, 2.0 ** -149 * 2.5, 3.4028235677973366e38]])
    got = ec.rn_f32(vals)
    for v, g in zip(vals, got):
        want = round_fraction(exact(v), "f32")
        if v < 0 and want == 0.0:
            want = -0.0
        assert g == want, (v, g, want)


# ---------------------------------------------------------------- E1 ordered GEMM

def test_gemm_ordered_is_correctly_rounded_when_fp64_sum_is_exact():
    # bf16 inputs with K = 6 and a narrow exponent range: every fp64 partial sum is exact,
    # so E1 must equal the exact dot product rounded once to fp32.
    rng = np.random.default_rng(13)
    P = lw.to_dtype(rng.standard_normal((5, 6)), "bf16")
    Q = lw.to_dtype(rng.standard_normal((7, 6)), "bf16")
    got = ec.gemm_ordered(P, Q)
    Pd, Qd = P.double().numpy(), Q.double().numpy()
    for i in range(5):
        for j in range(7):
            assert got[i, j] == round_fraction(dot_exact(Pd[i], Qd[j]), "f32")


def test_golden_linear_chain_and_plain_definition():
    cases = json.load(open(GOLDEN))["linear"]
    for c in cases:
        act, adt = c["act"], c["adapter"]
        x, W = _mat(c["x"], act), _mat(c["W"], act)
        b = _vec(c["b"], act)
        A, B = _mat(c["A"], adt), _mat(c["B"], adt)
        rs = _hex(c["request_scale"])
        y = ec.chain_linear(x, W, b, A, B, c["alpha"], c["rank"], c["strength"], rs, act, adt)
        want = np.array([[_hex(v) for v in r] for r in c["expected"]])
        assert np.array_equal(y, want), (c["name"], y, want)
        y64 = lo.lora_linear(x, W, b, A, B, c["alpha"], c["rank"], c["strength"], rs)
        want64 = np.array([[_hex(v) for v in r] for r in c["exact_fp64"]])
        if c["name"].startswith("k_ascending"):
            continue  # the fp64 plain definition itself cancels here; only the chain is pinned
        assert np.array_equal(y64, want64), (c["name"], y64, want64)


def test_golden_dense_patch_chain():
    for c in json.load(open(GOLDEN))["patch"]:
        dt = c["dtype"]
        dst = _vec([c["dst"]], dt)
        src = _vec([c["src"]], "bf16" if dt == "bf16" else "bf16")
        got = ec.chain_dense_patch(dst, src, _hex(c["strength"]), c["mode"], dt)
        assert got[0] == _hex(c["expected"]), (c["name"], got[0].hex(), c["expected"])


# ---------------------------------------------------------------- O1 plain definition

def _frac_lora_linear(x, W, b, A, B, s):
    T, K = x.shape
    N = W.shape[0]
    r = A.shape[0] if A is not None else 0
    out = [[Fraction(0)] * N for _ in range(T)]
    for m in range(T):
        t = [dot_exact(x[m], A[q]) for q in range(r)] if A is not None else []
        for n in range(N):
            v = dot_exact(x[m], W[n])
            if b is not None:
                v += exact(b[n])
            if A is not None:
                v += s * sum((t[q] * exact(B[n, q]) for q in range(r)), Fraction(0))
            out[m][n] = v
    return out


@pytest.mark.parametrize("T,K,N,r,seed", [(3, 4, 2, 3, 0), (2, 3, 4, 1, 1), (4, 2, 3, 4, 2), (1, 4, 4, 2, 3)])
def test_lora_linear_brute_force_fraction(T, K, N, r, seed):
    d = lw.small_linear_inputs(T, K, N, r, seed, bias=True, alpha=3.0, strength=0.6, request_scale=1.3)
    s = lo.combined_scale(d["alpha"], d["rank"], d["strength"], d["request_scale"])
    xd, Wd, bd, Ad, Bd = (lo.f64(d[k]) for k in ("x", "W", "b", "A", "B"))
    exact_y = _frac_lora_linear(xd, Wd, bd, Ad, Bd, Fraction(s))
    y = lo.lora_linear(d["x"], d["W"], d["b"], d["A"], d["B"], d["alpha"], d["rank"], d["strength"],
                       d["request_scale"])
    assert y.shape == (T, N)
    scale = max(abs(float(v)) for row in exact_y for v in row)
    for m in range(T):
        for n in range(N):
            assert abs(y[m, n] - float(exact_y[m][n])) <= 1e-14 * scale


def test_combined_scale_is_alpha_over_rank_times_strength_times_request():
    assert lo.combined_scale(16, 8, 1.0, 1.0) == 2.0
    assert lo.combined_scale(16, 8, 0.5, 1.0) == 1.0
    assert lo.combined_scale(64, 64, 1.0, 0.7) == 0.7
    assert lo.combined_scale(32, 16, 1.0, 1.0) == 2.0  # alpha / rank, not alpha / sqrt(rank)


@pytest.mark.parametrize("case", ["s0", "B0", "none", "neg0"])
def test_inactive_adapter_reduces_to_library_linear(case):
    d = lw.small_linear_inputs(9, 33, 17, 4, 5, bias=True)
    A, B, strength = d["A"], d["B"], 1.0
    if case == "s0":
        strength = 0.0
    elif case == "neg0":
        strength = -0.0
    elif case == "B0":
        B = torch.zeros_like(B)
    else:
        A = B = None
    y = lo.lora_linear(d["x"], d["W"], d["b"], A, B, d["alpha"], d["rank"], strength, 1.0)
    ref = torch.nn.functional.linear(d["x"].double(), d["W"].double(), d["b"].double()).numpy()
    assert np.array_equal(y, ref)
    yc = ec.chain_linear(d["x"], d["W"], d["b"], A, B, d["alpha"], d["rank"], strength, 1.0)
    yb = ec.chain_linear(d["x"], d["W"], d["b"], None, None, d["alpha"], d["rank"], 1.0, 1.0)
    assert np.array_equal(yc, yb) or case == "B0"
    if case == "B0":  # zero delta: base + 0 keeps base's value (no exact zeros in base here)
        assert not np.any(yb == 0)
        assert np.array_equal(yc, yb)


def test_merged_equals_factored():
    d = lw.small_linear_inputs(40, 72, 56, 8, 7, bias=True, alpha=16, strength=0.8, request_scale=0.7)
    s = lo.combined_scale(d["alpha"], d["rank"], d["strength"], d["request_scale"])
    y = lo.lora_linear(d["x"], d["W"], d["b"], d["A"], d["B"], d["alpha"], d["rank"], d["strength"],
                       d["request_scale"])
    Wm = lo.merged_weight(d["W"], d["A"], d["B"], s)
    y_merged = lo.f64(d["x"]) @ Wm.T + lo.f64(d["b"])[None, :]
    assert np.max(np.abs(y - y_merged)) <= 1e-12 * np.max(np.abs(y))
    # and the merged weight itself is W + s*B@A elementwise, checked exactly on a few entries
    Wd, Ad, Bd = lo.f64(d["W"]), lo.f64(d["A"]), lo.f64(d["B"])
    for n, k in [(0, 0), (55, 71), (13, 40)]:
        want = exact(Wd[n, k]) + Fraction(s) * dot_exact(Bd[n], Ad[:, k])
        assert abs(Wm[n, k] - float(want)) <= 1e-15 * max(1.0, abs(float(want)))


def test_pure_low_rank_when_base_is_zero():
    d = lw.small_linear_inputs(3, 5, 4, 2, 9, bias=False, alpha=2.0, strength=1.5)
    Wz = torch.zeros_like(d["W"])
    y = lo.lora_linear(d["x"], Wz, None, d["A"], d["B"], d["alpha"], d["rank"], d["strength"], 1.0)
    s = Fraction(lo.combined_scale(d["alpha"], d["rank"], d["strength"], 1.0))
    ex = _frac_lora_linear(lo.f64(d["x"]), lo.f64(Wz), None, lo.f64(d["A"]), lo.f64(d["B"]), s)
    for m in range(3):
        for n in range(4):
            assert abs(y[m, n] - float(ex[m][n])) <= 1e-15 * (abs(float(ex[m][n])) + 1e-300)


# ---------------------------------------------------------------- stacked

def _stacked_case(seed, bias=True, adt="bf16"):
    rng = np.random.default_rng(seed)
    T, K = 11, 24
    n_cols, ranks, alphas, offs = (7, 5, 9), (3, 2, 4), (6.0, 2.0, 2.0), (0, 9, 14)
    x = lw.to_dtype(rng.standard_normal((T, K)), "bf16")
    W = lw.to_dtype(rng.standard_normal((25, K)) / 5, "bf16")  # 2 columns (7, 8) and 23, 24 are base-only
    b = lw.to_dtype(rng.standard_normal(25) / 7, "bf16") if bias else None
    groups = []
    for n, r, a, o in zip(n_cols, ranks, alphas, offs):
        groups.append(dict(A=lw.to_dtype(rng.standard_normal((r, K)) / 5, adt),
                           B=lw.to_dtype(rng.standard_normal((n, r)) / 3, adt),
                           rank=r, alpha=a, col_offset=o, n_cols=n))
    return x, W, b, groups


def test_stacked_equals_per_group_layers():
    x, W, b, groups = _stacked_case(21)
    y = lo.lora_linear_stacked(x, W, b, groups, 0.9, 1.1)
    yc = ec.chain_stacked(x, W, b, groups, 0.9, 1.1)
    covered = np.zeros(25, bool)
    for g in groups:
        o, n = g["col_offset"], g["n_cols"]
        covered[o:o + n] = True
        y1 = lo.lora_linear(x, W[o:o + n], b[o:o + n], g["A"], g["B"], g["alpha"], g["rank"], 0.9, 1.1)
        assert np.array_equal(y[:, o:o + n], y1)
        c1 = ec.chain_linear(x, W[o:o + n], b[o:o + n], g["A"], g["B"], g["alpha"], g["rank"], 0.9, 1.1)
        assert np.array_equal(yc[:, o:o + n], c1)
    base = torch.nn.functional.linear(x.double(), W.double(), b.double()).numpy()
    assert np.array_equal(y[:, ~covered], base[:, ~covered])


# ---------------------------------------------------------------- 4-bit codes

def test_nf4_nibble_order_and_block_index_exhaustive():
    N, K = 3, 256  # 4 blocks of 64 per row; every code in both nibble positions at block edges
    codes = np.zeros((N, K // 2), np.uint8)
    for n in range(N):
        for j in range(K // 2):
            lo_c = (j + n) % 16
            hi_c = (3 * j + 5 * n + 7) % 16
            codes[n, j] = lo_c | (hi_c << 4)
    cb = torch.tensor([2.0 ** (c - 8) for c in range(16)], dtype=torch.float32)
    absmax = torch.tensor([float(i + 1) for i in range(N * K // 64)], dtype=torch.float32)
    W = lo.nf4_dequant(torch.from_numpy(codes), absmax, cb, K, 64)
    We = ec.chain_nf4_weight(torch.from_numpy(codes), absmax, cb, K, 64)
    seen = set()
    for n in range(N):
        for k in range(K):
            byte = int(codes[n, k // 2])
            code = (byte & 0xF) if k % 2 == 0 else (byte >> 4)
            blk = (n * K + k) // 64
            want = 2.0 ** (code - 8) * (blk + 1)
            assert W[n, k] == want, (n, k)
            seen.add((code, k % 2))
            # (blk + 1) * 2^(code - 8) has at most 4 significant bits: exact in bf16
            assert We[n, k] == want
    assert len(seen) == 32


def test_nf4_unpack_codes_hand_written_bytes():
    # byte j holds element 2j in bits 0-3 and element 2j+1 in bits 4-7
    codes = np.array([[0x3A, 0xF0], [0x01, 0x9C]], np.uint8)
    got = lo.nf4_unpack_codes(codes, 4)
    assert got.tolist() == [[0xA, 0x3, 0x0, 0xF], [0x1, 0x0, 0xC, 0x9]]


def test_rn_dispatches_to_the_named_rounding():
    # bf16 keeps 8 significant bits (spacing 2^-7 in [1, 2), 2^-6 in [2, 4)), fp32 24; worked by hand:
    # 1 + 2^-9: a quarter spacing above 1; 1 + 2^-8: a tie, to the even 1; 1 + 3 2^-8: a tie between
    # 1 + 2^-7 (odd) and 1 + 2^-6 (even); -3 - 2^-7 - 2^-12: past the midpoint -3 - 2^-7, so away;
    # 1 + 2^-30: below fp32's spacing 2^-23 at 1
    # (the bf16 rounding takes fp32-representable values, as the chain produces them)
    v = np.array([1.0 + 2.0 ** -9, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -3.0 - 2.0 ** -7 - 2.0 ** -12])
    assert ec.rn(v, "bf16").tolist() == [1.0, 1.0, 1.0 + 2.0 ** -6, -3.015625]
    assert ec.rn(v, "f32").tolist() == v.tolist()
    assert ec.rn(np.array([1.0 + 2.0 ** -30]), "f32").tolist() == [1.0]
    with pytest.raises(ValueError):
        ec.rn(v, "f16")


def test_nf4_weight_rounds_product_to_bf16():
    codes = torch.tensor([[0x10]], dtype=torch.uint8)  # element 0: code 0, element 1: code 1
    cb = torch.tensor([1.0 + 2.0 ** -8] + [1.0 + 2.0 ** -7 + 2.0 ** -8] + [0.0] * 14, dtype=torch.float32)
    absmax = torch.tensor([1.0], dtype=torch.float32)
    We = ec.chain_nf4_weight(codes, absmax, cb, 2, 2)
    assert We[0, 0] == 1.0                # tie -> even
    assert We[0, 1] == 1.0 + 2.0 ** -6    # tie -> even (up)


def _nf4_tiny(seed, T=3, N=2, K=128):
    """A tiny 4-bit layer over two 64-element blocks per row: every code appears in both nibble
    positions of every block of every row, the NF4-style codebook of the workloads (values with many
    significant bits), absmax of mixed magnitudes."""
    rng = np.random.default_rng(seed)
    codes = np.zeros((N, K // 2), np.uint8)
    for n in range(N):
        for j in range(K // 2):
            codes[n, j] = (j % 16) | (((j // 2 + 5 * n + 3) % 16) << 4)
    absmax = torch.tensor(np.abs(rng.standard_normal(N * K // 64)) * 0.3 + 0.05, dtype=torch.float32)
    cb = lw.nf4_style_codebook()
    x = lw.to_dtype(rng.standard_normal((T, K)), "bf16")
    A = lw.to_dtype(rng.standard_normal((4, K)) / 11, "bf16")
    B = lw.to_dtype(rng.standard_normal((N, 4)) * 0.2, "bf16")
    b = lw.to_dtype(rng.standard_normal(N) * 0.1, "bf16")
    return torch.from_numpy(codes), absmax, cb, x, A, B, b


def test_nf4_layer_against_exact_rationals():
    """The 4-bit layer (unpacked codes x block absmax, then the LoRA linear) against exact rationals:
    the only difference allowed is float64 rounding of the sums (a relative 1e-12 of the absolute
    terms). A wrong nibble, block, operand or scale fails by orders of magnitude more."""
    codes, absmax, cb, x, A, B, b = _nf4_tiny(40)
    alpha, rank, strength, rs = 8.0, 4, 0.8, 0.7
    y = lo.lora_linear_nf4(x, codes, absmax, cb, 64, b, A, B, alpha, rank, strength, rs)
    X, Am, Bm, bm = (lo.f64(v) for v in (x, A, B, b))
    am, cbv, cd = lo.f64(absmax), lo.f64(cb), codes.numpy()
    T, K = X.shape
    N = cd.shape[0]
    s = Fraction(alpha) / rank * Fraction(strength) * Fraction(rs)
    assert y.shape == (T, N)
    for n in range(N):
        w = []
        for k in range(K):
            byte = int(cd[n, k // 2])
            c = byte & 0xF if k % 2 == 0 else byte >> 4
            w.append(exact(cbv[c]) * exact(am[(n * K + k) // 64]))
        for t in range(T):
            base = sum((exact(X[t, k]) * w[k] for k in range(K)), Fraction(0)) + exact(bm[n])
            low = sum((dot_exact(X[t], Am[q]) * exact(Bm[n, q]) for q in range(rank)), Fraction(0))
            want = base + s * low
            scale = sum(abs(float(exact(X[t, k]) * w[k])) for k in range(K)) + 1.0
            assert abs(y[t, n] - float(want)) <= 1e-12 * scale, (t, n, y[t, n], float(want))


def test_chain_nf4_hand_worked_rows():
    """chain_nf4 on a 3 x 128 layer with rows=[2, 0], each rounding point worked with exact rationals
    and the IEEE rules (tests/fraction_ref.py): W = RN_bf16(RN_f32(cb[c] . absmax)); base =
    RN_bf16(RN_f32(G(x, W) + b)); t = RN_bf16(G(x, A)); d = RN_bf16(G(t, B)); one pass per non-unit
    factor; y = RN_bf16(RN_f32(base + d)). x, A and B are small dyadic values, so every float64 sum
    of E1 is exact and G is the correctly rounded exact dot product."""
    rng = np.random.default_rng(41)
    T, N, K, r = 3, 2, 128, 2
    codes = np.zeros((N, K // 2), np.uint8)
    for n in range(N):
        for j in range(K // 2):
            codes[n, j] = (j % 16) | (((3 * j + n) % 16) << 4)
    codes = torch.from_numpy(codes)
    absmax = torch.tensor([0.7, 1.3, 0.45, 2.1], dtype=torch.float32)
    cb = lw.nf4_style_codebook()
    x = lw.to_dtype(rng.integers(-4, 5, (T, K)) / 8.0, "bf16")
    A = lw.to_dtype(rng.integers(-3, 4, (r, K)) / 16.0, "bf16")
    B = lw.to_dtype(rng.integers(-3, 4, (N, r)) / 4.0, "bf16")
    b = lw.to_dtype(np.array([0.3, -0.2]), "bf16")
    alpha, strength, rs = 3.0, 0.8, 1.0   # factors 1.5, 0.8 (request scale 1 skipped)
    rows = [2, 0]
    got = ec.chain_nf4(x, codes, absmax, cb, 64, b, A, B, alpha, r, strength, rs, rows=rows)
    assert got.shape == (len(rows), N)
    X, Am, Bm, bm, am, cbv = (lo.f64(v) for v in (x, A, B, b, absmax, cb))
    cd = codes.numpy()
    R = lambda q, f: Fraction(round_fraction(q, f))
    Wd = [[R(R(exact(cbv[(int(cd[n, k // 2]) & 0xF) if k % 2 == 0 else int(cd[n, k // 2]) >> 4])
                   * exact(am[(n * K + k) // 64]), "f32"), "bf16") for k in range(K)] for n in range(N)]
    f1 = R(Fraction(alpha) / r, "f32")
    f2 = R(exact(strength), "f32")
    for i, t in enumerate(rows):
        tt = [R(R(dot_exact(X[t], Am[q]), "f32"), "bf16") for q in range(r)]
        for n in range(N):
            g = R(sum((exact(X[t, k]) * Wd[n][k] for k in range(K)), Fraction(0)), "f32")
            base = R(R(g + exact(bm[n]), "f32"), "bf16")
            d = R(R(sum((tt[q] * exact(Bm[n, q]) for q in range(r)), Fraction(0)), "f32"), "bf16")
            d = R(R(d * f1, "f32"), "bf16")
            d = R(R(d * f2, "f32"), "bf16")
            want = R(R(base + d, "f32"), "bf16")
            assert got[i, n] == float(want), (t, n, got[i, n], float(want))
    # rows=None is every row in order, and the same values
    full = ec.chain_nf4(x, codes, absmax, cb, 64, b, A, B, alpha, r, strength, rs)
    assert np.array_equal(full[rows], got)


# ---------------------------------------------------------------- the accuracy metric

def test_rel_rms_hand_computed():
    """||y - ref||_2 / ||ref||_2 over all elements, divided by the reference's norm."""
    assert lo.rel_rms(np.array([3.0, 4.5]), np.array([3.0, 4.0])) == pytest.approx(0.1, rel=1e-15)
    # over the flattened matrix (not a mean of per-row errors: that would give 0.3)
    ref = np.array([[1.0, 2.0], [2.0, 4.0]])           # norm 5
    y = ref + np.array([[0.0, 0.0], [0.0, -3.0]])      # error norm 3
    assert lo.rel_rms(y, ref) == pytest.approx(0.6, rel=1e-15)
    # the reference's norm, not the result's (that would give 0.5)
    assert lo.rel_rms(np.array([6.0, 8.0]), np.array([3.0, 4.0])) == pytest.approx(1.0, rel=1e-15)
    # torch tensors are widened exactly
    assert lo.rel_rms(torch.tensor([3.0, 4.5], dtype=torch.bfloat16), np.array([3.0, 4.0])) == \
        pytest.approx(0.1, rel=1e-15)
    assert lo.rel_rms(ref, ref) == 0.0


# ---------------------------------------------------------------- dense patch

def test_dense_patch_chain_matches_exact_rounding_random():
    rng = np.random.default_rng(31)
    dst = lw.to_dtype(rng.standard_normal(300), "bf16")
    diff = lw.to_dtype(rng.standard_normal(300) * 1e-3, "bf16")
    special = torch.tensor([0.0, -0.0, 3.3895e38, -3.3895e38, 1e-40, -1e-40], dtype=torch.bfloat16)
    dst = torch.cat([dst, special])
    diff = torch.cat([diff, torch.tensor([-0.0, 0.0, 3.3895e38, 1.0, 1e-40, 1e-41], dtype=torch.bfloat16)])
    for strength in (0.8, 1.0, -2.5):
        got = ec.chain_dense_patch(dst, diff, strength, "add", "bf16")
        s32 = exact(round_fraction(exact(strength), "f32"))
        for i in range(len(dst)):
            a, b = float(dst[i]), float(diff[i])
            prod = round_fraction(exact(b) * s32, "f32")
            if math.isinf(prod):
                tot = prod
            else:
                tot = round_fraction(exact(a) + exact(prod), "f32") if not math.isinf(a) else a
            want = tot if math.isinf(tot) else round_fraction(exact(tot), "bf16")
            g = got[i]
            if want == 0.0:
                assert g == 0.0  # sign of exact zeros: IEEE sum rules, checked separately
            else:
                assert g == want, (i, a, b, strength, g, want)
        rep = ec.chain_dense_patch(dst, diff, strength, "replace", "bf16")
        for i in range(len(dst)):
            p = round_fraction(exact(float(diff[i])) * s32, "f32")
            want = p if math.isinf(p) else round_fraction(exact(p), "bf16")
            assert rep[i] == want or (want == 0.0 and rep[i] == 0.0)


def test_dense_patch_plain_definition():
    dst = torch.tensor([1.0, -2.0, 0.5], dtype=torch.bfloat16)
    src = torch.tensor([0.25, 0.5, -1.0], dtype=torch.bfloat16)
    assert np.array_equal(lo.dense_patch(dst, src, 2.0, "add"), [1.5, -1.0, -1.5])
    assert np.array_equal(lo.dense_patch(dst, src, 0.0, "add"), [1.0, -2.0, 0.5])
    assert np.array_equal(lo.dense_patch(dst, src, 2.0, "replace"), [0.5, 1.0, -2.0])


# ---------------------------------------------------------------- exactness on dyadic inputs

def _representable(q: Fraction, fmt: str) -> bool:
    return Fraction(round_fraction(q, fmt)) == q


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dyadic_inputs_every_tier_is_exact(seed):
    d = lw.dyadic_linear_inputs(6, 40, 9, 3, seed, bias=True)
    xd, Wd, bd, Ad, Bd = (lo.f64(d[k]) for k in ("x", "W", "b", "A", "B"))
    alpha, rank, strength, rs = 3.0, 3, 2.0, 0.5  # combined scale 1.0; chain multiplies by 2 then 0.5
    ex = _frac_lora_linear(xd, Wd, bd, Ad, Bd, Fraction(1))
    # every intermediate representable: t, d and y in bf16
    for m in range(6):
        for q in range(3):
            assert _representable(dot_exact(xd[m], Ad[q]), "bf16")
        for n in range(9):
            assert _representable(ex[m][n], "bf16")
    y = lo.lora_linear(d["x"], d["W"], d["b"], d["A"], d["B"], alpha, rank, strength, rs)
    yc = ec.chain_linear(d["x"], d["W"], d["b"], d["A"], d["B"], alpha, rank, strength, rs)
    for m in range(6):
        for n in range(9):
            assert y[m, n] == float(ex[m][n])
            assert yc[m, n] == float(ex[m][n])


# ---------------------------------------------------------------- the accuracy gate is discriminating

def test_chain_error_is_within_gate_and_nonzero():
    d = lw.small_linear_inputs(48, 256, 80, 16, 41, bias=True, alpha=16, strength=0.8, request_scale=0.7)
    y64 = lo.lora_linear(d["x"], d["W"], d["b"], d["A"], d["B"], d["alpha"], d["rank"], d["strength"],
                         d["request_scale"])
    yc = ec.chain_linear(d["x"], d["W"], d["b"], d["A"], d["B"], d["alpha"], d["rank"], d["strength"],
                         d["request_scale"])
    e = lo.rel_rms(yc, y64)
    assert 1e-4 < e < 4e-3
    # a single bf16 rounding of the fp64 result is better than the chain
    e1 = lo.rel_rms(ec.rn_bf16(ec.rn_f32(y64)), y64)
    assert e1 < e


# ------------------------------------------------------------------ several adapters on one layer

def _int_mat(rng, shape, lo=-3, hi=4, dtype="bf16"):
    """Small integers: every product and sum below is exact in float64 (and in bf16 inputs)."""
    return lw.to_dtype(rng.integers(lo, hi, size=shape).astype(np.float64), dtype)


def _multi_case(seed, T=5, K=6, N=7, ranks=(2, 3, 1), spans=((0, 7), (2, 4), (5, 2)), with_c=True):
    rng = np.random.default_rng(seed)
    x, W, b = _int_mat(rng, (T, K)), _int_mat(rng, (N, K)), _int_mat(rng, (N,))
    ads = []
    for i, (r, (o, n)) in enumerate(zip(ranks, spans)):
        ads.append(dict(A=_int_mat(rng, (r, K)), B=_int_mat(rng, (n, r)),
                        c=_int_mat(rng, (n,)) if with_c and i != 1 else None,
                        rank=r, alpha=[2.0, 1.5, 4.0][i] * r, strength=[1.0, 0.5, -2.0][i],
                        col_offset=o, n_cols=n))
    return x, W, b, ads


def test_multi_brute_force_fraction():
    """Overlapping adapters with legacy biases against exact rationals, element by element."""
    x, W, b, ads = _multi_case(0)
    rs = 0.75
    y = lo.lora_linear_multi(x, W, b, ads, rs)
    X, Wn, bn = (lo.f64(v) for v in (x, W, b))
    T, N = y.shape
    for t in range(T):
        for n in range(N):
            v = dot_exact(X[t], Wn[n]) + exact(bn[n])
            for a in ads:
                o, nc = a["col_offset"], a["n_cols"]
                if not o <= n < o + nc:
                    continue
                s = Fraction(a["alpha"]) / a["rank"] * Fraction(a["strength"]) * Fraction(rs)
                A, B = lo.f64(a["A"]), lo.f64(a["B"])
                u = sum((dot_exact(X[t], A[q]) * exact(B[n - o, q]) for q in range(a["rank"])), Fraction(0))
                v += s * u
                if a["c"] is not None:  # the legacy vector: strength and request scale, not alpha / rank
                    v += Fraction(a["strength"]) * Fraction(rs) * exact(lo.f64(a["c"])[n - o])
            assert y[t, n] == float(v), (t, n)


def test_multi_one_adapter_reduces_to_the_single_layer():
    d = lw.small_linear_inputs(9, 16, 11, 4, 5, bias=True, alpha=6.0)
    ad = dict(A=d["A"], B=d["B"], c=None, rank=4, alpha=6.0, strength=0.8, col_offset=0, n_cols=11)
    y = lo.lora_linear_multi(d["x"], d["W"], d["b"], [ad], 0.7)
    assert np.array_equal(y, lo.lora_linear(d["x"], d["W"], d["b"], d["A"], d["B"], 6.0, 4, 0.8, 0.7))
    yc = ec.chain_multi(d["x"], d["W"], d["b"], [ad], 0.7)
    assert np.array_equal(yc, ec.chain_linear(d["x"], d["W"], d["b"], d["A"], d["B"], 6.0, 4, 0.8, 0.7))


def test_multi_disjoint_adapters_equal_stacked_groups():
    rng = np.random.default_rng(3)
    x, W, b = _int_mat(rng, (4, 8)), _int_mat(rng, (10, 8)), _int_mat(rng, (10,))
    groups = [dict(A=_int_mat(rng, (2, 8)), B=_int_mat(rng, (4, 2)), rank=2, alpha=3.0, col_offset=0, n_cols=4),
              dict(A=_int_mat(rng, (3, 8)), B=_int_mat(rng, (5, 3)), rank=3, alpha=1.5, col_offset=5, n_cols=5)]
    ads = [dict(g, c=None, strength=0.5) for g in groups]
    assert np.array_equal(lo.lora_linear_multi(x, W, b, ads, 2.0), lo.lora_linear_stacked(x, W, b, groups, 0.5, 2.0))
    assert np.array_equal(ec.chain_multi(x, W, b, ads, 2.0), ec.chain_stacked(x, W, b, groups, 0.5, 2.0))


def test_multi_equals_one_adapter_of_concatenated_rank_and_merged_weight():
    """Two adapters on all columns == one adapter [A1; A2], [s1 B1 | s2 B2] with unit scale and the
    bias b + u1 c1 + u2 c2 (u_i = strength_i . request scale) == the merged weight W + s1 B1 A1 +
    s2 B2 A2 with that bias (integer data: exact)."""
    x, W, b, ads = _multi_case(7, ranks=(2, 3), spans=((0, 7), (0, 7)))
    ads[1]["c"] = _int_mat(np.random.default_rng(8), (7,))
    rs = 0.5
    y = lo.lora_linear_multi(x, W, b, ads, rs)
    s = [lo.combined_scale(a["alpha"], a["rank"], a["strength"], rs) for a in ads]
    A_cat = np.concatenate([lo.f64(a["A"]) for a in ads])
    B_cat = np.concatenate([si * lo.f64(a["B"]) for si, a in zip(s, ads)], axis=1)
    b_all = lo.f64(b) + sum(a["strength"] * rs * lo.f64(a["c"]) for a in ads)
    assert np.array_equal(y, lo.lora_linear(x, W, b_all, A_cat, B_cat, 5.0, 5, 1.0, 1.0))
    W_m = lo.f64(W) + sum(si * (lo.f64(a["B"]) @ lo.f64(a["A"])) for si, a in zip(s, ads))
    assert np.array_equal(y, lo.f64(x) @ W_m.T + b_all[None, :])


def test_multi_chain_legacy_bias_is_its_own_pass_after_the_delta():
    """Hand-worked (bf16 throughout):
    (a) base 1, one adapter with d = 2^-8 (unit scales) and legacy vector c = 2^-8 on the same column:
        1 + 2^-8 is half a bf16 spacing above 1, a tie, so y = RN(1 + d) = 1, then RN(1 + c) = 1
        again; folding c into the rank GEMM before its rounding would give d = 2^-7 and y = 1 + 2^-7.
    (b) two adapters each with d = 2^-8 on the same column: 1 + 2^-8 rounds to 1 after the first and
        again after the second, so y = 1 (adding 2^-8 + 2^-8 first would give 1 + 2^-7).
    (c) alpha / rank = 4, strength 0.5, request scale 0.75, B = 0, c = 1: the vector takes 0.5 then
        0.75 (bf16 0.375), not 4 . 0.5 . 0.75 = 1.5."""
    bf = lambda rows: lw.to_dtype(np.array(rows, dtype=np.float64), "bf16")
    one = dict(A=bf([[1.0]]), B=bf([[2.0 ** -8]]), c=None, rank=1, alpha=1.0, strength=1.0, col_offset=0, n_cols=1)
    y = ec.chain_multi(bf([[1.0]]), bf([[1.0]]), None, [dict(one, c=bf([2.0 ** -8]))], 1.0)
    assert y[0, 0] == 1.0
    assert lo.lora_linear_multi(bf([[1.0]]), bf([[1.0]]), None, [dict(one, c=bf([2.0 ** -8]))], 1.0)[0, 0] == \
        1.0 + 2.0 ** -7
    y2 = ec.chain_multi(bf([[1.0]]), bf([[1.0]]), None, [one, dict(one)], 1.0)
    assert y2[0, 0] == 1.0
    assert lo.lora_linear_multi(bf([[1.0]]), bf([[1.0]]), None, [one, dict(one)], 1.0)[0, 0] == 1.0 + 2.0 ** -7
    z = dict(A=bf([[1.0]]), B=bf([[0.0]]), c=bf([1.0]), rank=2, alpha=8.0, strength=0.5, col_offset=0, n_cols=1)
    z["A"] = bf([[1.0], [1.0]])
    z["B"] = bf([[0.0, 0.0]])
    assert ec.chain_multi(bf([[1.0]]), bf([[0.0]]), None, [z], 0.75)[0, 0] == 0.375
    assert lo.lora_linear_multi(bf([[1.0]]), bf([[0.0]]), None, [z], 0.75)[0, 0] == 0.375


def test_multi_inactive_adapter_drops_its_bias():
    x, W, b, ads = _multi_case(11)
    ads0 = [dict(a) for a in ads]
    ads0[0]["strength"] = 0.0
    y = lo.lora_linear_multi(x, W, b, ads0, 1.0)
    assert np.array_equal(y, lo.lora_linear_multi(x, W, b, ads0[1:], 1.0))


# ------------------------------------------------------------------ merge W <- W + s.B.A

def test_merge_chain_against_exact_rounding():
    """Each rounding point of the exact merge against Fraction arithmetic rounded by the IEEE rules."""
    rng = np.random.default_rng(21)
    N, K, r = 5, 7, 3
    W = lw.to_dtype(rng.standard_normal((N, K)) * 0.05, "bf16")
    A = lw.to_dtype(rng.standard_normal((r, K)) / 3, "bf16")
    B = lw.to_dtype(rng.standard_normal((N, r)) * 0.1, "bf16")
    for alpha, strength in ((3.0, 0.7), (3.0, 1.0)):
        got = ec.chain_merge(W, A, B, alpha, r, strength)
        s32 = round_fraction(Fraction(alpha) / r * Fraction(strength), "f32")
        Wn, An, Bn = lo.f64(W), lo.f64(A), lo.f64(B)
        for n in range(N):
            for k in range(K):
                g = round_fraction(sum((exact(Bn[n, q]) * exact(An[q, k]) for q in range(r)), Fraction(0)), "f32")
                d = g if s32 == 1.0 else round_fraction(exact(g) * exact(s32), "f32")
                v = round_fraction(exact(Wn[n, k]) + exact(d), "f32")
                assert got[n, k] == round_fraction(exact(v), "bf16"), (alpha, strength, n, k)


def test_merge_chain_hand_worked():
    """W = 1, B.A = 2^-8: 1 + 2^-8 is half the bf16 spacing (2^-7) above 1, a tie, and rounds to the
    even neighbour 1 -- the update is rounded away entirely. With s = 3, 1 + 3 . 2^-8 is 1.5 spacings
    above 1, again a tie, between 1 + 2^-7 (odd) and 1 + 2^-6 (even): the merge gives 1 + 2^-6, twice
    the 1 + 3 . 2^-8 the plain definition keeps."""
    bf = lambda rows: lw.to_dtype(np.array(rows, dtype=np.float64), "bf16")
    W, A, B = bf([[1.0]]), bf([[2.0 ** -4]]), bf([[2.0 ** -4]])
    assert ec.chain_merge(W, A, B, 1.0, 1, 1.0)[0, 0] == 1.0
    assert ec.chain_merge(W, A, B, 3.0, 1, 1.0)[0, 0] == 1.0 + 2.0 ** -6
    # the plain definition keeps the whole update (fp64)
    assert lo.merged_weight(W, A, B, 3.0)[0, 0] == 1.0 + 3 * 2.0 ** -8


def test_merged_weight_linear_equals_the_adapter_layer():
    """x.(W + s.B.A)^T + b == the LoRA linear (integer data: exact)."""
    rng = np.random.default_rng(22)
    x, W, b = _int_mat(rng, (4, 6)), _int_mat(rng, (5, 6)), _int_mat(rng, (5,))
    A, B = _int_mat(rng, (2, 6)), _int_mat(rng, (5, 2))
    s = lo.combined_scale(3.0, 2, 0.5, 1.0)
    y_merged = lo.f64(x) @ lo.merged_weight(W, A, B, s).T + lo.f64(b)[None, :]
    assert np.array_equal(y_merged, lo.lora_linear(x, W, b, A, B, 3.0, 2, 0.5, 1.0))


# ------------------------------------------------------------------ backward

def test_backward_matches_central_differences():
    """The loss L = <G, y> is linear in x, in A (B fixed), in B (A fixed) and in b, so a central
    difference along any direction equals the directional derivative up to float64 rounding."""
    rng = np.random.default_rng(31)
    T, K, N, r = 5, 7, 6, 3
    x, W, A, B = (rng.standard_normal(sh) for sh in ((T, K), (N, K), (r, K), (N, r)))
    b, G = rng.standard_normal(N), rng.standard_normal((T, N))
    alpha, st, rs = 4.5, 0.8, 0.7
    L = lambda x_, A_, B_, b_: float((G * lo.lora_linear(x_, W, b_, A_, B_, alpha, r, st, rs)).sum())
    dx, dA, dB, db = lo.lora_linear_backward(x, W, A, B, G, alpha, r, st, rs)
    h = 1e-3
    for grad, idx in ((dx, 0), (dA, 1), (dB, 2), (db, 3)):
        E = rng.standard_normal(grad.shape)
        args_p = [x, A, B, b]
        args_m = [x, A, B, b]
        args_p[idx] = args_p[idx] + h * E
        args_m[idx] = args_m[idx] - h * E
        fd = (L(*args_p) - L(*args_m)) / (2 * h)
        assert abs(fd - float((grad * E).sum())) <= 1e-9 * max(1.0, abs(fd)), idx


def test_backward_brute_force_fraction():
    """Element by element against exact rationals (small integers, dyadic scale)."""
    rng = np.random.default_rng(32)
    T, K, N, r = 3, 4, 5, 2
    x, W, A, B = (rng.integers(-3, 4, size=sh).astype(np.float64) for sh in ((T, K), (N, K), (r, K), (N, r)))
    G = rng.integers(-3, 4, size=(T, N)).astype(np.float64)
    alpha, st, rs = 3.0, 0.5, 0.75
    s = Fraction(alpha) / r * Fraction(st) * Fraction(rs)
    dx, dA, dB, db = lo.lora_linear_backward(x, W, A, B, G, alpha, r, st, rs)
    F = lambda v: Fraction(float(v))
    u = [[sum(F(G[t, n]) * F(B[n, q]) for n in range(N)) for q in range(r)] for t in range(T)]
    tt = [[sum(F(x[t, k]) * F(A[q, k]) for k in range(K)) for q in range(r)] for t in range(T)]
    for t in range(T):
        for k in range(K):
            v = sum(F(G[t, n]) * F(W[n, k]) for n in range(N)) + s * sum(u[t][q] * F(A[q, k]) for q in range(r))
            assert dx[t, k] == float(v)
    for q in range(r):
        for k in range(K):
            assert dA[q, k] == float(s * sum(u[t][q] * F(x[t, k]) for t in range(T)))
    for n in range(N):
        for q in range(r):
            assert dB[n, q] == float(s * sum(F(G[t, n]) * tt[t][q] for t in range(T)))
        assert db[n] == float(sum(F(G[t, n]) for t in range(T)))
