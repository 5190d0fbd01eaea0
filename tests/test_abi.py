"""The C-ABI boundary on the CPU: the library loads, exports every symbol the
header declares, and rejects each invalid argument with its status code
before anything is launched (no HIP call is made on these paths)."""
import math
import os
import re
import subprocess

import pytest

import rank_gemm_lora_amd as rg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_mi355x.h")

OK, NULL, SHAPE, DTYPE, NONFIN, ALIGN, OVERLAP, WS, UNSUP, HIP = range(10)
F32, BF16 = rg.LORA_F32, rg.LORA_BF16
LOSSLESS, EXACT = rg.LORA_LOSSLESS, rg.LORA_EXACT

# fake, well-separated, 256-byte-aligned device addresses: validation never dereferences them
X, W, Y, A, B, BIAS, WSP = (0x10_0000_0000 + i * 0x1_0000_0000 for i in range(7))


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"^(?:int|size_t|const char\*)\s+(\w+)\(", src, flags=re.M)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    assert {"lora_linear_fwd", "lora_linear_stacked_fwd", "lora_linear_nf4_fwd", "dense_patch_apply",
            "lora_linear_workspace_size", "lora_status_string", "lora_device_check"} <= names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", rg.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(rg._lib, name)


def test_one_hip_runtime_mapped():
    assert len(rg.hip_runtimes_mapped()) <= 1


def lin(**kw):
    a = dict(x=X, T=64, K=128, ldx=128, W=W, N=96, bias=BIAS, A=A, B=B, rank=8, adt=BF16, alpha=16.0,
             strength=1.0, rs=1.0, y=Y, ldy=96, act=BF16, q=LOSSLESS, ws=WSP, wsb=1 << 30)
    a.update(kw)
    return rg._lib.lora_linear_fwd(a["x"], a["T"], a["K"], a["ldx"], a["W"], a["N"], a["bias"], a["A"], a["B"],
                                   a["rank"], a["adt"], a["alpha"], a["strength"], a["rs"], a["y"], a["ldy"],
                                   a["act"], a["q"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(y=None), NULL), (dict(W=None), NULL), (dict(B=None), NULL),
    (dict(A=None), NULL),
    (dict(T=-1), SHAPE), (dict(K=0), SHAPE), (dict(N=0), SHAPE), (dict(ldx=64), SHAPE), (dict(ldy=95), SHAPE),
    (dict(rank=0), SHAPE), (dict(rank=5000), UNSUP),
    (dict(act=F32, adt=BF16), DTYPE), (dict(act=3), DTYPE), (dict(adt=-1), DTYPE), (dict(q=7), UNSUP),
    (dict(alpha=math.nan), NONFIN), (dict(strength=math.inf), NONFIN), (dict(rs=-math.inf), NONFIN),
    (dict(alpha=1e300), NONFIN),
    (dict(x=X + 2), ALIGN), (dict(K=124, ldx=128), ALIGN), (dict(ldx=132), ALIGN), (dict(A=A + 8), ALIGN),
    (dict(y=Y + 1), ALIGN),
    (dict(ws=WSP + 4), ALIGN),
    (dict(y=X + 64), OVERLAP), (dict(y=W), OVERLAP), (dict(y=B - 64), OVERLAP), (dict(ws=Y), OVERLAP),
    (dict(ws=None), WS), (dict(wsb=64 * 64 * 2 - 1), WS),
])
def test_linear_rejects(kw, code):
    assert lin(**kw) == code


def test_linear_valid_noop_and_inactive_need_no_workspace():
    assert lin(T=0) == OK                       # validated, nothing launched
    assert lin(T=0, x=None, y=None) == OK
    assert lin(T=0, A=None, B=None, ws=None, wsb=0) == OK
    assert lin(T=0, strength=0.0, ws=None, wsb=0) == OK
    # exact tier needs only element alignment
    assert lin(T=0, x=X + 2, q=EXACT) == OK
    assert lin(T=0, x=X + 1, q=EXACT) == ALIGN


def phase(ph, tile=0, **kw):
    a = dict(x=X, T=64, K=128, ldx=128, W=W, N=96, bias=BIAS, A=A, B=B, rank=8, adt=BF16, alpha=16.0,
             strength=1.0, rs=1.0, y=Y, ldy=96, act=BF16, q=LOSSLESS, ws=WSP, wsb=1 << 30)
    a.update(kw)
    return rg._lib.lora_linear_fwd_phase(ph, tile, a["x"], a["T"], a["K"], a["ldx"], a["W"], a["N"], a["bias"],
                                         a["A"], a["B"], a["rank"], a["adt"], a["alpha"], a["strength"], a["rs"],
                                         a["y"], a["ldy"], a["act"], a["q"], a["ws"], a["wsb"], None)


def test_phase_entry_point_validation():
    assert phase(3) == UNSUP and phase(-1) == UNSUP
    assert phase(0, tile=3) == UNSUP and phase(1, tile=-1) == UNSUP and phase(2, tile=1 << 20) == UNSUP
    assert all(phase(ph, tile=t, T=0) == OK for ph in (0, 1, 2) for t in (0, 1, 2))
    assert phase(0, q=EXACT) == UNSUP and phase(1, q=EXACT) == UNSUP and phase(2, q=EXACT) == UNSUP
    for ph in (0, 1, 2):                   # the same validation as lora_linear_fwd, before any launch
        assert phase(ph, T=0) == OK
        assert phase(ph, x=None) == NULL
        assert phase(ph, ldy=95) == SHAPE
        assert phase(ph, ws=None) == WS
        assert phase(ph, y=W) == OVERLAP
        assert phase(ph, strength=math.nan) == NONFIN


def test_workspace_size():
    ws = rg.lora_linear_workspace_size
    assert ws(32760, 1536, 8960, [64], BF16) == 32760 * 64 * 2
    assert ws(16384, 3072, 9216, [128, 128, 128], BF16) == 16384 * 384 * 2
    assert ws(100, 64, 96, [8, 70], BF16) == 100 * (64 + 128) * 2
    assert ws(64, 128, 96, [8], F32, EXACT) == 64 * 64 * 4
    # lossless fp32 adapter: t~ [T, 3R] bf16, A split [2 r_pad, K] and B split [N, 3 r_pad] bf16 per
    # group, each region rounded up to 256 bytes
    r256 = lambda v: -(-v // 256) * 256
    assert ws(65, 128, 96, [8], F32) == r256(65 * 192 * 2) + r256(2 * 64 * 128 * 2) + r256(96 * 192 * 2)
    assert ws(100, 200, 300, [8, 70], F32) == (r256(100 * 3 * 192 * 2) + r256(2 * 64 * 200 * 2) + r256(300 * 192 * 2)
                                               + r256(2 * 128 * 200 * 2) + r256(300 * 384 * 2))
    # fewer than 128 producer tiles of 128 tokens: K split into S chunks (stages of 64, at least 4 per
    # chunk, at most 8 chunks), fp32 partial sums [S, T, R] after t~ (256-byte aligned)
    assert ws(4352, 8960, 1536, [32], BF16) == r256(4352 * 64 * 2) + 8 * 4352 * 64 * 4
    assert ws(10000, 1536, 8960, [64], BF16) == r256(10000 * 64 * 2) + 4 * 10000 * 64 * 4
    assert ws(18871, 1536, 8960, [64], BF16) == 18871 * 64 * 2          # 148 tiles: no split
    assert ws(16384, 1536, 8960, [64], BF16) == 16384 * 64 * 2          # 128 tiles: no split
    assert ws(4352, 8960, 1536, [32], BF16, EXACT) == 4352 * 64 * 2
    assert ws(0, 128, 96, [8], BF16) == 0
    assert ws(65, 128, 96, [], BF16) == 0
    assert ws(10, 0, 96, [8], BF16) == 0


@pytest.mark.parametrize("T,K,N,ranks", [(1, 4096, 14336, [16]), (16, 1536, 8960, [64]), (64, 8960, 1536, [64]),
                                         (10, 128, 96, []), (33, 3072, 9216, [128, 128, 128]), (64, 64, 96, [8])])
def test_workspace_size_few_tokens(T, K, N, ranks):
    """T <= 64 (lossless): S fp32 partial sums [S, T, round_up(N, 64) + R] with S the header's chunk
    count, or the intermediate's layout when that is larger (the activation dtype is not an argument)."""
    R = sum(-(-r // 64) * 64 for r in ranks)
    row = T * (-(-N // 64) * 64 + R) * 4
    for adt in (BF16, F32):
        got = rg.lora_linear_workspace_size(T, K, N, ranks, adt)
        plain = T * R * (2 if adt == BF16 else 4)
        if adt == F32 and ranks:
            r256 = lambda v: -(-v // 256) * 256
            plain = r256(T * 3 * R * 2) + sum(r256(2 * (-(-r // 64) * 64) * K * 2) + r256(N * 3 * (-(-r // 64) * 64) * 2)
                                              for r in ranks)
        assert got >= plain
        if got != plain or got % row == 0:
            assert got % row == 0 and 1 <= got // row <= -(-K // 64), (got, row)
        if got != plain:  # the partial sums' layout: S as the header defines it
            assert got == _skinny_bytes(T, K, N, R), (got, _skinny_bytes(T, K, N, R))
    assert rg.lora_linear_workspace_size(T, K, N, ranks, BF16, EXACT) == T * R * 2


def stacked(groups, n_groups=None, **kw):
    a = dict(x=X, T=0, K=128, ldx=128, W=W, N=300, bias=None, adt=BF16, strength=1.0, rs=1.0, y=Y, ldy=304,
             act=BF16, q=LOSSLESS, ws=WSP, wsb=1 << 30)
    a.update(kw)
    gs = [rg.LoraGroup(A + i * 0x1000_0000, B + i * 0x1000_0000, r, 0, 1.0, o, n) for i, (r, o, n) in
          enumerate(groups)]
    arr = (rg.LoraGroup * max(1, len(gs)))(*gs)
    return rg._lib.lora_linear_stacked_fwd(a["x"], a["T"], a["K"], a["ldx"], a["W"], a["N"], a["bias"], arr,
                                           len(gs) if n_groups is None else n_groups, a["adt"], a["strength"],
                                           a["rs"], a["y"], a["ldy"], a["act"], a["q"], a["ws"], a["wsb"], None)


def test_stacked_group_validation():
    assert stacked([(8, 0, 100), (8, 100, 100), (8, 200, 100)]) == OK
    assert stacked([(8, 0, 100), (8, 99, 100)]) == SHAPE       # overlapping column ranges
    assert stacked([(8, 250, 100)]) == SHAPE                   # past N_total
    assert stacked([(8, -1, 10)]) == SHAPE
    assert stacked([(8, 0, 0)]) == SHAPE
    assert stacked([(8, 0, 10)] * 2, n_groups=9) == UNSUP
    assert stacked([], n_groups=-1) == SHAPE
    assert stacked([(0, 0, 10)]) == SHAPE


def multi(ads, n=None, **kw):
    a = dict(x=X, T=0, K=128, ldx=128, W=W, N=300, bias=None, adt=BF16, rs=1.0, y=Y, ldy=304, act=BF16,
             q=LOSSLESS, ws=WSP, wsb=1 << 30)
    a.update(kw)
    arr = [rg.LoraAdapter(A + i * 0x1000_0000, B + i * 0x1000_0000, c, r, 0, 8.0, st, o, nc)
           for i, (r, o, nc, st, c) in enumerate(ads)]
    n = len(arr) if n is None else n
    return rg._lib.lora_linear_multi_fwd(a["x"], a["T"], a["K"], a["ldx"], a["W"], a["N"], a["bias"],
                                         (rg.LoraAdapter * max(1, len(arr)))(*arr), n, a["adt"], a["rs"],
                                         a["y"], a["ldy"], a["act"], a["q"], a["ws"], a["wsb"], None)


def test_multi_validation():
    C = BIAS + 0x100
    assert multi([(8, 0, 300, 1.0, None), (16, 0, 300, 0.5, C), (4, 100, 50, 2.0, None)]) == OK  # overlap allowed
    assert multi([(8, 0, 300, 1.0, None)] * 9) == UNSUP
    assert multi([], n=-1) == SHAPE
    assert multi([(8, 0, 301, 1.0, None)]) == SHAPE                  # past N
    assert multi([(8, 0, 300, math.inf, None)]) == NONFIN            # per-adapter strength checked
    assert multi([(8, 0, 300, 1.0, C + 1)]) == ALIGN                 # bf16 bias needs 2-byte alignment
    assert multi([(8, 0, 300, 1.0, Y + 2)], T=4) == OVERLAP          # legacy bias inside the output
    assert multi([(8, 0, 300, 1.0, None)], rs=math.nan) == NONFIN
    # a legacy bias of an active adapter adds an fp32 [N] vector at the front of the workspace
    mk = lambda c, st=1.0: [rg.LoraAdapter(A, B, c, 8, 0, 8.0, st, 0, 300)]
    ws = rg.lora_linear_multi_workspace_size
    plain = rg.lora_linear_workspace_size(4096, 128, 300, [8], BF16)
    assert ws(4096, 128, 300, mk(None), BF16) == plain
    assert ws(4096, 128, 300, mk(C), BF16) == (300 * 4 + 255) // 256 * 256 + plain
    assert ws(4096, 128, 300, mk(C, 0.0), BF16) == plain           # zero strength: inactive
    assert ws(4096, 128, 300, mk(C), BF16, EXACT) == rg.lora_linear_workspace_size(4096, 128, 300, [8], BF16, EXACT)


def _skinny_bytes(T, K, N, ldt):
    """The few-token layout the header documents: S fp32 partial sums [S, T, round_up(N, 64) + ldt],
    S = the number of K chunks (at most 32, each a multiple of 128 of at least 512 elements)."""
    c = -(-K // 32)
    c = max(512, -(-c // 128) * 128)
    S = -(-K // c)
    return S * T * (-(-N // 64) * 64 + ldt) * 4


def test_few_token_workspace_covers_active_subsets():
    """At 64 tokens a call takes the few-token layout when its ACTIVE adapters' padded ranks sum to at
    most 4096; the query, given every adapter's rank, must cover that layout even when all the
    ranks together exceed 4096. 8 adapters of rank 1024, 7 of them at strength 0: sized by the query,
    the call passes the workspace check (it stops at the overlap check that follows, so nothing
    launches)."""
    T, K, N = 64, 8960, 8960
    ranks = [1024] * 8
    need_active = _skinny_bytes(T, K, N, 1024)
    q = rg.lora_linear_workspace_size(T, K, N, ranks, BF16)
    assert q >= _skinny_bytes(T, K, N, 4096) >= need_active
    arr = [rg.LoraAdapter(A + i * 0x1000_0000, B + i * 0x1000_0000, None, 1024, 0, 1024.0,
                          1.0 if i == 3 else 0.0, 0, N) for i in range(8)]
    mq = rg.lora_linear_multi_workspace_size(T, K, N, arr, BF16)
    assert mq >= q
    st = rg._lib.lora_linear_multi_fwd(X, T, K, K, W, N, None, (rg.LoraAdapter * 8)(*arr), 8, BF16, 1.0,
                                       X, N, BF16, LOSSLESS, WSP, mq, None)
    assert st == OVERLAP, st        # (WORKSPACE here would mean the documented query was too small)
    st = rg._lib.lora_linear_multi_fwd(X, T, K, K, W, N, None, (rg.LoraAdapter * 8)(*arr), 8, BF16, 1.0,
                                       X, N, BF16, LOSSLESS, WSP, need_active - 1, None)
    assert st == WS


def merge(**kw):
    a = dict(W=W, wdt=BF16, N=300, K=128, A=A, B=B, rank=8, adt=BF16, alpha=8.0, strength=1.0, q=LOSSLESS)
    a.update(kw)
    return rg._lib.lora_merge_apply(a["W"], a["wdt"], a["N"], a["K"], a["A"], a["B"], a["rank"], a["adt"],
                                    a["alpha"], a["strength"], a["q"], None)


def test_merge_validation():
    assert merge(strength=0.0, N=0) == OK          # empty weight: nothing to do
    assert merge(wdt=7) == DTYPE
    assert merge(q=5) == UNSUP
    assert merge(N=-1) == SHAPE
    assert merge(rank=0) == SHAPE
    assert merge(rank=2000) == UNSUP
    assert merge(alpha=math.nan) == NONFIN
    assert merge(strength=math.inf) == NONFIN
    assert merge(A=None) == NULL
    assert merge(K=100) == ALIGN                    # lossless: K a multiple of 8
    assert merge(W=W + 8) == ALIGN                  # lossless: 16-byte aligned weight
    assert merge(B=W + 0x100) == OVERLAP            # B inside the weight
    assert merge(strength=0.0) == OK                # zero scale: nothing launched


def nf4(**kw):
    a = dict(x=X, T=0, K=128, ldx=128, codes=W, absmax=W + 0x1000_0000, cb=W + 0x2000_0000, bs=64, N=96,
             bias=None, A=A, B=B, rank=16, adt=BF16, alpha=32.0, y=Y, ldy=96, q=LOSSLESS)
    a.update(kw)
    return rg._lib.lora_linear_nf4_fwd(a["x"], a["T"], a["K"], a["ldx"], a["codes"], a["absmax"], a["cb"],
                                       a["bs"], a["N"], a["bias"], a["A"], a["B"], a["rank"], a["adt"],
                                       a["alpha"], 1.0, 1.0, a["y"], a["ldy"], a["q"], WSP, 1 << 30, None)


def test_nf4_workspace_query():
    q = rg.lora_linear_nf4_workspace_size
    # up to 64 tokens (lossless): the skinny partial sums, the weight dequantized in registers
    assert q(64, 256, 300, 16, BF16) == rg.lora_linear_workspace_size(64, 256, 300, [16], BF16)
    assert q(64, 256, 300, 0, BF16) == rg.lora_linear_workspace_size(64, 256, 300, [], BF16) > 0
    assert q(64, 256, 300, 16, BF16, EXACT) == rg.lora_linear_workspace_size(64, 256, 300, [16], BF16, EXACT)
    # from 65 tokens (lossless) a bf16 panel of the weight follows the adapter's share, 256-byte aligned
    ad = rg.lora_linear_workspace_size(65, 256, 300, [16], BF16)
    assert q(65, 256, 300, 16, BF16) == (ad + 255) // 256 * 256 + 300 * 256 * 2
    ad = rg.lora_linear_workspace_size(600, 256, 300, [16], BF16)
    assert q(600, 256, 300, 16, BF16) == (ad + 255) // 256 * 256 + 300 * 256 * 2
    assert q(600, 256, 300, 0, BF16) == 300 * 256 * 2
    assert q(600, 256, 300, 16, BF16, EXACT) == rg.lora_linear_workspace_size(600, 256, 300, [16], BF16, EXACT)
    assert q(0, 256, 300, 16, BF16) == 0


def nf4_ex(dequant, **kw):
    a = dict(x=X, T=0, K=128, ldx=128, codes=W, absmax=W + 0x1000_0000, cb=W + 0x2000_0000, bs=64, N=96,
             bias=None, A=A, B=B, rank=16, adt=BF16, alpha=32.0, y=Y, ldy=96, q=LOSSLESS)
    a.update(kw)
    return rg._lib.lora_linear_nf4_fwd_ex(a["x"], a["T"], a["K"], a["ldx"], a["codes"], a["absmax"], a["cb"],
                                          a["bs"], a["N"], a["bias"], a["A"], a["B"], a["rank"], a["adt"],
                                          a["alpha"], 1.0, 1.0, a["y"], a["ldy"], a["q"], dequant, WSP, 1 << 30,
                                          None)


def test_nf4_dequant_choice_validation():
    for d in (rg.LORA_NF4_AUTO, rg.LORA_NF4_PANEL, rg.LORA_NF4_IN_GEMM):
        assert nf4_ex(d) == OK
        assert nf4_ex(d, adt=F32) in (OK, UNSUP)
    assert nf4_ex(3) == UNSUP and nf4_ex(-1) == UNSUP
    # the in-GEMM form: bf16 adapter with a rank that is a multiple of 8, or no adapter
    assert nf4_ex(rg.LORA_NF4_IN_GEMM, adt=F32) == UNSUP
    assert nf4_ex(rg.LORA_NF4_IN_GEMM, rank=12) == UNSUP
    assert nf4_ex(rg.LORA_NF4_IN_GEMM, A=None, B=None, rank=0) == OK
    assert nf4_ex(rg.LORA_NF4_PANEL, adt=F32) == OK and nf4_ex(rg.LORA_NF4_AUTO, rank=12) == OK
    # the other checks come first, as for lora_linear_nf4_fwd
    assert nf4_ex(rg.LORA_NF4_IN_GEMM, bs=32) == UNSUP
    assert nf4_ex(rg.LORA_NF4_IN_GEMM, K=96, ldx=96) == SHAPE
    assert nf4_ex(rg.LORA_NF4_IN_GEMM, codes=None) == NULL


def test_nf4_validation():
    assert nf4() == OK
    assert nf4(bs=32) == UNSUP
    assert nf4(K=96, ldx=96) == SHAPE
    assert nf4(codes=None) == NULL
    assert nf4(cb=None) == NULL
    assert nf4(absmax=W + 0x1000_0002) == ALIGN


def patch(dshape, sshape, **kw):
    a = dict(dst=X, ddt=BF16, src=W, sdt=BF16, strength=0.8, mode=rg.LORA_PATCH_ADD)
    a.update(kw)
    I64 = rg.ctypes.c_int64
    ds = (I64 * max(1, len(dshape)))(*dshape)
    ss = (I64 * max(1, len(sshape)))(*sshape)
    return rg._lib.dense_patch_apply(a["dst"], a["ddt"], ds, len(dshape), a["src"], a["sdt"], ss, len(sshape),
                                     a["strength"], a["mode"], None)


def test_dense_patch_validation():
    assert patch([0, 5], [0, 5]) == OK                      # empty: nothing to do
    assert patch([3, 4], [4, 3]) == SHAPE                   # full-shape compare, not numel
    assert patch([12], [3, 4]) == SHAPE
    assert patch([3, 4], [3, 4], strength=math.nan) == NONFIN
    assert patch([3, 4], [3, 4], mode=9) == UNSUP
    assert patch([3, 4], [3, 4], ddt=5) == DTYPE
    assert patch([3, 4], [3, 4], src=X + 8) == OVERLAP
    assert patch([3, 4], [3, 4], dst=None) == NULL
    assert patch([3, 4], [3, 4], dst=X + 1) == ALIGN


def test_status_strings():
    for s in range(10):
        assert rg.lora_status_string(s)
    assert "unknown" in rg.lora_status_string(99)


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "rank_gemm_lora_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, flags=re.M), f
                assert "exact_chain" not in text and "lora_oracle" not in text, f


def bwd(**kw):
    a = dict(x=X, T=0, K=128, ldx=128, W=W, N=96, A=A, B=B, rank=8, alpha=8.0, dy=Y, lddy=96, dx=BIAS, lddx=128,
             dA=WSP + 0x1000_0000, dB=WSP + 0x2000_0000, db=WSP + 0x3000_0000, tt=None, ldt=0)
    a.update(kw)
    return rg._lib.lora_linear_bwd(a["x"], a["T"], a["K"], a["ldx"], a["W"], a["N"], a["A"], a["B"], a["rank"],
                                   a["alpha"], 1.0, 1.0, a["dy"], a["lddy"], a["dx"], a["lddx"], a["dA"], a["dB"],
                                   a["db"], a["tt"], a["ldt"], WSP, 1 << 30, None)


def test_backward_forward_t_validation():
    # (T = 0: validation only, nothing launched; rank 8 pads to 64 columns of t~)
    tt = WSP + 0x4000_0000
    assert bwd(dA=None, dB=None, db=None, dx=None, tt=tt, ldt=64) == OK
    assert bwd(dA=None, dB=None, db=None, dx=None, tt=tt, ldt=63) == SHAPE      # fewer columns than the padded rank
    assert bwd(dA=None, dB=None, db=None, dx=None, tt=tt + 1, ldt=64) == ALIGN  # not bf16-aligned
    assert bwd(T=4, dA=None, dB=None, db=tt, dx=None, tt=tt, ldt=64) == OVERLAP  # an output over t~
    assert bwd(T=4, dA=None, dB=None, db=None, dx=None, tt=WSP, ldt=64) == OVERLAP  # t~ inside the workspace


def test_backward_validation():
    assert bwd(dA=None, dB=None, db=None, dx=None) == OK     # (T = 0 with nothing to write)
    assert bwd(rank=0) == SHAPE
    assert bwd(lddy=90) == SHAPE
    assert bwd(N=100, lddy=104) == ALIGN                      # N a multiple of 8
    assert bwd(alpha=math.nan) == NONFIN
    assert bwd(A=None) == NULL
    assert bwd(dx=BIAS, W=None) == NULL                       # dx needs the weight
    assert bwd(dx=None, W=None, dA=None, dB=None, db=None) == OK
    assert bwd(db=X + 64, T=4) == OVERLAP                     # a gradient inside the input
    assert bwd(dB=WSP + 0x3000_0000 - 8, T=4) == OVERLAP      # dB runs into db
    sz = rg.lora_linear_bwd_workspace_size
    assert sz(32760, 1536, 8960, 64) > sz(32760, 1536, 8960, 64, False) > 0   # W^T only with dx
    assert sz(0, 1536, 8960, 64) == 0


def test_noalloc_scratch_size_matches_the_header():
    """The binding's copy of LORA_NOALLOC_SCRATCH_BYTES is the header's value."""
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "lora_mi355x.h")).read()
    m = re.search(r"#define LORA_NOALLOC_SCRATCH_BYTES \((\d+)ull \* 1024ull \* 1024ull\)", hdr)
    assert m is not None
    assert rg.LORA_NOALLOC_SCRATCH_BYTES == int(m.group(1)) * 1024 * 1024
    # the few-token layout of a 64-token call 8960 -> 8960 fits
    assert rg.lora_linear_workspace_size(64, 8960, 8960, [64], BF16) <= rg.LORA_NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("T,K,S", [(129, 512, 2), (129, 768, 3), (129, 1024, 4), (6529, 2048, 5), (5377, 2048, 6),
                                   (4609, 2048, 7), (129, 2048, 8), (16384, 2048, 1)])
def test_producer_split_count_in_the_workspace(T, K, S):
    """The lossless bf16 workspace holds t~ [T, 64] bf16 and, with a producer K split into S parts,
    S fp32 partial sums [S, T, 64] after it (256-byte aligned): the split counts the GPU tests of
    each count expect."""
    r256 = lambda v: -(-v // 256) * 256
    got = rg.lora_linear_workspace_size(T, K, 96, [16], BF16)
    want = T * 64 * 2 if S == 1 else r256(T * 64 * 2) + S * T * 64 * 4
    assert got == want, (got, want)
