"""Benchmark of the fused LoRA linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: the synthetic video-DiT FFN pair at 32760 tokens, rank 64 -- up
projection 1536 -> 8960 (no bias), then down projection 8960 -> 1536 (bias in
the epilogue), alpha 64, strength 1.0, request scale 0.7, bf16, lossless tier.
One step = both layers over one batch, inputs resident in HBM. Prints one JSON
line: fused TFLOP/s (algorithmic FLOPs: 2 T (K N + K r + r N) per layer), the
overhead over the base GEMM alone (min of this library's base-only path and
torch's F.linear), the roofline of the dominant kernel, and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "fused LoRA-linear TFLOP/s + % overhead vs base GEMM (tokens=32760, r=64)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fused_gemm_ffn_pair.json")
KERNEL_SOURCES = ["rank_gemm_lora_amd/csrc/gemm.hip", "rank_gemm_lora_amd/csrc/common.hpp",
                  "rank_gemm_lora_amd/csrc/launch.hpp"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def layer_flops(T, K, N, r):
    return 2.0 * T * (K * N + K * r + r * N)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the per-config measurements of the other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters) and exit")
    ap.add_argument("--layer-only", action="store_true",
                    help="only run the timed fused steps (for counter collection) and exit")
    ap.add_argument("--workload", choices=["attn_proj", "qkv_bf16", "qkv_f32", "nf4_layer", "nf4_layer_in_gemm",
                                           "nf4_tokens256", "multi_ffn_up", "few_ffn_up", "few_ffn_down", "nf4_vector",
                                           "backward_ffn_up", "backward_ffn_down"],
                    help="only run this workload's fused call (--warmup + --steps times; for counter runs) and exit")
    ap.add_argument("--write-traffic", metavar="DIR",
                    help="turn the four counter runs in DIR (f/, w/: FETCH_SIZE / WRITE_SIZE of --layer-only; "
                         "cf/, cw/: the same of --copy-probe) into the traffic file and exit")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.write_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs a layer on a single MI355X "
              "(token-parallel sharding of a layer needs no collective). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.copy_probe:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": src.numel() * 2, "launches": 3}), flush=True)
        return

    if args.workload:
        run_workload(torch, dev, args.workload, args.warmup, args.steps)
        return

    import lora_workloads as lw
    import rank_gemm_lora_amd as rg
    t0 = time.time()
    up_h, down_h = lw.ffn_pair_inputs()
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    layers = []
    for spec, h in ((lw.FFN_UP, up_h), (lw.FFN_DOWN, down_h)):
        d = {k: (v.to(dev) if hasattr(v, "to") else v) for k, v in h.items()}
        T, K, N, r = spec.T, spec.K, spec.N, spec.rank
        y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(1, rg.lora_linear_workspace_size(T, K, N, [r], rg.LORA_BF16)), dtype=torch.uint8, device=dev)
        layers.append(dict(spec=spec, d=d, y=y, ws=ws, T=T, K=K, N=N, r=r))
    del up_h, down_h
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def call(L, lora=True, phase=0):
        d = L["d"]
        args = (d["x"].data_ptr(), L["T"], L["K"], L["K"], d["W"].data_ptr(), L["N"],
                None if d["b"] is None else d["b"].data_ptr(),
                d["A"].data_ptr() if lora else None, d["B"].data_ptr() if lora else None,
                L["r"], rg.LORA_BF16, d["alpha"], d["strength"], d["request_scale"],
                L["y"].data_ptr(), L["N"], rg.LORA_BF16, rg.LORA_LOSSLESS,
                L["ws"].data_ptr(), L["ws"].numel(), sp)
        if phase == 0:
            rg.lora_linear_fwd(*args)
        else:
            rg.lora_linear_fwd_phase(phase, 0, *args)

    def step():
        for L in layers:
            call(L)

    # ---------------- timed region: K steps of the library call, events only around it
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps

    # ---------------- per-kernel pass (for the roofline): K more steps, each layer call
    # split into its two launches (phase 1: rank-wide producer, phase 2: fused GEMM) with an
    # event recorded after each on the launch stream
    n_ev = args.steps * len(layers) * 2 + 1
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    i = 0
    evs[0].record(stream)
    for _ in range(args.steps):
        for L in layers:
            for ph in (1, 2):
                call(L, phase=ph)
                i += 1
                evs[i].record(stream)
    torch.cuda.synchronize()
    prod_ms = [0.0] * len(layers)   # per launch, averaged over the steps
    gemm_ms = [0.0] * len(layers)
    for s_ in range(args.steps):
        for li in range(len(layers)):
            k = (s_ * len(layers) + li) * 2
            prod_ms[li] += evs[k].elapsed_time(evs[k + 1]) / args.steps
            gemm_ms[li] += evs[k + 1].elapsed_time(evs[k + 2]) / args.steps
    if args.layer_only:
        # the per-launch means a kernel trace of this process reports for the per-kernel pass
        print(json.dumps({"ms_per_step": round(ms_per_step, 4), "timed_steps": args.steps,
                          "warmup_steps": args.warmup,
                          "gemm_ms_per_launch": [round(x, 4) for x in gemm_ms],
                          "producer_ms_per_launch": [round(x, 4) for x in prod_ms]}), flush=True)
        return

    flops = [layer_flops(L["T"], L["K"], L["N"], L["r"]) for L in layers]
    step_flops = sum(flops)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    # ---------------- base GEMM alone: own base-only path and torch F.linear (hipBLASLt)
    # The overhead compares like with like: a base step is both layers' base GEMMs back to back,
    # as the fused step runs them (so each layer finds the caches as the other layer left them: the
    # 587 MB input of the down layer flushes the up layer's operands from the 256 MB Infinity
    # Cache), once per choice of base path per layer (this library's base-only call or
    # hipBLASLt), the fastest choice kept. Every variant is timed the same way (back-to-back loops
    # of 10 steps between two events on the stream) in 5 interleaved rounds, keeping the median
    # round. Per-layer base times (each layer alone in a loop) are reported beside it.
    def loop_ms(fn, n=10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    F = torch.nn.functional
    base_fn = [[(lambda L=L: call(L, lora=False)), (lambda L=L: F.linear(L["d"]["x"], L["d"]["W"], L["d"]["b"]))]
               for L in layers]
    fns = {"fused_step": step}
    for c0 in (0, 1):
        for c1 in (0, 1):
            fns[f"base_{c0}{c1}"] = (lambda c0=c0, c1=c1: (base_fn[0][c0](), base_fn[1][c1]()))
    for li in range(len(layers)):
        fns[f"own{li}"] = base_fn[li][0]
        fns[f"torch{li}"] = base_fn[li][1]
    for fn in fns.values():
        fn()
    torch.cuda.synchronize()
    rounds = {k: [] for k in fns}
    for _ in range(5):
        for k, fn in fns.items():
            rounds[k].append(loop_ms(fn))
    med = {k: sorted(v)[len(v) // 2] for k, v in rounds.items()}
    base = [dict(own_ms=med[f"own{li}"], torch_ms=med[f"torch{li}"],
                 min_ms=min(med[f"own{li}"], med[f"torch{li}"])) for li in range(len(layers))]
    base_key = min((k for k in med if k.startswith("base_")), key=lambda k: med[k])
    base_ms = med[base_key]
    overhead = med["fused_step"] / base_ms - 1.0
    base_choice = ["own" if base_key[5 + li] == "0" else "hipblaslt" for li in range(len(layers))]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    probe = mfma_probe(torch, stream, cus)

    # ---------------- roofline of the dominant kernel: the fused GEMM (phase 2)
    # algorithmic FLOPs per launch 2 T (K N + r N); the producer (phase 1) is HBM-bound:
    # algorithmic bytes per launch = x once (T K 2) + A (r K 2) + t~ written (T r_pad 2)
    gemm_flops = [2.0 * L["T"] * (L["K"] * L["N"] + L["r"] * L["N"]) for L in layers]
    achieved = sum(gemm_flops) / (sum(gemm_ms) * 1e-3) / 1e12
    prod_bytes = [2.0 * (L["T"] * L["K"] + L["r"] * L["K"] + L["T"] * ((L["r"] + 63) // 64 * 64)) for L in layers]
    prod_gbs = sum(prod_bytes) / (sum(prod_ms) * 1e-3) / 1e9
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_hash") == kernel_hash():
            traffic = tr.get("bytes_per_launch")
    except FileNotFoundError:
        pass
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": "fused LoRA GEMM (gemm_flow16_kernel), FFN up + down launches",
                "per_launch_ms": [round(x, 4) for x in gemm_ms],
                "producer": {"bound": "hbm", "achieved": round(prod_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(prod_gbs / PEAK_HBM_GBS, 4),
                             "per_launch_ms": [round(x, 4) for x in prod_ms]}}

    # ---------------- CPU oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layers, args.cpu_seconds)

    # ---------------- every other workload: fused time, base time, roofline, oracle beside it
    layer_cfg = [{"in": L["K"], "out": L["N"], "rank": L["r"], "bias": L["d"]["b"] is not None} for L in layers]
    layers_meta = [{"K": L["K"], "N": L["N"]} for L in layers]
    configs = None
    if not args.headline_only:
        del layers, L, d
        torch.cuda.empty_cache()
        configs = config_sweep(torch, dev, stream, with_oracle=not args.no_cpu_baseline)
        torch.cuda.empty_cache()
        configs["token_regimes"] = token_regimes(torch, dev, with_oracle=not args.no_cpu_baseline)

    per_layer = [{"layer": f"{L['K']}->{L['N']}", "producer_ms": round(p_, 4), "gemm_ms": round(g_, 4),
                  "base_own_ms": round(b_["own_ms"], 4), "base_hipblaslt_ms": round(b_["torch_ms"], 4)}
                 for L, p_, g_, b_ in zip(layers_meta, prod_ms, gemm_ms, base)]
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s",
        "overhead_vs_base": round(overhead, 4), "base_ms": round(base_ms, 4),
        "fused_step_ms_same_timing": round(med["fused_step"], 4), "base_step_choice": base_choice,
        "overhead_vs_per_layer_base": round(med["fused_step"] / sum(b["min_ms"] for b in base) - 1.0, 4),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "ffn_pair_tokens32760_rank64", "tokens": 32760, "layers": layer_cfg,
                   "alpha": 64.0, "strength": 1.0, "request_scale": 0.7, "quality": "lossless"},
        "per_layer": per_layer,
        "pct_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "mfma_ceiling": probe,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if configs is not None:
        # the other workloads: one JSON line of their own on stderr (stdout carries the headline only)
        print(json.dumps({"configs": configs}), file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


def run_workload(torch, dev, name, warmup, steps):
    """One workload's fused call, warmup + steps times on the current stream (for rocprofv3 runs);
    prints the mean launch time of the timed steps."""
    import lora_workloads as lw
    import rank_gemm_lora_amd as rg
    d2 = lambda t: None if t is None else t.to(dev)
    if name == "attn_proj":
        h = lw.linear_inputs(lw.ATTN_PROJ)
        x, W, b, A, B = (d2(h[k]) for k in ("x", "W", "b", "A", "B"))
        sp = lw.ATTN_PROJ
        y = torch.empty((sp.T, sp.N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(rg.lora_linear_workspace_size(sp.T, sp.K, sp.N, [sp.rank], rg.LORA_BF16), dtype=torch.uint8,
                         device=dev)
        fn = lambda: rg.lora_linear(x, W, b, A, B, sp.alpha, sp.strength, sp.request_scale, out=y, workspace=ws)
    elif name in ("qkv_bf16", "qkv_f32"):
        sp = lw.QKV_STACKED if name == "qkv_bf16" else dataclasses.replace(lw.QKV_STACKED, adapter="f32",
                                                                           name="qkv_stacked_f32")
        h = lw.stacked_inputs(sp)
        x, W, b = d2(h["x"]), d2(h["W"]), d2(h["b"])
        groups = [dict(g, A=d2(g["A"]), B=d2(g["B"])) for g in h["groups"]]
        Nt = sum(sp.n_cols)
        adt = rg.LORA_F32 if name == "qkv_f32" else rg.LORA_BF16
        y = torch.empty((sp.T, Nt), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(rg.lora_linear_workspace_size(sp.T, sp.K, Nt, list(sp.ranks), adt), dtype=torch.uint8,
                         device=dev)
        fn = lambda: rg.lora_linear_stacked(x, W, b, groups, sp.strength, sp.request_scale, out=y, workspace=ws)
    elif name in ("nf4_layer", "nf4_layer_in_gemm", "nf4_tokens256"):
        # the 4-bit layer as configured (the automatic choice: the panel at 8192 tokens), the same
        # with the weight dequantized inside the GEMM, and its first 256 tokens (automatic: in the GEMM)
        sp = lw.NF4_LAYER
        h = lw.nf4_inputs(sp)
        x, codes, absmax, cb, A, B, b = (d2(h[k]) for k in ("x", "codes", "absmax", "codebook", "A", "B", "b"))
        T = 256 if name == "nf4_tokens256" else sp.T
        x = x[:T]
        dq = "in_gemm" if name == "nf4_layer_in_gemm" else "auto"
        y = torch.empty((T, sp.N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(rg.lora_linear_nf4_workspace_size(T, sp.K, sp.N, sp.rank, rg.LORA_BF16),
                         dtype=torch.uint8, device=dev)
        fn = lambda: rg.lora_linear_nf4(x, codes, absmax, cb, sp.N, b, A, B, sp.alpha, sp.strength,
                                        sp.request_scale, out=y, workspace=ws, dequant=dq)
    elif name in ("few_ffn_up", "few_ffn_down"):  # 64 tokens: the few-token kernel and its finishing kernel
        sp = lw.FEW_FFN_UP if name == "few_ffn_up" else lw.FEW_FFN_DOWN
        h = lw.linear_inputs(sp)
        x, W, b, A, B = (d2(h[k]) for k in ("x", "W", "b", "A", "B"))
        y = torch.empty((sp.T, sp.N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(rg.lora_linear_workspace_size(sp.T, sp.K, sp.N, [sp.rank], rg.LORA_BF16), dtype=torch.uint8,
                         device=dev)
        fn = lambda: rg.lora_linear(x, W, b, A, B, sp.alpha, sp.strength, sp.request_scale, out=y, workspace=ws)
    elif name == "nf4_vector":  # one token through the 4-bit weight (dequantized in registers)
        sp = lw.NF4_VECTOR
        h = lw.nf4_inputs(sp)
        x, codes, absmax, cb, A, B, b = (d2(h[k]) for k in ("x", "codes", "absmax", "codebook", "A", "B", "b"))
        y = torch.empty((sp.T, sp.N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(1, rg.lora_linear_nf4_workspace_size(sp.T, sp.K, sp.N, sp.rank, rg.LORA_BF16)),
                         dtype=torch.uint8, device=dev)
        fn = lambda: rg.lora_linear_nf4(x, codes, absmax, cb, sp.N, b, A, B, sp.alpha, sp.strength,
                                        sp.request_scale, out=y, workspace=ws)
    elif name in ("backward_ffn_up", "backward_ffn_down"):  # dx, dA, dB, db with t~ from the forward call
        up_h, down_h = lw.ffn_pair_inputs()
        sp, h = (lw.FFN_UP, up_h) if name == "backward_ffn_up" else (lw.FFN_DOWN, down_h)
        del up_h, down_h
        x, W, A, B = d2(h["x"]), d2(h["W"]), d2(h["A"]), d2(h["B"])
        T, K, N, r = sp.T, sp.K, sp.N, sp.rank
        dy = torch.randn((T, N), device=dev, generator=torch.Generator(device=dev).manual_seed(17)).to(torch.bfloat16)
        ws = torch.empty(max(1, rg.lora_linear_bwd_workspace_size(T, K, N, r)), dtype=torch.uint8, device=dev)
        outs = (torch.empty((T, K), dtype=torch.bfloat16, device=dev), torch.empty((r, K), device=dev),
                torch.empty((N, r), device=dev), torch.empty((N,), device=dev))
        fws = torch.empty(max(1, rg.lora_linear_workspace_size(T, K, N, [r], rg.LORA_BF16)), dtype=torch.uint8,
                          device=dev)
        rg.lora_linear(x, W, d2(h["b"]), A, B, sp.alpha, sp.strength, sp.request_scale, workspace=fws)
        rp = -(-r // 64) * 64
        sid = torch.cuda.current_stream().cuda_stream
        fn = lambda: rg.lora_linear_bwd(x.data_ptr(), T, K, K, W.data_ptr(), N, A.data_ptr(), B.data_ptr(), r,
                                        sp.alpha, sp.strength, sp.request_scale, dy.data_ptr(), N,
                                        outs[0].data_ptr(), K, outs[1].data_ptr(), outs[2].data_ptr(),
                                        outs[3].data_ptr(), fws.data_ptr(), rp, ws.data_ptr(), ws.numel(), sid)
    else:  # multi_ffn_up
        sp = lw.MULTI_FFN_UP
        h = lw.multi_inputs(sp)
        x, W, b = d2(h["x"]), d2(h["W"]), d2(h["b"])
        ads = [dict(a, A=d2(a["A"]), B=d2(a["B"]), c=d2(a["c"])) for a in h["adapters"]]
        y = torch.empty((sp.T, sp.N), dtype=torch.bfloat16, device=dev)
        fn = lambda: rg.lora_linear_multi(x, W, b, ads, sp.request_scale, out=y)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    e.record(stream)
    torch.cuda.synchronize()
    print(json.dumps({"workload": name, "steps": steps, "ms_per_call": round(a.elapsed_time(e) / max(steps, 1), 4)}),
          flush=True)


def _launch_stats(torch, stream, fn, n=100, warm=10):
    """Median, p10 and p90 (ms) of n launches of fn, each between its own pair of events."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return {"median": round(t[n // 2], 5), "p10": round(t[n // 10], 5), "p90": round(t[(9 * n) // 10], 5)}


def _graph_stats(torch, fn, out, n=50, reps=5):
    """GPU time (ms) of one call of fn, replayed from a captured HIP graph (no host time per
    call): median, p10, p90 over `reps` batches of n replays. Before timing, three replays
    each separated by eager work are checked bit for bit against the eager result in `out`."""
    fn()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise RuntimeError("graph replay differs from the eager call")
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / n)
    ts.sort()
    return {"median": round(ts[len(ts) // 2], 5), "p10": round(ts[0], 5), "p90": round(ts[-1], 5),
            "timing": f"HIP graph replay, {reps} x {n}"}


def token_regimes(torch, dev, with_oracle=True):
    """The pages' other token regimes: Z-Image-Turbo (4352 tokens, rank 32: attention
    projection and FFN pair), MiniMax-H3 per rank (18871 tokens, rank 64: FFN pair), a
    64-token FFN pair and the single-vector 4-bit layer. Each call is timed by graph replay
    (fused, this library's base-only path, torch F.linear); MFMA-bound entries report
    TFLOP/s, the few-token ones HBM GB/s on the algorithmic bytes."""
    import lora_workloads as lw
    import rank_gemm_lora_amd as rg
    F = torch.nn.functional
    out = {}

    def d2(t):
        return None if t is None else t.to(dev)

    def entry(name, spec, h):
        x, W, b, A, B = (d2(h[k]) for k in ("x", "W", "b", "A", "B"))
        T, K, N, r = spec.T, spec.K, spec.N, spec.rank
        y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(1, rg.lora_linear_workspace_size(T, K, N, [r], rg.LORA_BF16)), dtype=torch.uint8,
                         device=dev)
        fused = _graph_stats(torch, lambda: rg.lora_linear(x, W, b, A, B, spec.alpha, spec.strength,
                                                            spec.request_scale, out=y, workspace=ws), y)
        own = _graph_stats(torch, lambda: rg.lora_linear(x, W, b, None, None, 1.0, out=y, workspace=ws), y)["median"]
        yt = torch.empty_like(y)
        tor = _graph_stats(torch, lambda: yt.copy_(F.linear(x, W, b)), yt)["median"]
        byt = 2 * (T * K + N * K + T * N + (N if b is not None else 0) + r * (K + N))
        fl = 2.0 * T * (K * N + K * r + r * N)
        e = _gemm_entry(fl, fused, own, tor, byt)
        e["workload"] = f"{name}: T={T} K={K} N={N} r={r} bf16/bf16"
        if T <= 64:
            gbs = byt / (fused["median"] * 1e-3) / 1e9
            e.update(bound="hbm", achieved_gbs=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4))
        if with_oracle:
            e["cpu_oracle"] = _oracle_time(lambda: _oracle_linear(h, spec), fl)
        return e

    out["zimage_attn"] = entry("Z-Image attention projection", lw.ZIMAGE_ATTN, lw.linear_inputs(lw.ZIMAGE_ATTN))
    for tag, (su, sd) in (("zimage", (lw.ZIMAGE_FFN_UP, lw.ZIMAGE_FFN_DOWN)), ("h3", (lw.H3_FFN_UP, lw.H3_FFN_DOWN)),
                          ("few", (lw.FEW_FFN_UP, lw.FEW_FFN_DOWN))):
        hu, hd = lw.ffn_pair_inputs(su, sd)
        out[f"{tag}_ffn_up"] = entry(f"{tag} FFN up", su, hu)
        out[f"{tag}_ffn_down"] = entry(f"{tag} FFN down", sd, hd)
        del hu, hd
        torch.cuda.empty_cache()

    spec = lw.NF4_VECTOR
    h = lw.nf4_inputs(spec)
    x, codes, absmax, cb, A, B, b = (d2(h[k]) for k in ("x", "codes", "absmax", "codebook", "A", "B", "b"))
    T, K, N, r = spec.T, spec.K, spec.N, spec.rank
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, rg.lora_linear_nf4_workspace_size(T, K, N, r, rg.LORA_BF16)), dtype=torch.uint8,
                     device=dev)
    fused = _graph_stats(torch, lambda: rg.lora_linear_nf4(x, codes, absmax, cb, N, b, A, B, spec.alpha, out=y,
                                                            workspace=ws), y)
    own = _graph_stats(torch, lambda: rg.lora_linear_nf4(x, codes, absmax, cb, N, b, None, None, spec.alpha,
                                                          out=y, workspace=ws), y)["median"]
    byt = 2 * (T * K + T * N) + N * K // 2 + 4 * (N * K // spec.blocksize) + 2 * r * (K + N)
    gbs = byt / (fused["median"] * 1e-3) / 1e9
    e = _gemm_entry(2.0 * T * (K * N + K * r + r * N), fused, own, None, byt)
    e.update(workload=f"4-bit weight, single vector: T={T} K={K} N={N} r={r}", bound="hbm",
             achieved_gbs=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4),
             note="overhead against the 4-bit base path")
    out["nf4_vector"] = e
    return out


def _gemm_entry(flops, ms, base_own, base_torch, bytes_alg):
    """TFLOP/s, share of the bf16 MFMA peak and overhead over the faster base path."""
    tf = flops / (ms["median"] * 1e-3) / 1e12
    base = min(b for b in (base_own, base_torch) if b is not None)
    return {"tflops": round(tf, 1), "pct_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "ms": ms, "base_ms": {"own": base_own, "torch": base_torch},
            "overhead_vs_base": round(ms["median"] / base - 1.0, 4), "bound": "mfma",
            "algorithmic_flop": flops, "algorithmic_bytes": bytes_alg}


def config_sweep(torch, dev, stream, with_oracle=True):
    """The other workloads of the method at their full sizes, each timed over 100 launches
    (median, p10, p90): attention projection, stacked q/k/v (bf16 and fp32 adapters), the
    4-bit layer, the dense patches and the tiny fp32 layer. FLOPs count what the method
    computes (2 T (K N + K r + r N) per adapter layer), bytes each tensor once."""
    import lora_workloads as lw
    import rank_gemm_lora_amd as rg
    F = torch.nn.functional
    out = {}

    def d2(t):
        return None if t is None else t.to(dev)

    def linear_case(spec, tag):
        h = lw.linear_inputs(spec)
        x, W, b, A, B = (d2(h[k]) for k in ("x", "W", "b", "A", "B"))
        T, K, N, r = spec.T, spec.K, spec.N, spec.rank
        y = torch.empty((T, N), dtype=x.dtype, device=dev)
        adt = rg.LORA_F32 if spec.adapter == "f32" else rg.LORA_BF16
        ws = torch.empty(max(1, rg.lora_linear_workspace_size(T, K, N, [r], adt)), dtype=torch.uint8, device=dev)
        fused = _launch_stats(torch, stream, lambda: rg.lora_linear(x, W, b, A, B, spec.alpha, spec.strength,
                                                                     spec.request_scale, out=y, workspace=ws))
        own = _launch_stats(torch, stream, lambda: rg.lora_linear(x, W, b, None, None, spec.alpha, out=y,
                                                                   workspace=ws))["median"]
        tor = _launch_stats(torch, stream, lambda: F.linear(x, W, b))["median"]
        esz = x.element_size()
        byt = esz * (T * K + N * K + T * N + (N if b is not None else 0)) + A.element_size() * r * (K + N)
        e = _gemm_entry(2.0 * T * (K * N + K * r + r * N), fused, own, tor, byt)
        e["workload"] = f"{tag}: T={T} K={K} N={N} r={r} {spec.act}/{spec.adapter}"
        if with_oracle:
            e["cpu_oracle"] = _oracle_time(lambda: _oracle_linear(h, spec), e["algorithmic_flop"])
        return e

    out["attn_proj"] = linear_case(lw.ATTN_PROJ, "attention projection")
    torch.cuda.empty_cache()

    for adapter in ("bf16", "f32"):
        spec = lw.QKV_STACKED if adapter == "bf16" else dataclasses.replace(lw.QKV_STACKED, adapter="f32",
                                                                           name="qkv_stacked_f32")
        h = lw.stacked_inputs(spec)
        x, W, b = d2(h["x"]), d2(h["W"]), d2(h["b"])
        groups = [dict(g, A=d2(g["A"]), B=d2(g["B"])) for g in h["groups"]]
        T, K = spec.T, spec.K
        Nt = sum(spec.n_cols)
        y = torch.empty((T, Nt), dtype=x.dtype, device=dev)
        adt = rg.LORA_F32 if adapter == "f32" else rg.LORA_BF16
        ws = torch.empty(max(1, rg.lora_linear_workspace_size(T, K, Nt, list(spec.ranks), adt)), dtype=torch.uint8,
                         device=dev)
        fused = _launch_stats(torch, stream, lambda: rg.lora_linear_stacked(x, W, b, groups, spec.strength,
                                                                             spec.request_scale, out=y, workspace=ws))
        own = _launch_stats(torch, stream, lambda: rg.lora_linear(x, W, b, None, None, 1.0, out=y,
                                                                   workspace=ws))["median"]
        tor = _launch_stats(torch, stream, lambda: F.linear(x, W, b))["median"]
        fl = 2.0 * T * (K * Nt + sum(r * (K + n) for r, n in zip(spec.ranks, spec.n_cols)))
        esz = 4 if adapter == "f32" else 2
        byt = 2 * (T * K + Nt * K + T * Nt) + esz * sum(r * (K + n) for r, n in zip(spec.ranks, spec.n_cols))
        e = _gemm_entry(fl, fused, own, tor, byt)
        e["workload"] = f"stacked q/k/v: T={T} K={K} N=3x3072 r=3x128 bf16/{adapter}"
        if adapter == "f32":
            e["note"] = ("the fp32 adapter products run on bf16 MFMA over a hi/lo bf16 split of the fp32 values "
                         "(x.hi(A) + x.lo(A), then a rank-3r K-extension); about 2^-16 relative to fp32 products")
        if with_oracle:
            e["cpu_oracle"] = _oracle_time(lambda: _oracle_stacked(h, spec), fl)
        out["qkv_stacked_" + adapter] = e
        del x, W, b, groups, y, ws, h
        torch.cuda.empty_cache()

    spec = lw.MULTI_FFN_UP
    h = lw.multi_inputs(spec)
    x, W, b = d2(h["x"]), d2(h["W"]), d2(h["b"])
    ads = [dict(a, A=d2(a["A"]), B=d2(a["B"]), c=d2(a["c"])) for a in h["adapters"]]
    T, K, N = spec.T, spec.K, spec.N
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    cads = [rg.LoraAdapter(a["A"].data_ptr(), a["B"].data_ptr(), 0 if a["c"] is None else a["c"].data_ptr(),
                           a["rank"], 0, a["alpha"], a["strength"], a["col_offset"], a["n_cols"]) for a in ads]
    ws = torch.empty(max(1, rg.lora_linear_multi_workspace_size(T, K, N, cads, rg.LORA_BF16)), dtype=torch.uint8,
                     device=dev)
    fused = _launch_stats(torch, stream, lambda: rg.lora_linear_multi(x, W, b, ads, spec.request_scale, out=y,
                                                                       workspace=ws))
    own = _launch_stats(torch, stream, lambda: rg.lora_linear(x, W, b, None, None, 1.0, out=y,
                                                               workspace=ws))["median"]
    tor = _launch_stats(torch, stream, lambda: F.linear(x, W, b))["median"]
    rs = [a["rank"] for a in ads]
    fl = 2.0 * T * (K * N + sum(r * (K + a["n_cols"]) for r, a in zip(rs, ads)))
    byt = 2 * (T * K + N * K + T * N) + 2 * sum(r * (K + a["n_cols"]) + a["n_cols"] for r, a in zip(rs, ads))
    e = _gemm_entry(fl, fused, own, tor, byt)
    e["workload"] = (f"two adapters on one layer: T={T} K={K} N={N}, r=64 (strength 1) + r=32 (strength 0.5, "
                     f"legacy lora_B bias)")
    if with_oracle:
        e["cpu_oracle"] = _oracle_time(lambda: _oracle_multi(h, spec), fl)
    out["multi_ffn_up"] = e
    del x, W, b, ads, y, ws, h
    torch.cuda.empty_cache()

    spec = lw.NF4_LAYER
    h = lw.nf4_inputs(spec)
    x, codes, absmax, cb, A, B, b = (d2(h[k]) for k in ("x", "codes", "absmax", "codebook", "A", "B", "b"))
    T, K, N, r = spec.T, spec.K, spec.N, spec.rank
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, rg.lora_linear_nf4_workspace_size(T, K, N, r, rg.LORA_BF16)), dtype=torch.uint8,
                     device=dev)
    fused = _launch_stats(torch, stream, lambda: rg.lora_linear_nf4(x, codes, absmax, cb, N, b, A, B, spec.alpha,
                                                                     out=y, workspace=ws))
    own = _launch_stats(torch, stream, lambda: rg.lora_linear_nf4(x, codes, absmax, cb, N, b, None, None,
                                                                   spec.alpha, out=y, workspace=ws))["median"]
    # hipBLASLt on the same GEMM with the weight already dequantized to bf16 (plain torch ops)
    c = codes.to(torch.int64)
    idx = torch.stack((c & 15, c >> 4), dim=-1).reshape(N, K)
    W_deq = (cb[idx] * absmax.repeat_interleave(spec.blocksize).reshape(N, K)).to(torch.bfloat16)
    del c, idx
    tor = _launch_stats(torch, stream, lambda: F.linear(x, W_deq, b))["median"]
    byt = 2 * (T * K + T * N) + N * K // 2 + 4 * (N * K // spec.blocksize) + 2 * r * (K + N)
    e = _gemm_entry(2.0 * T * (K * N + K * r + r * N), fused, own, None, byt)
    e["workload"] = f"4-bit weight: T={T} K={K} N={N} r={r}, codebook + fp32 absmax per 64"
    e["bf16_hipblaslt_ms"] = tor
    # the weight dequantized inside the GEMM instead of once into the panel (the same output bits)
    e["in_gemm_ms"] = _launch_stats(torch, stream, lambda: rg.lora_linear_nf4(
        x, codes, absmax, cb, N, b, A, B, spec.alpha, out=y, workspace=ws, dequant="in_gemm"))["median"]
    # the first 256 tokens of the layer: the automatic choice is the in-GEMM form there
    x256, y256 = x[:256], y[:256]
    e["tokens256"] = {m + "_ms": _launch_stats(torch, stream, lambda: rg.lora_linear_nf4(
        x256, codes, absmax, cb, N, b, A, B, spec.alpha, out=y256, workspace=ws, dequant=m))["median"]
        for m in ("in_gemm", "panel")}
    e["note"] = ("overhead against the 4-bit base path (torch has no 4-bit GEMM); bf16_hipblaslt_ms: "
                 "hipBLASLt on the same GEMM with the weight dequantized to bf16 beforehand, for context")
    if with_oracle:
        e["cpu_oracle"] = _oracle_time(lambda: _oracle_nf4(h, spec), e["algorithmic_flop"])
    out["nf4_layer"] = e
    del x, codes, absmax, cb, A, B, b, y, ws, W_deq
    torch.cuda.empty_cache()

    for spec in (lw.PATCH_WEIGHT, lw.PATCH_NORM):
        h = lw.patch_inputs(spec)
        dst, diff = d2(h["dst"]), d2(h["diff"])
        n = dst.numel()
        for mode in ("add", "replace"):
            ms = _launch_stats(torch, stream, lambda: rg.dense_patch(dst, diff, spec.strength, mode))
            byt = (3 if mode == "add" else 2) * n * 2
            gbs = byt / (ms["median"] * 1e-3) / 1e9
            e = {"workload": f"dense patch {mode}: shape={list(spec.shape)} bf16", "ms": ms,
                 "bound": "hbm" if n > 1 << 20 else "launch latency", "achieved_gbs": round(gbs, 1),
                 "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": byt}
            if with_oracle and mode == "add":
                e["cpu_oracle"] = _oracle_time(lambda: _oracle_patch(h, spec), None, byt)
            out[f"{spec.name}_{mode}"] = e
        del dst, diff, h
        torch.cuda.empty_cache()

    # backward of the FFN pair (dx, dA, dB, db), against hipBLASLt's dy.W alone
    up_h, down_h = lw.ffn_pair_inputs()
    for spec, h in ((lw.FFN_UP, up_h), (lw.FFN_DOWN, down_h)):
        x, W, A, B = d2(h["x"]), d2(h["W"]), d2(h["A"]), d2(h["B"])
        T, K, N, r = spec.T, spec.K, spec.N, spec.rank
        dy = torch.randn((T, N), device=dev, generator=torch.Generator(device=dev).manual_seed(17)).to(torch.bfloat16)
        ws = torch.empty(max(1, rg.lora_linear_bwd_workspace_size(T, K, N, r)), dtype=torch.uint8, device=dev)
        outs = (torch.empty((T, K), dtype=torch.bfloat16, device=dev), torch.empty((r, K), device=dev),
                torch.empty((N, r), device=dev), torch.empty((N,), device=dev))
        sp = stream.cuda_stream
        # the forward call of the same layer (untimed): its workspace starts with t~ [T, rank_pad]
        rp = -(-r // 64) * 64
        fws = torch.empty(max(1, rg.lora_linear_workspace_size(T, K, N, [r], rg.LORA_BF16)), dtype=torch.uint8,
                          device=dev)
        rg.lora_linear(x, W, d2(h["b"]), A, B, spec.alpha, spec.strength, spec.request_scale, workspace=fws)

        def bwd(t_tilde):
            rg.lora_linear_bwd(x.data_ptr(), T, K, K, W.data_ptr(), N, A.data_ptr(), B.data_ptr(), r, spec.alpha,
                               spec.strength, spec.request_scale, dy.data_ptr(), N, outs[0].data_ptr(), K,
                               outs[1].data_ptr(), outs[2].data_ptr(), outs[3].data_ptr(), t_tilde,
                               rp if t_tilde else 0, ws.data_ptr(), ws.numel(), sp)
        ms = _launch_stats(torch, stream, lambda: bwd(fws.data_ptr()), n=30)
        ms_re = _launch_stats(torch, stream, lambda: bwd(None), n=30)
        tor = _launch_stats(torch, stream, lambda: torch.matmul(dy, W), n=30)["median"]
        fl = 2.0 * T * (N * K + 2 * N * r + 3 * r * K)
        byt = 2 * (2 * T * N + 2 * T * K + N * K + r * (N + K)) + 4 * (r * K + N * r + N)
        e = _gemm_entry(fl, ms, None, tor, byt)
        e["workload"] = (f"backward (dx, dA, dB, db): T={T} K={K} N={N} r={r}, t~ taken from the forward call's "
                         f"workspace; base = hipBLASLt dy.W (dx without the adapter)")
        e["ms_recomputing_t"] = ms_re
        out[f"backward_{spec.name}"] = e
        del x, W, A, B, dy, ws, outs, fws
    del up_h, down_h
    torch.cuda.empty_cache()

    # merge W <- W + s.B.A (merge mode): HBM-bound rewrite of the weight; and how much of the update
    # a bf16 merge keeps -- the data behind keeping an adapter dynamic
    for spec in (lw.MERGE_WEIGHT, lw.MERGE_WEIGHT_SMALL):
        h = lw.merge_inputs(spec)
        W0, A, B = d2(h["W"]), d2(h["A"]), d2(h["B"])
        Wm = W0.clone()
        ms = _launch_stats(torch, stream, lambda: rg.lora_merge(Wm, A, B, spec.alpha, spec.strength))
        Wm.copy_(W0)
        rg.lora_merge(Wm, A, B, spec.alpha, spec.strength)
        s_ = spec.alpha / spec.rank * spec.strength
        upd = s_ * (B.double() @ A.double())
        kept = (Wm.double() - W0.double())
        lost = float((kept - upd).norm() / upd.norm())
        N, K, r = spec.N, spec.K, spec.rank
        byt = 2 * (2 * N * K + r * (N + K))
        gbs = byt / (ms["median"] * 1e-3) / 1e9
        e = {"workload": f"merge W += s.B.A: W=[{N}, {K}] bf16, r={r}, B~N(0, {spec.b_var:g})", "ms": ms,
             "bound": "hbm", "achieved_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
             "algorithmic_bytes": byt, "algorithmic_flop": 2.0 * N * K * r,
             "update_lost_fraction": round(lost, 4),
             "elements_changed_fraction": round(float((Wm != W0).double().mean()), 4)}
        out[spec.name] = e
        del W0, A, B, Wm, upd, kept, h
        torch.cuda.empty_cache()

    spec = lw.TINY_FP32
    h = lw.linear_inputs(spec)
    x, W, b, A, B = (d2(h[k]) for k in ("x", "W", "b", "A", "B"))
    y = torch.empty((spec.T, spec.N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, rg.lora_linear_workspace_size(spec.T, spec.K, spec.N, [spec.rank], rg.LORA_F32)), dtype=torch.uint8,
                     device=dev)
    ms = _launch_stats(torch, stream, lambda: rg.lora_linear(x, W, b, A, B, spec.alpha, out=y, workspace=ws))
    out["tiny_fp32"] = {"workload": "tiny fp32: T=64 K=128 N=96 r=8", "ms": ms, "bound": "launch latency",
                        "note": "back-to-back calls from Python: the figure is mostly the host's time per call"}
    return out


def _oracle_time(fn, flops, nbytes=None):
    """Wall time of one oracle call on the host (numpy float64, threaded BLAS)."""
    t = time.perf_counter()
    fn()
    dt = time.perf_counter() - t
    r = {"seconds": round(dt, 3), "threads": _blas_threads()}
    if flops:
        r["tflops"] = round(flops / dt / 1e12, 4)
    if nbytes:
        r["gbs"] = round(nbytes / dt / 1e9, 2)
    return r


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"),
                   default=len(os.sched_getaffinity(0)))
    except Exception:
        return len(os.sched_getaffinity(0))


def _oracle_linear(h, spec):
    from oracle import lora_oracle as lo
    return lo.lora_linear(h["x"], h["W"], h["b"], h["A"], h["B"], spec.alpha, spec.rank, spec.strength,
                          spec.request_scale)


def _oracle_multi(h, spec):
    from oracle import lora_oracle as lo
    return lo.lora_linear_multi(h["x"], h["W"], h["b"], h["adapters"], spec.request_scale)


def _oracle_stacked(h, spec):
    from oracle import lora_oracle as lo
    return lo.lora_linear_stacked(h["x"], h["W"], h["b"], h["groups"], spec.strength, spec.request_scale)


def _oracle_nf4(h, spec):
    from oracle import lora_oracle as lo
    return lo.lora_linear_nf4(h["x"], h["codes"], h["absmax"], h["codebook"], spec.blocksize, h["b"], h["A"],
                              h["B"], spec.alpha, spec.rank, spec.strength, spec.request_scale)


def _oracle_patch(h, spec):
    from oracle import lora_oracle as lo
    return lo.dense_patch(h["dst"], h["diff"], spec.strength, "add")


def _counter_means(csv_path, counter):
    """Mean counter value (KiB) per dispatch, keyed by (kernel kind, grid size)."""
    import csv
    import statistics
    vals = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            n = r["Kernel_Name"]
            kind = ("gemm" if "gemm_flow16_kernel" in n else "producer" if "down_kernel" in n
                    else "copy" if "copyBuffer" in n else None)
            if kind is None:
                continue
            vals.setdefault((kind, int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
    return {k: statistics.mean(v) for k, v in vals.items()}


def write_traffic(d):
    """HBM-side bytes per launch of the fused GEMM from FETCH_SIZE / WRITE_SIZE, each
    scaled by what the same counter reads for a plain 1 GiB device copy."""
    import glob
    import lora_workloads as lw

    def one(sub, counter):
        paths = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)
        assert paths, f"no counter_collection.csv under {os.path.join(d, sub)}"
        return _counter_means(paths[0], counter)
    f, w = one("f", "FETCH_SIZE"), one("w", "WRITE_SIZE")
    cf, cw = one("cf", "FETCH_SIZE"), one("cw", "WRITE_SIZE")
    kib = (1 << 30) / 1024
    fs = kib / max(v for (k, _), v in cf.items() if k == "copy")
    ws = kib / max(v for (k, _), v in cw.items() if k == "copy")
    launches = []
    for spec in (lw.FFN_UP, lw.FFN_DOWN):
        tiles = -(-spec.T // 256) * -(-spec.N // 256)
        key = ("gemm", tiles * 256)
        fb, wb = f[key] * 1024 * fs, w[key] * 1024 * ws
        alg = 2.0 * (spec.T * spec.K + spec.N * spec.K + spec.T * 64 + spec.N * spec.rank + spec.T * spec.N) \
            + (2.0 * spec.N if spec.bias else 0.0)
        launches.append({"layer": f"{spec.K}->{spec.N}", "FETCH_SIZE_KiB": round(f[key]), "WRITE_SIZE_KiB": round(w[key]),
                         "fetch_bytes": round(fb), "write_bytes": round(wb), "algorithmic_bytes": round(alg)})
    out = {"kernel_hash": kernel_hash(), "fetch_scale": fs, "write_scale": ws,
           "bytes_per_launch": round(sum(L["fetch_bytes"] + L["write_bytes"] for L in launches) / len(launches)),
           "algorithmic_bytes_per_launch": round(sum(L["algorithmic_bytes"] for L in launches) / len(launches)),
           "per_launch": launches,
           "commands": [
               "rocprofv3 --pmc FETCH_SIZE -d <dir>/f -o f --output-format csv -- python3 bench.py --layer-only --steps 2 --warmup 1",
               "rocprofv3 --pmc WRITE_SIZE -d <dir>/w -o w --output-format csv -- python3 bench.py --layer-only --steps 2 --warmup 1",
               "rocprofv3 --pmc FETCH_SIZE -d <dir>/cf -o cf --output-format csv -- python3 bench.py --copy-probe",
               "rocprofv3 --pmc WRITE_SIZE -d <dir>/cw -o cw --output-format csv -- python3 bench.py --copy-probe",
               "python3 bench.py --write-traffic <dir>"]}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out), flush=True)


def cpu_baseline(layers, target_s):
    """The fp64 oracle (as it stands) on the first rows of both layers' inputs."""
    import numpy as np
    from oracle import lora_oracle as lo
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"),
                    default=len(os.sched_getaffinity(0)))
    except Exception:
        cores = len(os.sched_getaffinity(0))
    host = []
    for L in layers:
        d = L["d"]
        host.append({k: (d[k].cpu() if d[k] is not None else None) for k in ("x", "W", "b", "A", "B")})

    def run(rows):
        t = time.perf_counter()
        fl = 0.0
        for L, h in zip(layers, host):
            lo.lora_linear(h["x"][:rows], h["W"], h["b"], h["A"], h["B"], L["d"]["alpha"], L["r"],
                           L["d"]["strength"], L["d"]["request_scale"])
            fl += layer_flops(rows, L["K"], L["N"], L["r"])
        return time.perf_counter() - t, fl

    rows = 256
    dt, fl = run(rows)
    while dt < target_s / 2 and rows < layers[0]["T"]:
        rows = min(layers[0]["T"], int(rows * max(2.0, min(8.0, target_s / max(dt, 1e-3) / 2))))
        dt, fl = run(rows)
    return {"value": float(f"{fl / dt / 1e12:.4g}"), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {rows} of 32760 tokens of both FFN layers, numpy float64, {dt:.1f}s",
            "cpu": cpu_model()}


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), else the machine type."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def mfma_probe(torch, stream, cus):
    """Matrix-core ceiling and shader clock under a pure MFMA load (lora_mfma_probe): one
    workgroup of 8 waves per compute unit, back-to-back MFMAs; rate from HIP events,
    clock from the shader-cycle / real-time counters of each workgroup."""
    import rank_gemm_lora_amd as rg
    sink = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2 * cus, dtype=torch.int64, device="cuda")
    iters = 1 << 12
    sp = stream.cuda_stream
    rg.lora_mfma_probe(256, cus, sink.data_ptr(), clocks.data_ptr(), sp)  # warm-up
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    rg.lora_mfma_probe(iters, cus, sink.data_ptr(), clocks.data_ptr(), sp)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    flops = cus * 8 * iters * 64 * 16384.0
    c = clocks.view(-1, 2).double().sum(0)
    ghz = float(c[0] / (c[1] / 100e6)) / 1e9 if c[1] > 0 else None
    return {"tflops": round(flops / (ms * 1e-3) / 1e12, 1), "clock_ghz": None if ghz is None else round(ghz, 3),
            "ms": round(ms, 3), "what": "back-to-back v_mfma_f32_16x16x32_bf16, no memory traffic, 2 waves per SIMD"}


if __name__ == "__main__":
    main()
