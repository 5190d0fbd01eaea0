"""Helpers for the GPU parity tests: moving seeded inputs to the device and
comparing the HIP path's outputs with the oracle's."""
import sys

import numpy as np
import torch

from oracle import lora_oracle as lo

DEV = "cuda:0"
LOSSLESS_BF16_GATE = 4e-3  # relative RMS against fp64 (bf16 outputs)
LOSSLESS_F32_GATE = 1e-6   # relative RMS against fp64 (fp32 outputs)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(t):
    return None if t is None else t.to(DEV).contiguous()


def host64(t):
    return t.detach().to("cpu").double().numpy()


def assert_bitwise(y_gpu, y_ref, what=""):
    g = host64(y_gpu)
    assert g.shape == y_ref.shape, (what, g.shape, y_ref.shape)
    bad = np.argwhere(~((g == y_ref) | (np.isnan(g) & np.isnan(y_ref))))
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}: " \
                          f"gpu {g[tuple(bad[0])]!r} ref {y_ref[tuple(bad[0])]!r}"


def assert_gate(y_gpu, y64, y_chain=None, gate=LOSSLESS_BF16_GATE, what=""):
    """Lossless acceptance: relative RMS <= gate and, when the chain is given,
    no larger than the separate-pass chain's error against the same fp64 result."""
    e = lo.rel_rms(host64(y_gpu), y64)
    msg = f"{what}: rel_rms {e:.3e}"
    if y_chain is not None:
        ec = lo.rel_rms(y_chain, y64)
        msg += f" chain {ec:.3e}"
        say(msg)
        assert e <= ec, msg
    else:
        say(msg)
    assert e <= gate, msg
    return e


def sample_rows(T, n_each=32, seed=0, tile=256):
    """First rows, the last (ragged) tile's rows, and random rows in between."""
    rng = np.random.default_rng(seed)
    head = np.arange(min(n_each, T))
    last_tile = (T - 1) // tile * tile
    tail = np.arange(max(last_tile, T - n_each), T)
    mid = rng.choice(T, size=min(n_each, T), replace=False)
    return np.unique(np.concatenate([head, tail, mid]))
