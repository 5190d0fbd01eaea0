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


def sample_rows(T, seed=0, n_head=16, n_rand=16, min_rows=256, tile=256):
    """The first rows, every row of the last (ragged) 256-token tile and random rows in between:
    at least ``min_rows`` rows, or all of them when T is smaller."""
    if T <= min_rows:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    head = np.arange(min(n_head, T))
    tail = np.arange((T - 1) // tile * tile, T)
    chosen = np.union1d(head, tail)
    pool = np.setdiff1d(np.arange(T), chosen)
    need = max(n_rand, min_rows - len(chosen))
    mid = rng.choice(pool, size=min(need, len(pool)), replace=False)
    return np.union1d(chosen, mid)


def nan_out(T, N, dtype=torch.bfloat16):
    """An output buffer filled with NaN: after the call, no NaN left means every element was written."""
    return torch.full((T, N), float("nan"), dtype=dtype, device=DEV)
