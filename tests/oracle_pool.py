"""Row-parallel evaluation of the CPU oracle for the GPU tests.

The rows of a linear layer are independent, so the oracle's ordered-fp64 chain
(one Python-level step per k) runs on chunks of rows in a few spawned worker
processes. The workers import numpy and ``oracle`` only and never touch the
GPU; every argument reaches them as numpy arrays (bf16 and fp32 values widened
exactly to float64, 4-bit codes as uint8).
"""
from __future__ import annotations

import concurrent.futures as cf
import importlib
import multiprocessing as mp
import os

import numpy as np

_ARGS = None


def _to_numpy(v):
    if hasattr(v, "detach"):  # torch tensor
        t = v.detach().cpu()
        return t.numpy().copy() if str(t.dtype) == "torch.uint8" else t.double().numpy()
    if isinstance(v, dict):
        return {k: _to_numpy(u) for k, u in v.items()}
    if isinstance(v, (list, tuple)):
        return type(v)(_to_numpy(u) for u in v)
    return v


def _init(args):
    global _ARGS
    _ARGS = args


def _run(job):
    mod, name, x_rows, kwargs = job
    fn = getattr(importlib.import_module(mod), name)
    return fn(x_rows, *_ARGS, **kwargs)


def workers() -> int:
    return max(1, min(8, len(os.sched_getaffinity(0))))


def rows_parallel(fn, x, rows, args=(), kwargs=None, chunk=16) -> np.ndarray:
    """fn(x[rows], *args, **kwargs) with fn a function of ``oracle`` whose first argument is x and
    whose output rows follow x's rows; evaluated on chunks of ``chunk`` rows in worker processes."""
    xr = _to_numpy(x)[np.asarray(rows)]
    a = _to_numpy(tuple(args))
    jobs = [(fn.__module__, fn.__name__, xr[i:i + chunk], dict(kwargs or {})) for i in range(0, len(xr), chunk)]
    n = min(workers(), len(jobs))
    if n <= 1:
        _init(a)
        return np.concatenate([_run(j) for j in jobs])
    # (a worker that dies raises BrokenProcessPool here instead of leaving the call waiting)
    with cf.ProcessPoolExecutor(n, mp_context=mp.get_context("spawn"), initializer=_init, initargs=(a,)) as pool:
        return np.concatenate(list(pool.map(_run, jobs, timeout=1800)))
