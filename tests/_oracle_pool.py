"""Whole-tensor parity at full workload sizes: the fp64 oracle's
per-(sequence, head) functions, unchanged, spread over a process pool, and
error statistics accumulated over every element of each output tensor.

TEST INFRASTRUCTURE.  The pool only distributes calls of the oracle's
per-(sequence, head) functions; the arithmetic is the oracle's.  Workers are spawned (no fork of a process that holds a GPU
context) with one BLAS thread each, and take the most expensive items first.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

from tests._parity import LSE_MAX_ABS, MAX_ABS, REL_L2


def _item(args):
    qb, kb, vb, dob, scale, causal, window = args
    from oracle import jfa_oracle as jo
    o, lse, _ = jo.sequence_forward(qb, kb, vb, scale, causal, window)
    dq, dk, dv = jo.sequence_backward(qb, kb, vb, dob, scale, causal, window)
    return o, lse, dq, dk, dv


def pool_size() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_items(items, cost):
    """Yields (index, (o, lse, dq, dk, dv)) for every item, most expensive
    first.  items[i] = (q, k, v, dout, scale, causal, window) of one
    (sequence, head); cost[i] orders the work."""
    order = sorted(range(len(items)), key=lambda i: -cost[i])
    keep = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in keep:
        os.environ[k] = "1"
    try:
        ctx = mp.get_context("spawn")
        with ctx.Pool(pool_size()) as pool:
            for i, res in zip(order, pool.imap(_item, [items[i] for i in order], chunksize=1)):
                yield i, res
    finally:
        for k, v in keep.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _call(args):
    module, fn, fargs = args
    import importlib
    return getattr(importlib.import_module(module), fn)(*fargs)


def run_calls(module: str, fn: str, arg_lists, cost):
    """Yields (index, result) of module.fn(*arg_lists[i]) for every i, most
    expensive first, in the same pool (an oracle function, unchanged)."""
    order = sorted(range(len(arg_lists)), key=lambda i: -cost[i])
    keep = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in keep:
        os.environ[k] = "1"
    try:
        ctx = mp.get_context("spawn")
        with ctx.Pool(pool_size()) as pool:
            work = [(module, fn, arg_lists[i]) for i in order]
            for i, res in zip(order, pool.imap(_call, work, chunksize=4)):
                yield i, res
    finally:
        for k, v in keep.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


class WholeTensor:
    """max |got - ref| and ||got - ref|| / ||ref|| over a whole tensor fed in
    pieces (the same numbers tests._parity.compare gives on the assembled
    tensor), checked against the bar at the end."""

    def __init__(self, name, max_abs=MAX_ABS, rel_l2=REL_L2):
        self.name, self.max_abs_bar, self.rel_bar = name, max_abs, rel_l2
        self.max_abs, self.d2, self.r2, self.n = 0.0, 0.0, 0.0, 0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert got.shape == ref.shape, (self.name, got.shape, ref.shape)
        assert np.all(np.isfinite(got)), f"{self.name}: non-finite values"
        if got.size == 0:
            return
        diff = got - ref
        self.max_abs = max(self.max_abs, float(np.max(np.abs(diff))))
        self.d2 += float(np.sum(diff * diff))
        self.r2 += float(np.sum(ref * ref))
        self.n += got.size

    def check(self):
        rel = float(np.sqrt(self.d2 / self.r2)) if self.r2 > 0 else float(np.sqrt(self.d2))
        print(f"  {self.name}: {self.n} elements, max abs {self.max_abs:.3e}, rel L2 {rel:.3e}", flush=True)
        assert self.max_abs <= self.max_abs_bar, f"{self.name}: max abs err {self.max_abs:.3e} > {self.max_abs_bar}"
        assert rel <= self.rel_bar, f"{self.name}: rel L2 err {rel:.3e} > {self.rel_bar}"


class WholeLse:
    """lse over a whole tensor: the same -inf pattern, max-abs bar elsewhere."""

    def __init__(self, name, max_abs=LSE_MAX_ABS):
        self.name, self.bar, self.max_abs, self.n = name, max_abs, 0.0, 0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        ninf = np.isneginf(ref)
        assert np.array_equal(np.isneginf(got), ninf), f"{self.name}: -inf pattern differs"
        if (~ninf).any():
            self.max_abs = max(self.max_abs, float(np.max(np.abs(got[~ninf] - ref[~ninf]))))
        self.n += got.size

    def check(self):
        print(f"  {self.name}: {self.n} elements, max abs {self.max_abs:.3e}", flush=True)
        assert self.max_abs <= self.bar, f"{self.name}: max abs err {self.max_abs:.3e} > {self.bar}"
