"""Row-parallel evaluation of the oracle on the host's cores.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every query row of the attention definition is evaluated on its own: its
output depends on its own query vector and the keys it may see, never on
another row.  ``prefill_causal``, ``verify_fp8kv`` and ``prefill_causal_e4m3``
therefore take a ``rows`` argument, and a large output can be produced by
evaluating disjoint row subsets in separate processes and putting the pieces
back in row order.  Nothing in a row's arithmetic changes: each worker calls
the same oracle function on the same inputs.

Workers are started fresh ("spawn"), each with single-threaded BLAS, one per
host core (at most ``limit``); the inputs reach them through POSIX shared
memory, which is released when the call returns.
"""

from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
from multiprocessing import shared_memory

import numpy as np

from . import attention

_FUNCS = {
    "prefill_causal": attention.prefill_causal,
    "verify_fp8kv": attention.verify_fp8kv,
    "prefill_causal_e4m3": attention.prefill_causal_e4m3,
}

_BLAS_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


def host_cores(limit: int = 16) -> int:
    """Cores this process may run on, at most ``limit``."""
    return max(1, min(limit, len(os.sched_getaffinity(0))))


def _attach(specs):
    blocks, arrays = [], []
    for spec in specs:
        if spec[0] == "shm":
            _, name, shape, dtype = spec
            shm = shared_memory.SharedMemory(name=name)
            blocks.append(shm)
            arrays.append(np.ndarray(shape, dtype=np.dtype(dtype), buffer=shm.buf))
        else:
            arrays.append(spec[1])
    return blocks, arrays


def _work(func_name, specs, rows):
    blocks, args = _attach(specs)
    try:
        o, lse = _FUNCS[func_name](*args, rows=rows)
        return np.ascontiguousarray(o), np.ascontiguousarray(lse)
    finally:
        del args
        for b in blocks:
            b.close()


def run_rows(func_name: str, args, rows=None, n_rows: int | None = None, procs: int | None = None,
             chunks_per_proc: int = 4):
    """Evaluate oracle function ``func_name`` (one of prefill_causal, verify_fp8kv,
    prefill_causal_e4m3) on ``rows`` (all ``n_rows`` rows when None), split over
    ``procs`` worker processes.  ``args`` are the function's positional arguments
    before ``rows``; numpy arrays among them are shared, other values are passed
    as they are.  Returns (o, lse) for the rows in the given order, as the
    function itself would."""
    if func_name not in _FUNCS:
        raise ValueError(f"unknown oracle function {func_name}")
    if rows is None:
        if n_rows is None:
            raise ValueError("give rows or n_rows")
        rows = np.arange(n_rows)
    rows = np.asarray(rows, dtype=np.int64)
    procs = host_cores() if procs is None else max(1, int(procs))
    n_chunks = max(1, min(rows.size, procs * chunks_per_proc))
    # interleaved chunks: each holds rows from the whole range, so their costs match
    order = np.argsort(rows, kind="stable")
    pieces = [order[i::n_chunks] for i in range(n_chunks)]
    shms, specs = [], []
    try:
        for a in args:
            if isinstance(a, np.ndarray) and a.nbytes > 0:
                shm = shared_memory.SharedMemory(create=True, size=a.nbytes)
                shms.append(shm)
                np.ndarray(a.shape, dtype=a.dtype, buffer=shm.buf)[...] = a
                specs.append(("shm", shm.name, a.shape, a.dtype.str))
            else:
                specs.append(("val", a))
        saved = {k: os.environ.get(k) for k in _BLAS_ENV}
        for k in _BLAS_ENV:
            os.environ[k] = "1"
        try:
            # a worker that dies (for instance in a script without a __main__ guard,
            # which spawn re-imports) breaks the executor instead of being restarted
            with cf.ProcessPoolExecutor(max_workers=min(procs, n_chunks),
                                        mp_context=mp.get_context("spawn")) as ex:
                results = list(ex.map(_work, [func_name] * n_chunks, [specs] * n_chunks,
                                      [rows[p] for p in pieces]))
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()
    o0, l0 = results[0]
    o = np.empty((rows.size,) + o0.shape[1:], dtype=o0.dtype)
    lse = np.empty((rows.size,) + l0.shape[1:], dtype=l0.dtype)
    for p, (op, lp) in zip(pieces, results):
        o[p] = op
        lse[p] = lp
    return o, lse
