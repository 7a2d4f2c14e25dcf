"""Runs oracle functions over row chunks of large arrays in a pool of fresh Python
processes, for the full-size byte comparisons (test infrastructure: it calls only
`oracle/`). Every quantizer of the path is local to 128-row blocks (1x128 and 1x32 row
groups, 128x128 weight blocks, 128x1 column groups of 128 consecutive rows), and the
producers are row-wise, so chunks of a multiple of 128 rows reproduce the whole-tensor
results exactly.

The workers are spawned interpreters (not forks of a process that holds the GPU); they
import numpy and the oracle only.
"""

from __future__ import annotations

import atexit
import importlib
import multiprocessing as mp
import os

import numpy as np

_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        n = max(1, min(16, os.cpu_count() or 1))
        _POOL = mp.get_context("spawn").Pool(n)
        atexit.register(_POOL.terminate)
    return _POOL


def _run(task):
    mod, name, args, kwargs = task
    return getattr(importlib.import_module(mod), name)(*args, **kwargs)


def map_rows(fn, arr, *extra, chunk_rows=512, **kwargs):
    """[fn(arr[r:r+chunk_rows], *extra, **kwargs) for each chunk], computed in the pool."""
    assert chunk_rows % 128 == 0
    tasks = [(fn.__module__, fn.__name__, (np.ascontiguousarray(arr[r:r + chunk_rows]),) + extra, kwargs)
             for r in range(0, arr.shape[0], chunk_rows)]
    return _pool().map(_run, tasks, chunksize=1)


def rows_then_cols(parts, n_rows_out, n_cols_out):
    """Concatenate per-chunk results: the first n_rows_out outputs along axis 0 (row-wise
    payloads and scales), the next n_cols_out along axis 1 (transposed 128x1 copies)."""
    out = []
    for i in range(n_rows_out):
        out.append(np.concatenate([p[i] for p in parts], axis=0))
    for i in range(n_rows_out, n_rows_out + n_cols_out):
        out.append(np.concatenate([p[i] for p in parts], axis=1))
    return out
