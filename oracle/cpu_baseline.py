"""Timed CPU oracle run used as the reported CPU baseline of the benchmark.

Test infrastructure: only the benchmark's CPU-baseline leg uses it.  Runs the oracle
exactly as it stands (decode every block of the sampled rows with the pure-Python
bijection, then the fp64 dot products; oracle/reference.py) in a process pool over rows
(at most 16 processes: the CPU share of a one-GPU machine), and reports the wall time.  It is a
reported baseline, not a target.
"""

import multiprocessing as mp
import time

import numpy as np

from . import parallel


def time_gemv_rows(packed, rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales, x, row_list,
                   procs=None):
    """Wall seconds for the oracle GEMV of `row_list` over a process pool (oracle/parallel.py),
    the number of processes used, and the oracle's fp64 (y [batch][len(row_list)], sum of
    |terms| of the same shape), so the caller can check its own output against it."""
    procs = procs or parallel.cores()
    procs = max(1, min(procs, len(row_list)))
    chunks = parallel._chunks(row_list, procs)
    parallel._JOB = (bytes(packed), rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales,
                     np.atleast_2d(x))
    try:
        with mp.get_context("fork").Pool(procs) as pool:
            pool.map(parallel._gemv_chunk, [[row_list[0]]] * procs)      # start every worker
            t0 = time.perf_counter()
            parts = pool.map(parallel._gemv_chunk, chunks)
            dt = time.perf_counter() - t0
    finally:
        parallel._JOB = None
    y = np.concatenate([p[0] for p in parts], axis=1)
    mag = np.concatenate([p[1] for p in parts], axis=1)
    assert y.shape[1] == len(row_list)
    return dt, procs, y, mag


def _search_chunk(args):
    blocks, M, mode = args
    from . import search
    return [search.search(b, M, mode) for b in blocks]


def time_search(blocks, M, mode, procs=None):
    """Wall seconds for the oracle's exact search (oracle/search.py) of every block in
    `blocks` (float64 [n][24]) over a process pool, the number of processes used, and the
    oracle's (global index, point) of every block in order."""
    procs = procs or parallel.cores()
    procs = max(1, min(procs, len(blocks)))
    chunks = [blocks[i::procs] for i in range(procs)]
    ctx = mp.get_context("fork")
    with ctx.Pool(procs) as pool:
        pool.map(_search_chunk, [(blocks[:1], M, mode)] * procs)   # warm the per-process tables
        t0 = time.perf_counter()
        parts = pool.map(_search_chunk, [(c, M, mode) for c in chunks])
        dt = time.perf_counter() - t0
    res = [None] * len(blocks)
    for i, part in enumerate(parts):
        res[i::procs] = part
    assert all(r is not None for r in res)
    return dt, procs, res
