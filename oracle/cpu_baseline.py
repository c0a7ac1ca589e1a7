"""Timed CPU oracle run used as the reported CPU baseline of the benchmark.

Runs the oracle exactly as it stands (decode every block of the sampled rows with the
pure-Python bijection, then the fp64 dot products; oracle/reference.py) in a process
pool over rows, and reports the wall time.  It is a reported baseline, not a target.
"""

import multiprocessing as mp
import os
import time

from . import reference


def _rows(args):
    packed, rows, cols, M, mode, sb, gb, gains, scales, x, row_list = args
    reference.gemv(packed, rows, cols, M, mode, sb, gb, gains, scales, x, row_list)
    return len(row_list)


def time_gemv_rows(packed, rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales, x, row_list,
                   procs=None):
    """Wall seconds for the oracle GEMV of `row_list`, and the number of processes used."""
    procs = procs or os.cpu_count() or 1
    procs = max(1, min(procs, len(row_list)))
    chunks = [row_list[i::procs] for i in range(procs)]
    args = [(packed, rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales, x, c) for c in chunks if c]
    ctx = mp.get_context("fork")
    with ctx.Pool(len(args)) as pool:
        pool.map(_rows, [(packed, rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales, x, [row_list[0]])])
        t0 = time.perf_counter()
        done = sum(pool.map(_rows, args))
        dt = time.perf_counter() - t0
    assert done == len(row_list)
    return dt, len(args)


def _search_chunk(args):
    blocks, M, mode = args
    from . import search
    for b in blocks:
        search.search(b, M, mode)
    return len(blocks)


def time_search(blocks, M, mode, procs=None):
    """Wall seconds for the oracle's exact search (oracle/search.py) of every block in
    `blocks` (float64 [n][24]) over a process pool, and the number of processes used."""
    procs = procs or os.cpu_count() or 1
    procs = max(1, min(procs, len(blocks)))
    chunks = [blocks[i::procs] for i in range(procs)]
    ctx = mp.get_context("fork")
    with ctx.Pool(procs) as pool:
        pool.map(_search_chunk, [(blocks[:1], M, mode)] * procs)   # warm the per-process tables
        t0 = time.perf_counter()
        done = sum(pool.map(_search_chunk, [(c, M, mode) for c in chunks]))
        dt = time.perf_counter() - t0
    assert done == len(blocks)
    return dt, procs
