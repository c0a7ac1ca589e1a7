"""Process-pool drivers for the oracle (test infrastructure, not the product path).

The oracle is plain and slow (pure-Python integers per block), so checks over whole
layers split the rows over worker processes.  Each worker runs the unchanged oracle
functions of reference.py and bijection.py on its share; nothing here computes anything
of its own.  The job's inputs are set before the pool forks, so the workers inherit the
packed stream instead of receiving a pickled copy per task.

Worker count: the host's usable cores, at most 16 (the CPU share of a one-GPU machine).
"""

import multiprocessing as mp
import os

import numpy as np

from . import reference
from .bijection import unrank

MAX_PROCS = 16
_JOB = None


def cores(limit=MAX_PROCS):
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, limit))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _chunks(items, procs, per_proc=4):
    items = list(items)
    n = max(1, min(len(items), procs * per_proc))
    step = (len(items) + n - 1) // n
    return [items[i:i + step] for i in range(0, len(items), step)]


def _run(job, fn, chunks, procs):
    global _JOB
    _JOB = job
    try:
        with mp.get_context("fork").Pool(procs) as pool:
            return pool.map(fn, chunks)
    finally:
        _JOB = None


def _gemv_chunk(rows):
    packed, nrows, cols, M, mode, sb, gb, gains, scales, x = _JOB
    return reference.gemv(packed, nrows, cols, M, mode, sb, gb, gains, scales, x, rows)


def gemv_rows(packed, rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales, x, row_list=None,
              procs=None):
    """reference.gemv over `row_list` (default: every row) in a process pool:
    fp64 y [batch][len(row_list)] and the sum-of-|terms| magnitudes of the same shape."""
    row_list = list(range(rows)) if row_list is None else list(row_list)
    procs = procs or cores()
    packed = bytes(packed)
    job = (packed, rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales, np.atleast_2d(x))
    parts = _run(job, _gemv_chunk, _chunks(row_list, procs), procs)
    y = np.concatenate([p[0] for p in parts], axis=1)
    mag = np.concatenate([p[1] for p in parts], axis=1)
    return y, mag


def _bf16_chunk(rows):
    packed, nrows, cols, M, mode, sb, gb, gains, scales = _JOB
    return np.stack([reference.decode_row_bf16(packed, nrows, cols, M, mode, sb, gb, gains, scales, r)
                     for r in rows])


def decode_rows_bf16(packed, rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales, row_list,
                     procs=None):
    """reference.decode_row_bf16 of every row in `row_list`: uint16 [len(row_list)][cols]."""
    procs = procs or cores()
    job = (bytes(packed), rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales)
    return np.concatenate(_run(job, _bf16_chunk, _chunks(row_list, procs), procs))


def _unrank_chunk(idx):
    (M,) = _JOB
    return np.array([unrank(int(I), M) for I in idx], dtype=np.int64).reshape(-1, 24)


def unrank_many(indices, M, procs=None):
    """bijection.unrank of every index: int64 points [n][24]."""
    procs = procs or cores()
    idx = [int(I) for I in indices]
    return np.concatenate(_run((M,), _unrank_chunk, _chunks(idx, procs), procs))


def _bf16_many_chunk(pairs):
    tensors = _JOB
    return [reference.decode_row_bf16(*tensors[i], r) for i, r in pairs]


def decode_rows_bf16_many(tensors, pairs, procs=None):
    """reference.decode_row_bf16 of rows of several tensors: `tensors` is a list of
    (packed bytes, rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales) and
    `pairs` a list of (tensor number, row); returns the uint16 rows in that order."""
    procs = procs or cores()
    parts = _run(list(tensors), _bf16_many_chunk, _chunks(pairs, procs), procs)
    return [row for part in parts for row in part]


def _blocks_bf16_chunk(items):
    M, mode, tables = _JOB
    return [reference.block_bf16(I, g, M, mode, tables[k], tables[k]) for k, I, g in items]


def blocks_bf16(items, M, mode, tables, procs=None):
    """reference.block_bf16 of many blocks: `items` is a list of (table number, shape index,
    gain index), `tables[k]` the fp16 gain table (shape-gain) or row scale (Euclidean) of
    item k's tensor; returns uint16 [len(items)][24]."""
    procs = procs or cores()
    parts = _run((M, mode, list(tables)), _blocks_bf16_chunk, _chunks(items, procs), procs)
    return np.array([b for part in parts for b in part], dtype=np.uint16).reshape(-1, 24)
