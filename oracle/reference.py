"""Reference decode and dequant-GEMV in fp64 (oracle).

What the fused kernel computes (papernotes.org page, 整体框架 and 关键设计 4;
gist.science page, Methodik / 4. Dequantisierungskernel): weight rows are cut into
24-long blocks along the input channels; each block's integer index is turned back
into a Leech lattice point and its inner product with the matching slice of the
activation vector is accumulated, so y = W_hat x without ever storing W_hat.

Readings taken (the pages leave these open):

* packing: a flat little-endian bitstream of fixed-width fields, one per block, in
  row-major block order; field j starts at bit f*j and holds shape | gain << shape_bits;
* reconstruction, shape-gain mode: w_hat = G[g] * v / |v| with |v| = 4 sqrt(m) in
  integer coordinates (papernotes.org page, 整体框架: the direction is a normalised
  point of the shell union, the magnitude is scalar-quantised);
* reconstruction, Euclidean mode: w_hat = s_row * v (raw integer coordinates times a
  per-row scale);
* K not a multiple of 24: x is treated as zero past K, and decoded weights past K are
  dropped;
* bf16 decode is bit-defined as bf16_rne(f32(v) * f32(f32(G[g]) * f32(1/(4 sqrt m)))),
  the reciprocal norm being computed in fp64 and rounded once to fp32;  Euclidean mode
  uses bf16_rne(f32(v) * f32(s_row)).

Everything here is plain loops over blocks with Python integers for the lattice
arithmetic and fp64 for every sum.
"""

import numpy as np

from .bijection import unrank
from .classes import find_class

DIM = 24
MODE_EUCLID = 0
MODE_SHAPEGAIN = 1


# ---------------------------------------------------------------------------
# bitstream

def read_field(packed: bytes, field_index: int, width: int) -> int:
    """Field `field_index` of a little-endian bitstream of `width`-bit fields."""
    bit = width * field_index
    first = bit >> 3
    last = (bit + width - 1) >> 3
    chunk = int.from_bytes(bytes(packed[first:last + 1]), "little")
    return (chunk >> (bit & 7)) & ((1 << width) - 1)


def blocks_per_row(cols: int) -> int:
    return (cols + DIM - 1) // DIM


def block_fields(packed, rows, cols, shape_bits, gain_bits, row):
    """(shape index, gain index) of every block of one row."""
    kb = blocks_per_row(cols)
    f = shape_bits + gain_bits
    out = []
    for b in range(kb):
        v = read_field(packed, row * kb + b, f)
        out.append((v & ((1 << shape_bits) - 1), v >> shape_bits))
    return out


# ---------------------------------------------------------------------------
# scales

def inv_norm_f64(m: int) -> float:
    return 1.0 / (4.0 * np.sqrt(float(m)))


def inv_norm_f32(m: int) -> np.float32:
    """1/(4 sqrt m) computed in fp64 and rounded once to fp32."""
    return np.float32(inv_norm_f64(m))


def block_scale_f64(mode, M, I, g, gains, row_scale):
    """fp64 multiplier applied to the integer point of a block."""
    if mode == MODE_SHAPEGAIN:
        m = find_class(I, M).m
        return float(np.float64(gains[g])) * inv_norm_f64(m)
    return float(np.float64(row_scale))


# ---------------------------------------------------------------------------
# decode

def decode_row_points(packed, rows, cols, M, shape_bits, gain_bits, row):
    """Integer lattice points of one row, shape [Kb*24] (pad columns included)."""
    out = []
    for I, _g in block_fields(packed, rows, cols, shape_bits, gain_bits, row):
        out.extend(unrank(I, M))
    return np.array(out, dtype=np.int64)


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def block_f32(I, g, M, mode, gains, row_scale):
    """fp32 values of one decoded block before the bf16 rounding: f32(v) * f32 scale, the
    scale being f32(G[g]) * f32(1/(4 sqrt m)) (shape-gain) or the row's scale (Euclidean)."""
    v = np.array(unrank(I, M), dtype=np.float32)
    if mode == MODE_SHAPEGAIN:
        m = find_class(I, M).m
        scale = np.float32(np.float32(gains[g]) * inv_norm_f32(m))
    else:
        scale = np.float32(row_scale)
    return v * scale


def block_bf16(I, g, M, mode, gains, row_scale):
    """bf16 bit patterns of one decoded block (all 24 values, pad columns included)."""
    return f32_to_bf16_bits(block_f32(I, g, M, mode, gains, row_scale))


def decode_row_bf16(packed, rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales, row):
    """bf16 bit patterns of one decoded row, shape [cols] (pad columns dropped)."""
    vals = np.empty(blocks_per_row(cols) * DIM, dtype=np.float32)
    rs = None if row_scales is None else row_scales[row]
    for b, (I, g) in enumerate(block_fields(packed, rows, cols, shape_bits, gain_bits, row)):
        vals[b * DIM:(b + 1) * DIM] = block_f32(I, g, M, mode, gains, rs)
    return f32_to_bf16_bits(vals[:cols])


# ---------------------------------------------------------------------------
# GEMV

def gemv_row(packed, rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales, x, row):
    """(y[b][row], sum_k |W_hat[row,k] x[b,k]|) in fp64 for every batch row b of x.

    x: array [batch][cols] (any float dtype; converted exactly to fp64)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    batch = x.shape[0]
    kb = blocks_per_row(cols)
    xp = np.zeros((batch, kb * DIM))
    xp[:, :cols] = x
    y = np.zeros(batch)
    mag = np.zeros(batch)
    for b, (I, g) in enumerate(block_fields(packed, rows, cols, shape_bits, gain_bits, row)):
        v = np.array(unrank(I, M), dtype=np.float64)
        if mode == MODE_SHAPEGAIN:
            scale = float(np.float64(gains[g])) * inv_norm_f64(find_class(I, M).m)
        else:
            scale = float(np.float64(row_scales[row]))
        seg = xp[:, b * DIM:(b + 1) * DIM]
        terms = (scale * v)[None, :] * seg
        y += terms.sum(axis=1)
        mag += np.abs(terms).sum(axis=1)
    return y, mag


def gemv(packed, rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales, x, row_list=None):
    """fp64 y[batch][len(row_list)] and the matching sum-of-|terms| magnitudes."""
    row_list = range(rows) if row_list is None else row_list
    ys, mags = [], []
    for r in row_list:
        y, mag = gemv_row(packed, rows, cols, M, mode, shape_bits, gain_bits, gains, row_scales, x, r)
        ys.append(y)
        mags.append(mag)
    return np.array(ys).T, np.array(mags).T


GEMV_REL_TOL = 1e-4


def gemv_within_tolerance(y_test, y_ref, mag, rel=GEMV_REL_TOL):
    """Elementwise |y - y_ref| <= rel * sum_k |W_hat x| (the normalised error bound)."""
    y_test = np.asarray(y_test, dtype=np.float64)
    return np.abs(y_test - y_ref) <= rel * mag


def normalized_errors(y_test, y_ref, mag):
    y_test = np.asarray(y_test, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.abs(y_test - y_ref) / mag
    return np.where(mag > 0, e, np.where(y_test == y_ref, 0.0, np.inf))
