"""Seeded synthetic inputs for LLVQ decode / dequant-GEMV workloads.

This module is shared by the tests, the benchmark and the CPU oracle checks.  It holds
none of the method's arithmetic: it draws random numbers, rounds activations to bf16
and writes fixed-width fields into a little-endian bitstream.  Anything that depends on
the lattice (the number of valid shape indices, the class table, decoding) comes from
the caller.

Streams: numpy default_rng(SeedSequence([workload_id, tensor_id, stream])) with
  stream 0 shape indices  (uniform over [0, index_count), unbiased)
  stream 1 gain indices   (uniform over 0..2^gain_bits - 1)
  stream 2 gain table     (sorted |N(0,1)| * sqrt(24), rounded to fp16)
  stream 3 row scales     (U(0.5, 2), rounded to fp16)
  stream 4 + b activation row b (N(0,1) fp32, rounded to bf16 unless fp32 is asked)
  stream 64 dense weights for fidelity rows (N(0, std^2) fp32)
"""

from dataclasses import dataclass, field

import numpy as np

DIM = 24
PAD_BYTES = 16          # readable slack past the last field (kernels may over-read)

MODE_EUCLID = 0
MODE_SHAPEGAIN = 1


def rng(workload: int, tensor: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([workload, tensor, stream]))


def blocks_per_row(cols: int) -> int:
    return (cols + DIM - 1) // DIM


def packed_nbytes(n_fields: int, width: int) -> int:
    """Bytes for n_fields fields of `width` bits, rounded up to 16 B, plus 16 B slack."""
    nbits = n_fields * width
    nbytes = (nbits + 7) // 8
    nbytes = (nbytes + 15) // 16 * 16
    return nbytes + PAD_BYTES


def pack_fields(values: np.ndarray, width: int) -> np.ndarray:
    """Write uint64 `values` as consecutive little-endian `width`-bit fields."""
    values = np.ascontiguousarray(values, dtype=np.uint64).ravel()
    n = values.size
    out = np.zeros(packed_nbytes(n, width), dtype=np.uint8)
    if n == 0:
        return out
    if width % 8 == 0 and width <= 64:
        nb = width // 8
        as_bytes = values.view(np.uint8).reshape(n, 8)[:, :nb]
        out[: n * nb] = as_bytes.ravel()
        return out
    # generic path: expand to bits, little-endian inside each field
    bits = ((values[:, None] >> np.arange(width, dtype=np.uint64)[None, :]) & np.uint64(1)).astype(np.uint8)
    flat = bits.ravel()
    packed = np.packbits(flat, bitorder="little")
    out[: packed.size] = packed
    return out


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even), returned as uint16 bit patterns."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Tensor:
    """One packed LLVQ weight tensor plus the activations it is applied to."""
    name: str
    mode: int
    rows: int
    cols: int
    max_shell: int
    shape_bits: int
    gain_bits: int
    shape_idx: np.ndarray          # uint64 [rows, Kb]
    gain_idx: np.ndarray           # uint64 [rows, Kb] (zeros when gain_bits == 0)
    scales_f16: np.ndarray         # fp16 gain table [2^gain_bits] or row scales [rows]
    packed: np.ndarray             # uint8 bitstream
    x_bits: np.ndarray = None      # uint16 bf16 bits [batch, cols] or None
    x_f32: np.ndarray = None       # fp32 [batch, cols] or None
    extra: dict = field(default_factory=dict)

    @property
    def kb(self) -> int:
        return blocks_per_row(self.cols)

    @property
    def field_bits(self) -> int:
        return self.shape_bits + self.gain_bits

    def x_as_f64(self) -> np.ndarray:
        if self.x_f32 is not None:
            return self.x_f32.astype(np.float64)
        return bf16_to_f32(self.x_bits).astype(np.float64)


def draw_indices(workload, tensor, shape, index_count) -> np.ndarray:
    return rng(workload, tensor, 0).integers(0, index_count, size=shape, dtype=np.uint64)


def draw_gain_table(workload, tensor, n, scale=1.0) -> np.ndarray:
    g = np.sort(np.abs(rng(workload, tensor, 2).standard_normal(n)) * np.sqrt(DIM)) * scale
    return g.astype(np.float16)


def gaussian_source(workload, n_blocks) -> np.ndarray:
    """n_blocks x 24 i.i.d. N(0, 1) samples (fp32), the memoryless Gaussian source."""
    return rng(workload, 0, 7).standard_normal((n_blocks, DIM)).astype(np.float32)


def chi_gain_table(levels, dim=DIM) -> np.ndarray:
    """Gain table for the norm of a dim-dimensional standard Gaussian vector (chi
    distribution with dim degrees of freedom): the conditional means of `levels` cells of
    equal probability, ascending, as fp16.  Uses E[R; a < R < b] = c (F'(b) - F'(a)) with
    F' the chi CDF of dim + 1 degrees of freedom and c = sqrt(2) G((dim+1)/2) / G(dim/2)."""
    from scipy import special, stats
    q = stats.chi(dim).ppf(np.linspace(0.0, 1.0, levels + 1))
    c = np.sqrt(2.0) * np.exp(special.gammaln((dim + 1) / 2.0) - special.gammaln(dim / 2.0))
    upper = stats.chi(dim + 1).cdf(q)
    return (c * np.diff(upper) * levels).astype(np.float16)


def gptq_layer(workload, rows, cols, samples, std=0.02):
    """The weights and activations behind gptq_problem: (W [rows][cols] fp32,
    X [samples][cols] fp32), H = X^T X / samples."""
    W = (rng(workload, 0, 8).standard_normal((rows, cols)) * std).astype(np.float32)
    r = rng(workload, 0, 9)
    mix = r.standard_normal((cols, cols)) / np.sqrt(cols) + np.eye(cols)
    scale = np.exp(0.5 * r.standard_normal(cols))
    X = (r.standard_normal((samples, cols)) @ mix) * scale
    return W, X.astype(np.float32)


def gptq_problem(workload, rows, cols, samples, std=0.02):
    """A layer for error-feedback quantisation: dense N(0, std^2) weights W [rows][cols]
    (fp32) and the Hessian H = X^T X / samples (fp64) of activations X [samples][cols] with
    correlated channels (standard normals mixed by I + a random Gaussian matrix / sqrt(cols))
    and log-normal channel scales exp(0.5 N(0, 1)) (some larger channels, as in LLM
    activations)."""
    W = (rng(workload, 0, 8).standard_normal((rows, cols)) * std).astype(np.float32)
    r = rng(workload, 0, 9)
    mix = r.standard_normal((cols, cols)) / np.sqrt(cols) + np.eye(cols)
    scale = np.exp(0.5 * r.standard_normal(cols))
    X = (r.standard_normal((samples, cols)) @ mix) * scale
    H = X.T @ X / samples
    return W, H


def draw_activations(workload, tensor, batch, cols, dtype="bf16"):
    xs = np.stack([rng(workload, tensor, 4 + b).standard_normal(cols).astype(np.float32)
                   for b in range(batch)])
    if dtype == "f32":
        return None, xs
    return bf16_round(xs), None


def make_tensor(name, workload, tensor, rows, cols, index_count, *, mode=MODE_SHAPEGAIN,
                max_shell=10, shape_bits=44, gain_bits=4, batch=1, x_dtype="bf16",
                gain_scale=1.0, override_rows=None) -> Tensor:
    """Random packed tensor.  `override_rows` = (shape_idx [r, Kb], gain_idx [r, Kb]) replaces
    the first r rows (used for the fidelity rows)."""
    kb = blocks_per_row(cols)
    shape_idx = draw_indices(workload, tensor, (rows, kb), index_count)
    if gain_bits:
        gain_idx = rng(workload, tensor, 1).integers(0, 1 << gain_bits, size=(rows, kb), dtype=np.uint64)
        scales = draw_gain_table(workload, tensor, 1 << gain_bits, gain_scale)
    else:
        gain_idx = np.zeros((rows, kb), dtype=np.uint64)
        scales = rng(workload, tensor, 3).uniform(0.5, 2.0, size=rows).astype(np.float16)
    if override_rows is not None:
        s_over, g_over = override_rows
        r = s_over.shape[0]
        shape_idx[:r] = s_over
        gain_idx[:r] = g_over
    fields = shape_idx | (gain_idx << np.uint64(shape_bits))
    packed = pack_fields(fields, shape_bits + gain_bits)
    xb, xf = draw_activations(workload, tensor, batch, cols, x_dtype) if batch else (None, None)
    return Tensor(name, mode, rows, cols, max_shell, shape_bits, gain_bits, shape_idx, gain_idx,
                  scales, packed, xb, xf)


# ---------------------------------------------------------------------------
# fields wider than 64 bits (other rates): 128-bit values as (lo, hi) uint64 pairs

def draw_indices_wide(workload, tensor, shape, index_count):
    """Uniform shape indices over [0, index_count) for counts up to 2^128, as (lo, hi)
    uint64 arrays: random words of index_count's bit length, redrawn while >= the count."""
    n = int(np.prod(shape))
    g = rng(workload, tensor, 0)
    nbits = (index_count - 1).bit_length()
    hb = max(nbits - 64, 0)
    lo = np.zeros(n, dtype=np.uint64)
    hi = np.zeros(n, dtype=np.uint64)
    todo = np.arange(n)
    c_lo, c_hi = np.uint64(index_count & (2**64 - 1)), np.uint64(index_count >> 64)
    while todo.size:
        if hb:
            l = g.integers(0, 2**64 - 1, size=todo.size, dtype=np.uint64, endpoint=True)
            h = g.integers(0, (1 << hb) - 1, size=todo.size, dtype=np.uint64, endpoint=True)
        else:
            l = g.integers(0, index_count, size=todo.size, dtype=np.uint64)
            h = np.zeros(todo.size, dtype=np.uint64)
        ok = (h < c_hi) | ((h == c_hi) & (l < c_lo))
        lo[todo[ok]] = l[ok]
        hi[todo[ok]] = h[ok]
        todo = todo[~ok]
    return lo.reshape(shape), hi.reshape(shape)


def pack_fields_wide(lo, hi, width: int) -> np.ndarray:
    """Write 128-bit values (lo | hi << 64) as consecutive little-endian `width`-bit fields."""
    lo = np.ascontiguousarray(lo, dtype=np.uint64).ravel()
    hi = np.ascontiguousarray(hi, dtype=np.uint64).ravel()
    n = lo.size
    out = np.zeros(packed_nbytes(n, width), dtype=np.uint8)
    if n == 0:
        return out
    parts = [((lo[:, None] >> np.arange(min(width, 64), dtype=np.uint64)[None, :]) & np.uint64(1)).astype(np.uint8)]
    if width > 64:
        parts.append(((hi[:, None] >> np.arange(width - 64, dtype=np.uint64)[None, :]) & np.uint64(1))
                     .astype(np.uint8))
    packed = np.packbits(np.concatenate(parts, axis=1).ravel(), bitorder="little")
    out[: packed.size] = packed
    return out


def make_wide_tensor(name, workload, tensor, rows, cols, index_count, *, mode=MODE_SHAPEGAIN, max_shell=42,
                     shape_bits=68, gain_bits=4, batch=1, x_dtype="bf16") -> Tensor:
    """Random packed tensor with fields of any width up to 128 bits; shape_idx is an object
    array of Python integers."""
    kb = blocks_per_row(cols)
    s_lo, s_hi = draw_indices_wide(workload, tensor, (rows, kb), index_count)
    if gain_bits:
        gain_idx = rng(workload, tensor, 1).integers(0, 1 << gain_bits, size=(rows, kb), dtype=np.uint64)
        scales = draw_gain_table(workload, tensor, 1 << gain_bits)
    else:
        gain_idx = np.zeros((rows, kb), dtype=np.uint64)
        scales = rng(workload, tensor, 3).uniform(0.5, 2.0, size=rows).astype(np.float16)
    f_lo, f_hi = s_lo.copy(), s_hi.copy()
    if shape_bits >= 64:
        f_hi |= gain_idx << np.uint64(shape_bits - 64)
    else:
        f_lo |= gain_idx << np.uint64(shape_bits)
        if shape_bits + gain_bits > 64:
            f_hi |= gain_idx >> np.uint64(64 - shape_bits)
    packed = pack_fields_wide(f_lo, f_hi, shape_bits + gain_bits)
    shape_idx = s_lo.astype(object) + (s_hi.astype(object) << 64)
    xb, xf = draw_activations(workload, tensor, batch, cols, x_dtype) if batch else (None, None)
    return Tensor(name, mode, rows, cols, max_shell, shape_bits, gain_bits, shape_idx, gain_idx,
                  scales, packed, xb, xf)


def fidelity_weights(workload, tensor, rows, cols, std=0.02) -> np.ndarray:
    """Dense N(0, std^2) fp32 weights for the fidelity rows."""
    return (rng(workload, tensor, 64).standard_normal((rows, cols)) * std).astype(np.float32)


# ---------------------------------------------------------------------------
# the five workloads (sizes as stated for the LLVQ benchmark configurations)

WORKLOADS = {
    1: "tiny 256x240 Euclidean GEMV, 25-bit indices over shells 2..3",
    2: "2-bit shape-gain GEMV 4096x4096 (q_proj-shaped), batch 1",
    3: "2-bit shape-gain GEMV pair 11008x4096 and 4096x11008 (MLP up/down), batch 1",
    4: "2-bit shape-gain small-batch GEMM 28672x8192, batch 1/4/8/16",
    5: "bulk decode-to-bf16 of a 7B-shaped weight set; 1e8-point index round trip",
}


def workload1(index_count_m3: int) -> Tensor:
    return make_tensor("c1_256x240", 1, 0, 256, 240, index_count_m3, mode=MODE_EUCLID,
                       max_shell=3, shape_bits=25, gain_bits=0, x_dtype="f32")


def workload2(index_count_m10: int, batch=1) -> Tensor:
    return make_tensor("c2_4096x4096", 2, 0, 4096, 4096, index_count_m10, batch=batch)


def workload3(index_count_m10: int, which: int, fidelity=None, batch=1) -> Tensor:
    """which = 0: 11008x4096 (rows x cols), 1: 4096x11008.  `fidelity` = (shape_idx,
    gain_idx) for the first rows, from the stored fixture."""
    rows, cols = ((11008, 4096), (4096, 11008))[which]
    return make_tensor(f"c3_{rows}x{cols}", 3, which, rows, cols, index_count_m10, batch=batch,
                       gain_scale=0.02, override_rows=fidelity)


def workload4(index_count_m10: int, batch: int) -> Tensor:
    return make_tensor("c4_28672x8192", 4, 0, 28672, 8192, index_count_m10, batch=batch)


def workload5_shapes():
    """(rows, cols) of the 7 tensors of one 7B-shaped layer, as listed: four 4096x4096
    and three 4096x11008; the weight set is 32 such layers."""
    return [(4096, 4096)] * 4 + [(4096, 11008)] * 3


def workload5_tensor(index_count_m10: int, layer: int, j: int) -> Tensor:
    rows, cols = workload5_shapes()[j]
    return make_tensor(f"c5_L{layer}_{j}", 5, layer * 8 + j, rows, cols, index_count_m10, batch=0)


def workload5_roundtrip_indices(index_count_m10: int, n: int, chunk: int = 0) -> np.ndarray:
    return rng(5, 1000 + chunk, 0).integers(0, index_count_m10, size=n, dtype=np.uint64)
