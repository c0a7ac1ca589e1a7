"""LLVQ (Leech-lattice vector quantization) decode and fused dequant-GEMV for MI355X.

Thin ctypes binding over the C ABI in include/llvq.h (libllvq.so, built in-tree by
weight_decompression_amd/build_lib.py).  Every computation runs in the HIP kernels;
this module only marshals arguments: torch tensors provide device memory and the
current HIP stream.  There is no CPU fallback: a call without the built library raises.
"""

import ctypes
import os

from .synth import MODE_EUCLID, MODE_SHAPEGAIN  # noqa: F401  (re-exported constants)

OUT_POINTS_I8 = 0
OUT_BF16 = 1
X_F32 = 0
X_BF16 = 1
SEARCH_ANGULAR = 0
SEARCH_EUCLID = 1
MAX_BATCH = 16

_ERRORS = {0: "ok", -1: "invalid argument", -2: "unsupported request", -3: "HIP launch error",
           -4: "request larger than the library's fixed workspace"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libllvq.so")
CHECKS_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libllvq_checks.so")

EXPORTED_SYMBOLS = ("llvq_index_count", "llvq_packed_bytes", "llvq_error_string",
                    "llvq_decode", "llvq_gemv", "llvq_encode_ref", "llvq_search", "llvq_quantize_workspace_bytes",
                    "llvq_quantize", "llvq_pack_fields", "llvq_decode_many",
                    "llvq_index_count_wide", "llvq_encode_wide", "llvq_quantize_noalloc",
                    "llvq_quantize_noalloc_max_blocks", "llvq_gptq_workspace_bytes", "llvq_gptq_factor",
                    "llvq_gptq_begin", "llvq_gptq_column", "llvq_device_checks")


class LlvqError(RuntimeError):
    def __init__(self, code, call):
        super().__init__(f"{call} failed: {_ERRORS.get(code, 'unknown')} ({code})")
        self.code = code


class Desc(ctypes.Structure):
    """llvq_desc: one packed weight tensor [rows][cols]."""
    _fields_ = [("mode", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("max_shell", ctypes.c_int32), ("shape_bits", ctypes.c_int32), ("gain_bits", ctypes.c_int32)]

    def __repr__(self):
        return (f"Desc(mode={self.mode}, rows={self.rows}, cols={self.cols}, max_shell={self.max_shell}, "
                f"shape_bits={self.shape_bits}, gain_bits={self.gain_bits})")


_libs = {}


def load_library(path=LIB_PATH):
    """Load libllvq.so (raises if it has not been built).

    torch is imported first: PyTorch wheels carry their own HIP runtime, and the
    library must bind to the same runtime as the streams and device pointers it is
    handed (loaded first, it would bind to the system runtime and every launch on a
    torch stream would fail)."""
    path = os.path.abspath(path)
    if path in _libs:
        return _libs[path]
    import torch  # noqa: F401  (selects the process's HIP runtime)
    if not os.path.exists(path):
        raise RuntimeError(f"LLVQ HIP library not found at {path}; build it with "
                           f"`python -m weight_decompression_amd.build_lib` (no CPU fallback exists)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, u64p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_uint64)
    dp = ctypes.POINTER(Desc)
    lib.llvq_index_count.argtypes = [i32, u64p]
    lib.llvq_index_count.restype = ctypes.c_int
    lib.llvq_index_count_wide.argtypes = [i32, u64p, u64p]
    lib.llvq_index_count_wide.restype = ctypes.c_int
    lib.llvq_packed_bytes.argtypes = [dp]
    lib.llvq_packed_bytes.restype = i64
    lib.llvq_error_string.argtypes = [ctypes.c_int]
    lib.llvq_error_string.restype = ctypes.c_char_p
    lib.llvq_decode.argtypes = [dp, vp, vp, i32, vp, vp, vp]
    lib.llvq_decode.restype = ctypes.c_int
    lib.llvq_gemv.argtypes = [dp, vp, vp, vp, i32, i32, vp, vp, vp]
    lib.llvq_gemv.restype = ctypes.c_int
    lib.llvq_encode_ref.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.llvq_encode_ref.restype = ctypes.c_int
    lib.llvq_encode_wide.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.llvq_encode_wide.restype = ctypes.c_int
    lib.llvq_search.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp]
    lib.llvq_search.restype = ctypes.c_int
    lib.llvq_quantize_workspace_bytes.argtypes = [dp]
    lib.llvq_quantize_workspace_bytes.restype = i64
    lib.llvq_quantize.argtypes = [dp, vp, vp, vp, vp, vp, vp]
    lib.llvq_quantize.restype = ctypes.c_int
    lib.llvq_quantize_noalloc.argtypes = [dp, vp, vp, vp, vp, vp]
    lib.llvq_quantize_noalloc.restype = ctypes.c_int
    lib.llvq_quantize_noalloc_max_blocks.argtypes = []
    lib.llvq_quantize_noalloc_max_blocks.restype = i64
    lib.llvq_gptq_workspace_bytes.argtypes = [i32]
    lib.llvq_gptq_workspace_bytes.restype = i64
    lib.llvq_gptq_factor.argtypes = [i32, vp, ctypes.c_double, vp, vp, vp, vp]
    lib.llvq_gptq_factor.restype = ctypes.c_int
    lib.llvq_gptq_begin.argtypes = [i32, i32, vp, vp, vp, vp]
    lib.llvq_gptq_begin.restype = ctypes.c_int
    lib.llvq_gptq_column.argtypes = [dp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.llvq_gptq_column.restype = ctypes.c_int
    lib.llvq_device_checks.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32]
    lib.llvq_device_checks.restype = ctypes.c_int
    lib.llvq_pack_fields.argtypes = [dp, vp, vp, vp]
    lib.llvq_pack_fields.restype = ctypes.c_int
    lib.llvq_decode_many.argtypes = [vp, i32, vp, vp, i32, vp, vp, vp]
    lib.llvq_decode_many.restype = ctypes.c_int
    _libs[path] = lib
    return lib


def _check(code, call):
    if code != 0:
        raise LlvqError(code, call)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ---------------------------------------------------------------------------
# argument checks: every tensor handed to the library is a contiguous device tensor of
# the right dtype and at least the size the call will touch, checked here before the
# library is loaded or a kernel launched (a short, strided or host buffer would
# otherwise become an out-of-bounds device access)

def _tensor(t, name, dtypes=None, min_bytes=0, nullable=False):
    import torch
    if t is None:
        if nullable:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    nbytes = t.numel() * t.element_size()
    if nbytes < min_bytes:
        raise ValueError(f"{name} holds {nbytes} bytes; the call needs at least {min_bytes}")


def _blocks(desc):
    if desc.rows <= 0 or desc.cols <= 0:
        raise ValueError(f"descriptor needs rows > 0 and cols > 0: {desc!r}")
    return desc.rows * ((desc.cols + 23) // 24)


def _packed_nbytes(desc):
    """Bytes of the packed stream (the layout of include/llvq.h: fields rounded up to a
    16-byte multiple, plus 16 bytes that kernels may over-read)."""
    from .synth import packed_nbytes
    return packed_nbytes(_blocks(desc), desc.shape_bits + desc.gain_bits)


def _scales_count(desc):
    return desc.rows if desc.mode == MODE_EUCLID else (1 << max(desc.gain_bits, 0))


def _check_decode_args(desc, packed, scales, out_kind, out, err_count, what="llvq_decode"):
    import torch
    _tensor(packed, f"{what}: packed", (torch.uint8, torch.int8), _packed_nbytes(desc))
    _tensor(err_count, f"{what}: err_count", (torch.int32,), 4, nullable=True)
    if out_kind == OUT_POINTS_I8:
        _tensor(out, f"{what}: out", (torch.int8,), _blocks(desc) * 24)
        _tensor(scales, f"{what}: scales", (torch.float16,), 0, nullable=True)
    elif out_kind == OUT_BF16:
        _tensor(out, f"{what}: out", (torch.bfloat16,), 2 * desc.rows * desc.cols)
        _tensor(scales, f"{what}: scales", (torch.float16,), 2 * _scales_count(desc))
    else:
        raise ValueError(f"{what}: out_kind must be OUT_POINTS_I8 or OUT_BF16, got {out_kind}")


def make_desc(mode, rows, cols, max_shell, shape_bits, gain_bits) -> Desc:
    return Desc(mode, rows, cols, max_shell, shape_bits, gain_bits)


def index_count(max_shell: int) -> int:
    """C_M as a Python integer (shells 2..42; past shell 33 it exceeds 64 bits)."""
    lo, hi = ctypes.c_uint64(), ctypes.c_uint64()
    _check(load_library().llvq_index_count_wide(max_shell, ctypes.byref(lo), ctypes.byref(hi)),
           "llvq_index_count_wide")
    return lo.value | (hi.value << 64)


def packed_bytes(desc: Desc) -> int:
    n = load_library().llvq_packed_bytes(ctypes.byref(desc))
    if n < 0:
        raise LlvqError(int(n), "llvq_packed_bytes")
    return n


def decode(desc, packed, scales, out_kind, out, err_count=None, stream=None):
    """Decode all blocks into `out` (int8 points [rows][Kb*24] or bf16 [rows][cols])."""
    _check_decode_args(desc, packed, scales, out_kind, out, err_count)
    _check(load_library().llvq_decode(ctypes.byref(desc), _ptr(packed), _ptr(scales), out_kind, _ptr(out),
                                      _ptr(err_count), _stream(stream)), "llvq_decode")


def gemv(desc, packed, scales, x, y, err_count=None, stream=None):
    """y[b][r] = sum_k W_hat[r][k] x[b][k]; x is fp32 or bf16 [batch][cols], y fp32 [batch][rows]."""
    import torch
    _tensor(x, "llvq_gemv: x", (torch.float32, torch.bfloat16))
    xd = X_BF16 if x.dtype == torch.bfloat16 else X_F32
    if x.dim() not in (1, 2) or x.shape[-1] != desc.cols:
        raise ValueError(f"llvq_gemv: x must be [batch][{desc.cols}] or [{desc.cols}], got {tuple(x.shape)}")
    batch = 1 if x.dim() == 1 else x.shape[0]
    if not 1 <= batch <= MAX_BATCH:
        raise ValueError(f"llvq_gemv: batch must be 1..{MAX_BATCH}, got {batch}")
    _tensor(packed, "llvq_gemv: packed", (torch.uint8, torch.int8), _packed_nbytes(desc))
    _tensor(scales, "llvq_gemv: scales", (torch.float16,), 2 * _scales_count(desc))
    _tensor(y, "llvq_gemv: y", (torch.float32,), 4 * batch * desc.rows)
    _tensor(err_count, "llvq_gemv: err_count", (torch.int32,), 4, nullable=True)
    _check(load_library().llvq_gemv(ctypes.byref(desc), _ptr(packed), _ptr(scales), _ptr(x), xd, batch, _ptr(y),
                                    _ptr(err_count), _stream(stream)), "llvq_gemv")


def _check_points(points, indices, err_count, words, what):
    import torch
    _tensor(points, f"{what}: points", (torch.int8,))
    if points.numel() % 24:
        raise ValueError(f"{what}: points must hold whole 24-vectors, got {points.numel()} values")
    n = points.numel() // 24
    _tensor(indices, f"{what}: indices", (torch.int64,), 8 * words * n)
    _tensor(err_count, f"{what}: err_count", (torch.int32,), 4, nullable=True)
    return n


def encode_ref(points, max_shell, indices, err_count=None, stream=None):
    """Rank int8 lattice points [n][24] into uint64 shape indices [n] (int64 tensor)."""
    n = _check_points(points, indices, err_count, 1, "llvq_encode_ref")
    _check(load_library().llvq_encode_ref(_ptr(points), n, max_shell, _ptr(indices), _ptr(err_count),
                                          _stream(stream)), "llvq_encode_ref")


def search(x, max_shell, objective, points, indices, err_count=None, stream=None):
    """Nearest point of shells 2..max_shell to each fp32 24-vector x [n][24]
    (SEARCH_ANGULAR or SEARCH_EUCLID): int8 points [n][24] and uint64 indices [n]
    (int64 tensor) are written."""
    import torch
    _tensor(x, "llvq_search: x", (torch.float32,))
    if x.numel() % 24:
        raise ValueError(f"llvq_search: x must hold whole 24-blocks, got {x.numel()} values")
    n = x.numel() // 24
    _tensor(points, "llvq_search: points", (torch.int8,), 24 * n)
    _tensor(indices, "llvq_search: indices", (torch.int64,), 8 * n)
    _tensor(err_count, "llvq_search: err_count", (torch.int32,), 4, nullable=True)
    _check(load_library().llvq_search(_ptr(x), n, max_shell, objective, _ptr(points), _ptr(indices),
                                      _ptr(err_count), _stream(stream)), "llvq_search")


def quantize_workspace_bytes(desc: Desc) -> int:
    n = load_library().llvq_quantize_workspace_bytes(ctypes.byref(desc))
    if n < 0:
        raise LlvqError(int(n), "llvq_quantize_workspace_bytes")
    return n


def quantize(desc, w, scales, packed, workspace, err_count=None, stream=None):
    """Quantise fp32 weights w [rows][cols] into the packed stream (uint8 tensor of
    packed_bytes(desc) bytes); workspace: quantize_workspace_bytes(desc) bytes of device memory."""
    import torch
    n = _blocks(desc)
    _tensor(w, "llvq_quantize: w", (torch.float32,), 4 * desc.rows * desc.cols)
    _tensor(scales, "llvq_quantize: scales", (torch.float16,), 2 * _scales_count(desc))
    _tensor(packed, "llvq_quantize: packed", (torch.uint8, torch.int8), _packed_nbytes(desc))
    _tensor(workspace, "llvq_quantize: workspace", None, (24 * n + 7) // 8 * 8 + 8 * n)
    _tensor(err_count, "llvq_quantize: err_count", (torch.int32,), 4, nullable=True)
    _check(load_library().llvq_quantize(ctypes.byref(desc), _ptr(w), _ptr(scales), _ptr(packed), _ptr(workspace),
                                        _ptr(err_count), _stream(stream)), "llvq_quantize")


def quantize_noalloc(desc, w, scales, packed, err_count=None, stream=None):
    """quantize() without a workspace argument: the library's own fixed device array is used
    (at most quantize_noalloc_max_blocks() blocks; calls that overlap on one GPU race)."""
    import torch
    _tensor(w, "llvq_quantize_noalloc: w", (torch.float32,), 4 * desc.rows * desc.cols)
    _tensor(scales, "llvq_quantize_noalloc: scales", (torch.float16,), 2 * _scales_count(desc))
    _tensor(packed, "llvq_quantize_noalloc: packed", (torch.uint8, torch.int8), _packed_nbytes(desc))
    _tensor(err_count, "llvq_quantize_noalloc: err_count", (torch.int32,), 4, nullable=True)
    _check(load_library().llvq_quantize_noalloc(ctypes.byref(desc), _ptr(w), _ptr(scales), _ptr(packed),
                                                _ptr(err_count), _stream(stream)), "llvq_quantize_noalloc")


def quantize_noalloc_max_blocks() -> int:
    return int(load_library().llvq_quantize_noalloc_max_blocks())


def pack_fields(desc, fields, packed, stream=None):
    """Write uint64 fields [rows * Kb] (int64 tensor) as the packed stream of desc."""
    import torch
    _tensor(fields, "llvq_pack_fields: fields", (torch.int64,), 8 * _blocks(desc))
    _tensor(packed, "llvq_pack_fields: packed", (torch.uint8, torch.int8), _packed_nbytes(desc))
    _check(load_library().llvq_pack_fields(ctypes.byref(desc), _ptr(fields), _ptr(packed), _stream(stream)),
           "llvq_pack_fields")


def decode_many(descs, packed, scales, out_kind, outs, err_count=None, stream=None):
    """llvq_decode of several tensors in one call (equal widths and shell range)."""
    n = len(descs)
    if not (len(packed) == len(outs) == n and (scales is None or len(scales) == n)):
        raise ValueError("llvq_decode_many: descs, packed, scales and outs need one entry per tensor")
    for i in range(n):
        _check_decode_args(descs[i], packed[i], None if scales is None else scales[i], out_kind, outs[i],
                           err_count, f"llvq_decode_many[{i}]")
    darr = (Desc * n)(*descs)
    parr = (ctypes.c_void_p * n)(*[p.data_ptr() for p in packed])
    sarr = None if scales is None else (ctypes.c_void_p * n)(*[x.data_ptr() for x in scales])
    oarr = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    _check(load_library().llvq_decode_many(ctypes.cast(darr, ctypes.c_void_p), n, ctypes.cast(parr, ctypes.c_void_p),
                                           None if sarr is None else ctypes.cast(sarr, ctypes.c_void_p), out_kind,
                                           ctypes.cast(oarr, ctypes.c_void_p), _ptr(err_count), _stream(stream)),
           "llvq_decode_many")


def encode_wide(points, max_shell, indices, err_count=None, stream=None):
    """llvq_encode_wide: int8 points [n][24] -> 128-bit indices as int64 pairs [n][2] (lo, hi)."""
    n = _check_points(points, indices, err_count, 2, "llvq_encode_wide")
    _check(load_library().llvq_encode_wide(_ptr(points), n, max_shell, _ptr(indices),
                                           _ptr(err_count), _stream(stream)), "llvq_encode_wide")
