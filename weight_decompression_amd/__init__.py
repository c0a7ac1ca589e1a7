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

_ERRORS = {0: "ok", -1: "invalid argument", -2: "unsupported request", -3: "HIP launch error"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libllvq.so")

EXPORTED_SYMBOLS = ("llvq_index_count", "llvq_packed_bytes", "llvq_error_string",
                    "llvq_decode", "llvq_gemv", "llvq_encode_ref", "llvq_search", "llvq_quantize_workspace_bytes",
                    "llvq_quantize", "llvq_pack_fields", "llvq_decode_many",
                    "llvq_index_count_wide", "llvq_encode_wide")


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
    _check(load_library().llvq_decode(ctypes.byref(desc), _ptr(packed), _ptr(scales), out_kind, _ptr(out),
                                      _ptr(err_count), _stream(stream)), "llvq_decode")


def gemv(desc, packed, scales, x, y, err_count=None, stream=None):
    """y[b][r] = sum_k W_hat[r][k] x[b][k]; x is fp32 or bf16 [batch][cols], y fp32 [batch][rows]."""
    import torch
    if x.dtype == torch.bfloat16:
        xd = X_BF16
    elif x.dtype == torch.float32:
        xd = X_F32
    else:
        raise TypeError("x must be float32 or bfloat16")
    batch = 1 if x.dim() == 1 else x.shape[0]
    _check(load_library().llvq_gemv(ctypes.byref(desc), _ptr(packed), _ptr(scales), _ptr(x), xd, batch, _ptr(y),
                                    _ptr(err_count), _stream(stream)), "llvq_gemv")


def encode_ref(points, max_shell, indices, err_count=None, stream=None):
    """Rank int8 lattice points [n][24] into uint64 shape indices [n] (int64 tensor)."""
    n = points.shape[0] if points.dim() > 1 else points.numel() // 24
    _check(load_library().llvq_encode_ref(_ptr(points), n, max_shell, _ptr(indices), _ptr(err_count),
                                          _stream(stream)), "llvq_encode_ref")


def search(x, max_shell, objective, points, indices, err_count=None, stream=None):
    """Nearest point of shells 2..max_shell to each fp32 24-vector x [n][24]
    (SEARCH_ANGULAR or SEARCH_EUCLID): int8 points [n][24] and uint64 indices [n]
    (int64 tensor) are written."""
    n = x.shape[0] if x.dim() > 1 else x.numel() // 24
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
    _check(load_library().llvq_quantize(ctypes.byref(desc), _ptr(w), _ptr(scales), _ptr(packed), _ptr(workspace),
                                        _ptr(err_count), _stream(stream)), "llvq_quantize")


def pack_fields(desc, fields, packed, stream=None):
    """Write uint64 fields [rows * Kb] (int64 tensor) as the packed stream of desc."""
    _check(load_library().llvq_pack_fields(ctypes.byref(desc), _ptr(fields), _ptr(packed), _stream(stream)),
           "llvq_pack_fields")


def decode_many(descs, packed, scales, out_kind, outs, err_count=None, stream=None):
    """llvq_decode of several tensors in one call (equal widths and shell range)."""
    n = len(descs)
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
    n = points.shape[0] if points.dim() > 1 else points.numel() // 24
    _check(load_library().llvq_encode_wide(_ptr(points), n, max_shell, _ptr(indices),
                                           _ptr(err_count), _stream(stream)), "llvq_encode_wide")
