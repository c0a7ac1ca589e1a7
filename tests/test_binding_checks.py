"""The Python binding checks every tensor before the library is loaded or a kernel
launched: host tensors, wrong dtypes, strided views and buffers shorter than the call
touches are refused with an exception and never reach the C ABI.

No GPU is needed: a tensor subclass that reports itself as a GPU tensor stands in for
device memory, and the library loader is replaced by a sentinel that fails the test if
it is reached (valid arguments must reach it)."""

import pytest
import torch

import weight_decompression_amd as wd
from weight_decompression_amd import synth


class _OnGpu(torch.Tensor):
    @property
    def is_cuda(self):
        return True


def g(t):
    return torch.Tensor._make_subclass(_OnGpu, t)


class _Reached(Exception):
    pass


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def sentinel(*a, **k):
        raise _Reached()
    monkeypatch.setattr(wd, "load_library", sentinel)


DESC = wd.make_desc(wd.MODE_SHAPEGAIN, 5, 100, 10, 44, 4)       # 5 rows x 5 blocks
KB = 5
PB = synth.packed_nbytes(5 * KB, 48)


def decode_args(**over):
    a = dict(packed=g(torch.zeros(PB, dtype=torch.uint8)), scales=g(torch.ones(16, dtype=torch.float16)),
             out_kind=wd.OUT_BF16, out=g(torch.empty(5, 100, dtype=torch.bfloat16)),
             err_count=g(torch.zeros(1, dtype=torch.int32)))
    a.update(over)
    return a


def test_valid_decode_reaches_the_library():
    with pytest.raises(_Reached):
        wd.decode(DESC, **decode_args())
    with pytest.raises(_Reached):
        wd.decode(DESC, **decode_args(out_kind=wd.OUT_POINTS_I8, out=g(torch.empty(5, KB * 24, dtype=torch.int8)),
                                      scales=None, err_count=None))


@pytest.mark.parametrize("bad", [
    dict(packed=g(torch.zeros(PB - 1, dtype=torch.uint8))),                 # short stream
    dict(packed=torch.zeros(PB, dtype=torch.uint8)),                        # host memory
    dict(packed=g(torch.zeros(PB, dtype=torch.float32))),                   # wrong dtype
    dict(out=g(torch.empty(5, 99, dtype=torch.bfloat16))),                  # short output
    dict(out=g(torch.empty(100, 5, dtype=torch.bfloat16)).t()),             # strided view
    dict(out=g(torch.empty(5, 100, dtype=torch.float16))),                  # wrong dtype
    dict(scales=g(torch.ones(15, dtype=torch.float16))),                    # short gain table
    dict(scales=None),                                                      # bf16 needs scales
    dict(err_count=g(torch.zeros(1, dtype=torch.int64))),
    dict(err_count=torch.zeros(1, dtype=torch.int32)),
    dict(out_kind=7),
])
def test_bad_decode_arguments_are_refused(bad):
    with pytest.raises((ValueError, TypeError)):
        wd.decode(DESC, **decode_args(**bad))


def test_points_output_size_is_rows_times_padded_blocks():
    short = g(torch.empty(5 * 100, dtype=torch.int8))     # rows*cols, not rows*Kb*24 = 600
    with pytest.raises(ValueError):
        wd.decode(DESC, **decode_args(out_kind=wd.OUT_POINTS_I8, out=short))


def gemv_args(batch=2, **over):
    a = dict(packed=g(torch.zeros(PB, dtype=torch.uint8)), scales=g(torch.ones(16, dtype=torch.float16)),
             x=g(torch.zeros(batch, 100, dtype=torch.bfloat16)), y=g(torch.empty(batch, 5)),
             err_count=None)
    a.update(over)
    return a


def test_valid_gemv_reaches_the_library():
    with pytest.raises(_Reached):
        wd.gemv(DESC, **gemv_args())
    with pytest.raises(_Reached):
        wd.gemv(DESC, **gemv_args(batch=1, x=g(torch.zeros(100)), y=g(torch.empty(5))))


@pytest.mark.parametrize("bad", [
    dict(x=g(torch.zeros(2, 99, dtype=torch.bfloat16))),                   # wrong length
    dict(x=g(torch.zeros(17, 100, dtype=torch.bfloat16)), y=g(torch.empty(17, 5))),   # batch > 16
    dict(x=g(torch.zeros(100, 2, dtype=torch.bfloat16)).t()),              # strided
    dict(x=g(torch.zeros(2, 100, dtype=torch.float16))),                   # dtype
    dict(x=torch.zeros(2, 100, dtype=torch.bfloat16)),                     # host
    dict(y=g(torch.empty(2, 4))),                                          # short y
    dict(y=g(torch.empty(2, 5, dtype=torch.float64))),
    dict(packed=g(torch.zeros(PB - 16, dtype=torch.uint8))),
])
def test_bad_gemv_arguments_are_refused(bad):
    with pytest.raises((ValueError, TypeError)):
        wd.gemv(DESC, **gemv_args(**bad))


def test_euclid_scales_are_per_row():
    d = wd.make_desc(wd.MODE_EUCLID, 5, 100, 3, 25, 0)
    pb = synth.packed_nbytes(5 * KB, 25)
    args = gemv_args(packed=g(torch.zeros(pb, dtype=torch.uint8)), scales=g(torch.ones(4, dtype=torch.float16)))
    with pytest.raises(ValueError):
        wd.gemv(d, **args)
    args["scales"] = g(torch.ones(5, dtype=torch.float16))
    with pytest.raises(_Reached):
        wd.gemv(d, **args)


def test_rank_search_quantize_pack_checks():
    pts = g(torch.zeros(10, 24, dtype=torch.int8))
    with pytest.raises(_Reached):
        wd.encode_ref(pts, 10, g(torch.empty(10, dtype=torch.int64)))
    for bad in (g(torch.empty(9, dtype=torch.int64)), g(torch.empty(10, dtype=torch.int32)),
                torch.empty(10, dtype=torch.int64)):
        with pytest.raises((ValueError, TypeError)):
            wd.encode_ref(pts, 10, bad)
    with pytest.raises(ValueError):
        wd.encode_ref(g(torch.zeros(10 * 24 + 1, dtype=torch.int8)), 10, g(torch.empty(11, dtype=torch.int64)))
    with pytest.raises(ValueError):
        wd.encode_wide(pts, 42, g(torch.empty(19, dtype=torch.int64)))       # needs 2 words per point
    with pytest.raises(_Reached):
        wd.encode_wide(pts, 42, g(torch.empty(10, 2, dtype=torch.int64)))

    x = g(torch.zeros(10, 24))
    with pytest.raises(_Reached):
        wd.search(x, 10, wd.SEARCH_ANGULAR, pts, g(torch.empty(10, dtype=torch.int64)))
    with pytest.raises(ValueError):
        wd.search(x, 10, wd.SEARCH_ANGULAR, g(torch.zeros(9, 24, dtype=torch.int8)),
                  g(torch.empty(10, dtype=torch.int64)))

    n = 5 * KB
    ws = (24 * n + 7) // 8 * 8 + 8 * n
    qa = dict(w=g(torch.zeros(5, 100)), scales=g(torch.ones(16, dtype=torch.float16)),
              packed=g(torch.zeros(PB, dtype=torch.uint8)), workspace=g(torch.zeros(ws, dtype=torch.uint8)))
    with pytest.raises(_Reached):
        wd.quantize(DESC, **qa)
    for k, bad in (("workspace", g(torch.zeros(ws - 1, dtype=torch.uint8))), ("w", g(torch.zeros(5, 99))),
                   ("packed", g(torch.zeros(PB - 1, dtype=torch.uint8)))):
        with pytest.raises(ValueError):
            wd.quantize(DESC, **dict(qa, **{k: bad}))

    with pytest.raises(_Reached):
        wd.pack_fields(DESC, g(torch.zeros(n, dtype=torch.int64)), g(torch.zeros(PB, dtype=torch.uint8)))
    with pytest.raises(ValueError):
        wd.pack_fields(DESC, g(torch.zeros(n - 1, dtype=torch.int64)), g(torch.zeros(PB, dtype=torch.uint8)))


def test_decode_many_checks_every_tensor():
    a = decode_args()
    with pytest.raises(_Reached):
        wd.decode_many([DESC, DESC], [a["packed"]] * 2, [a["scales"]] * 2, wd.OUT_BF16, [a["out"]] * 2)
    with pytest.raises(ValueError):
        wd.decode_many([DESC, DESC], [a["packed"], g(torch.zeros(8, dtype=torch.uint8))], [a["scales"]] * 2,
                       wd.OUT_BF16, [a["out"]] * 2)
    with pytest.raises(ValueError):
        wd.decode_many([DESC, DESC], [a["packed"]], [a["scales"]] * 2, wd.OUT_BF16, [a["out"]] * 2)


def test_python_packed_size_equals_the_library_s():
    import ctypes
    lib = ctypes.CDLL(wd.LIB_PATH)
    lib.llvq_packed_bytes.argtypes = [ctypes.POINTER(wd.Desc)]
    lib.llvq_packed_bytes.restype = ctypes.c_int64
    for d in (DESC, wd.make_desc(wd.MODE_EUCLID, 256, 240, 3, 25, 0), wd.make_desc(wd.MODE_SHAPEGAIN, 37, 1001, 10, 44, 4),
              wd.make_desc(wd.MODE_SHAPEGAIN, 3, 11008, 42, 68, 4), wd.make_desc(wd.MODE_SHAPEGAIN, 7, 30, 11, 46, 2)):
        assert wd._packed_nbytes(d) == lib.llvq_packed_bytes(ctypes.byref(d)), d
