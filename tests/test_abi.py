"""C-ABI contract checks that need no GPU: the library loads, exports every function
include/llvq.h declares, and its host-side validation rejects bad arguments before any
launch (a rejected call enqueues nothing, so these run on a CPU-only machine)."""

import ctypes
import os
import re

import pytest

import weight_decompression_amd as wd
from oracle import leech

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llvq.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(llvq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(wd.LIB_PATH):
        pytest.fail("libllvq.so is not built (run __graft_entry__.build())")
    return wd.load_library()


def test_exports_every_declared_function(lib):
    declared = header_functions()
    assert declared, "no functions found in include/llvq.h"
    assert set(declared) == set(wd.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_index_count_matches_oracle(lib):
    for M in range(2, 11):
        assert wd.index_count(M) == leech.index_count(M)
    out = ctypes.c_uint64()
    assert lib.llvq_index_count(1, ctypes.byref(out)) == -1
    assert lib.llvq_index_count(11, ctypes.byref(out)) == -1
    assert lib.llvq_index_count(10, None) == -1


def test_packed_bytes_rule(lib):
    d = wd.make_desc(wd.MODE_SHAPEGAIN, 4096, 11008, 10, 44, 4)
    nbits = 4096 * 459 * 48
    assert wd.packed_bytes(d) == (nbits // 8 + 15) // 16 * 16 + 16
    d1 = wd.make_desc(wd.MODE_EUCLID, 256, 240, 3, 25, 0)
    assert wd.packed_bytes(d1) == ((256 * 10 * 25 + 7) // 8 + 15) // 16 * 16 + 16


@pytest.mark.parametrize("bad", [
    dict(mode=2), dict(rows=0), dict(cols=-1), dict(max_shell=1),
    dict(max_shell=11),                  # C_11 > 2^44
    dict(max_shell=43, shape_bits=70),   # past the general decoder's shell range
    dict(shape_bits=43),                 # C_10 > 2^43
    dict(gain_bits=0),                   # shape-gain needs a gain field
    dict(gain_bits=9), dict(shape_bits=121),
    dict(mode=0, gain_bits=4),           # Euclidean mode has no gain field
])
def test_descriptor_validation(lib, bad):
    args = dict(mode=1, rows=8, cols=48, max_shell=10, shape_bits=44, gain_bits=4)
    args.update(bad)
    d = wd.Desc(args["mode"], args["rows"], args["cols"], args["max_shell"], args["shape_bits"], args["gain_bits"])
    assert lib.llvq_packed_bytes(ctypes.byref(d)) == -1
    dummy = ctypes.c_void_p(0x1000)
    assert lib.llvq_gemv(ctypes.byref(d), dummy, dummy, dummy, 1, 1, dummy, None, None) == -1
    assert lib.llvq_decode(ctypes.byref(d), dummy, dummy, 0, dummy, None, None) == -1


def test_pointer_and_batch_validation(lib):
    d = wd.make_desc(wd.MODE_SHAPEGAIN, 8, 48, 10, 44, 4)
    p = ctypes.c_void_p(0x10000)
    assert lib.llvq_gemv(ctypes.byref(d), None, p, p, 1, 1, p, None, None) == -1          # null packed
    assert lib.llvq_gemv(ctypes.byref(d), ctypes.c_void_p(0x10004), p, p, 1, 1, p, None, None) == -1  # misaligned
    assert lib.llvq_gemv(ctypes.byref(d), p, p, p, 1, 0, p, None, None) == -1             # batch 0
    assert lib.llvq_gemv(ctypes.byref(d), p, p, p, 1, 17, p, None, None) == -1            # batch 17
    assert lib.llvq_gemv(ctypes.byref(d), p, p, p, 7, 1, p, None, None) == -1             # bad x dtype
    assert lib.llvq_decode(ctypes.byref(d), p, p, 5, p, None, None) == -1                 # bad out kind
    assert lib.llvq_decode(ctypes.byref(d), p, None, 1, p, None, None) == -1              # bf16 needs scales
    assert lib.llvq_gemv(None, p, p, p, 1, 1, p, None, None) == -1                        # null descriptor


def test_encode_validation_and_empty(lib):
    p = ctypes.c_void_p(0x10000)
    assert lib.llvq_encode_ref(p, 10, 1, p, None, None) == -1
    assert lib.llvq_encode_ref(p, -1, 10, p, None, None) == -1
    assert lib.llvq_encode_ref(None, 10, 10, p, None, None) == -1
    assert lib.llvq_encode_ref(p, 10, 10, ctypes.c_void_p(0x10004), None, None) == -1
    assert lib.llvq_encode_ref(None, 0, 10, None, None, None) == 0                       # empty: no-op


def test_search_validation_and_empty(lib):
    p = ctypes.c_void_p(0x10000)
    assert lib.llvq_search(p, 10, 1, 0, p, p, None, None) == -1                           # max_shell < 2
    assert lib.llvq_search(p, 10, 14, 0, p, p, None, None) == -1                          # max_shell > 13
    assert lib.llvq_search(p, 10, 10, 2, p, p, None, None) == -1                          # bad objective
    assert lib.llvq_search(p, -1, 10, 0, p, p, None, None) == -1                          # negative n
    assert lib.llvq_search(None, 10, 10, 0, p, p, None, None) == -1                       # null x
    assert lib.llvq_search(p, 10, 10, 0, None, p, None, None) == -1                       # null points
    assert lib.llvq_search(p, 10, 10, 1, p, ctypes.c_void_p(0x10004), None, None) == -1   # indices alignment
    assert lib.llvq_search(ctypes.c_void_p(0x10002), 10, 10, 0, p, p, None, None) == -1   # x alignment
    assert lib.llvq_search(None, 0, 10, 0, None, None, None, None) == 0                   # empty: no-op


def test_quantize_validation(lib):
    p = ctypes.c_void_p(0x10000)
    d = wd.make_desc(wd.MODE_SHAPEGAIN, 4, 100, 10, 44, 4)
    assert lib.llvq_quantize_workspace_bytes(ctypes.byref(d)) == 4 * 5 * 32
    d3 = wd.make_desc(wd.MODE_EUCLID, 3, 25, 3, 25, 0)
    assert lib.llvq_quantize_workspace_bytes(ctypes.byref(d3)) == (3 * 2 * 24 + 7) // 8 * 8 + 3 * 2 * 8
    bad = wd.make_desc(wd.MODE_SHAPEGAIN, 4, 100, 11, 44, 4)         # C_11 > 2^44
    assert lib.llvq_quantize_workspace_bytes(ctypes.byref(bad)) == -1
    assert lib.llvq_quantize(ctypes.byref(bad), p, p, p, p, None, None) == -1
    d11 = wd.make_desc(wd.MODE_SHAPEGAIN, 4, 100, 11, 46, 2)         # shells past 10: up to 13
    assert lib.llvq_quantize_workspace_bytes(ctypes.byref(d11)) == 4 * 5 * 32
    d14 = wd.make_desc(wd.MODE_SHAPEGAIN, 4, 100, 14, 50, 4)
    assert lib.llvq_quantize_workspace_bytes(ctypes.byref(d14)) == -2
    assert lib.llvq_quantize(ctypes.byref(d), None, p, p, p, None, None) == -1                # null w
    assert lib.llvq_quantize(ctypes.byref(d), p, None, p, p, None, None) == -1                # null scales
    assert lib.llvq_quantize(ctypes.byref(d), p, p, ctypes.c_void_p(0x10008), p, None, None) == -1   # packed alignment
    assert lib.llvq_quantize(ctypes.byref(d), p, p, p, ctypes.c_void_p(0x10004), None, None) == -1   # workspace alignment
    assert lib.llvq_quantize(ctypes.byref(d), ctypes.c_void_p(0x10002), p, p, p, None, None) == -1   # w alignment
    assert lib.llvq_quantize(None, p, p, p, p, None, None) == -1


def test_error_strings(lib):
    for code in (0, -1, -2, -3, 42):
        assert isinstance(lib.llvq_error_string(code), bytes)


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not found"):
        wd.load_library(str(tmp_path / "missing.so"))


def test_pack_fields_validation(lib):
    p = ctypes.c_void_p(0x10000)
    d = wd.make_desc(wd.MODE_SHAPEGAIN, 4, 100, 10, 44, 4)
    assert lib.llvq_pack_fields(ctypes.byref(d), None, p, None) == -1
    assert lib.llvq_pack_fields(ctypes.byref(d), ctypes.c_void_p(0x10004), p, None) == -1
    assert lib.llvq_pack_fields(ctypes.byref(d), p, ctypes.c_void_p(0x10008), None) == -1
    assert lib.llvq_pack_fields(None, p, p, None) == -1


def test_decode_many_validation(lib):
    d = wd.make_desc(wd.MODE_SHAPEGAIN, 8, 48, 10, 44, 4)
    other = wd.make_desc(wd.MODE_SHAPEGAIN, 8, 48, 10, 46, 4)       # valid, other shape width
    assert lib.llvq_packed_bytes(ctypes.byref(other)) > 0
    p = ctypes.c_void_p(0x10000)

    def call(descs, n, packed=None, scales=None, kind=1, outs=None, err=None):
        darr = (wd.Desc * len(descs))(*descs)
        parr = (ctypes.c_void_p * len(descs))(*([p.value] * len(descs) if packed is None else packed))
        sarr = (ctypes.c_void_p * len(descs))(*([p.value] * len(descs) if scales is None else scales))
        oarr = (ctypes.c_void_p * len(descs))(*([p.value] * len(descs) if outs is None else outs))
        return lib.llvq_decode_many(ctypes.cast(darr, ctypes.c_void_p), n, ctypes.cast(parr, ctypes.c_void_p),
                                    ctypes.cast(sarr, ctypes.c_void_p), kind, ctypes.cast(oarr, ctypes.c_void_p),
                                    err, None)

    assert call([d], 0) == -1                                    # no tensors
    assert call([d] * 17, 17) == -1                              # more than 16
    assert call([d, other], 2) == -1                             # widths differ
    assert call([d, d], 2, kind=5) == -1                         # bad out kind
    assert call([d, d], 2, packed=[0x10000, 0x10008]) == -1      # misaligned stream
    assert call([d, d], 2, scales=[0x10000, 0]) == -1            # bf16 needs every gain table
    assert call([d, d], 2, kind=0, outs=[0x10000, 0x10002]) == -1    # int8 output not 4-aligned
    bad = wd.make_desc(wd.MODE_SHAPEGAIN, 8, 48, 10, 44, 4)
    bad.max_shell = 1
    assert call([d, bad], 2) == -1                               # invalid descriptor
    assert lib.llvq_decode_many(None, 1, p, p, 1, p, None, None) == -1


def test_wide_descriptors(lib):
    # other rates: shells past 10 and fields past 64 bits (the general decoder)
    for M in range(2, 43):
        lo, hi = ctypes.c_uint64(), ctypes.c_uint64()
        assert lib.llvq_index_count_wide(M, ctypes.byref(lo), ctypes.byref(hi)) == 0
        assert lo.value | (hi.value << 64) == leech.index_count(M)
    assert lib.llvq_index_count_wide(43, ctypes.byref(ctypes.c_uint64()), ctypes.byref(ctypes.c_uint64())) == -1
    assert wd.index_count(42) == leech.index_count(42)
    from weight_decompression_amd import synth
    for M, sb, gb in [(42, 68, 4), (12, 47, 1), (11, 46, 2), (10, 61, 3), (42, 120, 8)]:
        d = wd.make_desc(wd.MODE_SHAPEGAIN, 7, 100, M, sb, gb)
        assert lib.llvq_packed_bytes(ctypes.byref(d)) == synth.packed_nbytes(7 * 5, sb + gb)
    bad = [(42, 67, 4), (43, 70, 4), (42, 121, 4), (12, 46, 2)]     # too few shape bits, shell, width
    for M, sb, gb in bad:
        d = wd.make_desc(wd.MODE_SHAPEGAIN, 7, 100, M, sb, gb)
        assert lib.llvq_packed_bytes(ctypes.byref(d)) == -1, (M, sb, gb)
    d = wd.make_desc(wd.MODE_SHAPEGAIN, 7, 100, 42, 68, 4)
    p = ctypes.c_void_p(0x10000)
    assert lib.llvq_quantize_workspace_bytes(ctypes.byref(d)) == -2             # unsupported, not invalid
    assert lib.llvq_pack_fields(ctypes.byref(d), p, p, None) == -2
    assert lib.llvq_decode(ctypes.byref(d), ctypes.c_void_p(0x10004), p, 1, p, None, None) == -1
    assert lib.llvq_decode(ctypes.byref(d), p, None, 1, p, None, None) == -1
    assert lib.llvq_gemv(ctypes.byref(d), p, p, p, 1, 17, p, None, None) == -1
    assert lib.llvq_gemv(ctypes.byref(d), p, p, p, 3, 1, p, None, None) == -1
    e = wd.make_desc(wd.MODE_EUCLID, 7, 100, 24, 60, 1)                        # Euclidean: no gain field
    assert lib.llvq_packed_bytes(ctypes.byref(e)) == -1


def test_encode_wide_validation(lib):
    p = ctypes.c_void_p(0x10000)
    assert lib.llvq_encode_wide(p, 10, 43, p, None, None) == -1          # past shell 42
    assert lib.llvq_encode_wide(p, 10, 1, p, None, None) == -1
    assert lib.llvq_encode_wide(p, -1, 42, p, None, None) == -1
    assert lib.llvq_encode_wide(p, 10, 42, ctypes.c_void_p(0x10004), None, None) == -1
    assert lib.llvq_encode_wide(None, 0, 42, None, None, None) == 0      # empty: no-op
    assert lib.llvq_encode_ref(p, 10, 34, p, None, None) == -1           # 64-bit output: shells <= 33
