"""llvq_quantize_noalloc (the quantiser with the library's own fixed workspace) against
llvq_quantize (caller's workspace), both called through the C ABI: the packed streams
must be equal byte for byte and the error counts equal, on calls in a row whose sizes
shrink (so a call that read stale workspace contents of the previous, larger call would
show), and a request past the fixed maximum is refused before any launch."""

import ctypes

import numpy as np
import pytest
import torch

import weight_decompression_amd as wd
from weight_decompression_amd import synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _inputs(desc, seed, std, scales):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((desc.rows, desc.cols)) * std).astype(np.float32)
    w[desc.rows // 2, desc.cols // 3] = np.inf               # one invalid block, counted
    return torch.from_numpy(w).cuda(), torch.from_numpy(np.ascontiguousarray(scales, dtype=np.float16)).cuda()


def _with_workspace(lib, desc, w, s):
    pb = lib.llvq_packed_bytes(ctypes.byref(desc))
    packed = torch.full((pb,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = torch.empty(lib.llvq_quantize_workspace_bytes(ctypes.byref(desc)), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rc = lib.llvq_quantize(ctypes.byref(desc), ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(s.data_ptr()),
                           ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                           ctypes.c_void_p(err.data_ptr()), _stream())
    assert rc == 0
    torch.cuda.synchronize()
    return packed.cpu().numpy(), int(err.item())


def _no_alloc(lib, desc, w, s):
    pb = lib.llvq_packed_bytes(ctypes.byref(desc))
    packed = torch.full((pb,), 0x5A, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rc = lib.llvq_quantize_noalloc(ctypes.byref(desc), ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(s.data_ptr()),
                                   ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(err.data_ptr()), _stream())
    assert rc == 0
    torch.cuda.synchronize()
    return packed.cpu().numpy(), int(err.item())


def test_noalloc_quantize_equals_workspace_quantize_on_shrinking_calls():
    assert torch.cuda.is_available()
    lib = wd.load_library()
    max_blocks = lib.llvq_quantize_noalloc_max_blocks()
    assert max_blocks == 1 << 21
    gains = synth.draw_gain_table(3, 1, 16, 0.02)
    cases = [
        # the whole fixed workspace: 16384 rows x 128 blocks = 2^21 blocks
        ("shape-gain 44+4, 16384 x 3072 (2^21 blocks)", wd.make_desc(wd.MODE_SHAPEGAIN, 16384, 3072, 10, 44, 4),
         0.02, gains),
        # smaller, ragged, another shell range and field width
        ("shape-gain 46+2 (M = 11), 300 x 1001", wd.make_desc(wd.MODE_SHAPEGAIN, 300, 1001, 11, 46, 2), 1.0,
         synth.chi_gain_table(4)),
        # smaller still, Euclidean with per-row scales
        ("Euclidean 25-bit (M = 3), 37 x 100", wd.make_desc(wd.MODE_EUCLID, 37, 100, 3, 25, 0), 1.0,
         np.linspace(0.3, 0.6, 37)),
    ]
    for j, (label, desc, std, scales) in enumerate(cases):
        say(f"no-alloc quantise: {label}")
        w, s = _inputs(desc, 60 + j, std, scales)
        want, want_err = _with_workspace(lib, desc, w, s)
        got, got_err = _no_alloc(lib, desc, w, s)
        assert want_err == 1 and got_err == want_err, label
        assert np.array_equal(got, want), label
        # and once more: a repeated call on the same (now used) workspace gives the same
        got2, _ = _no_alloc(lib, desc, w, s)
        assert np.array_equal(got2, want), label


def test_noalloc_quantize_refuses_more_blocks_than_its_workspace():
    lib = wd.load_library()
    desc = wd.make_desc(wd.MODE_SHAPEGAIN, 16385, 3072, 10, 44, 4)      # 2^21 + 128 blocks
    dummy = torch.zeros(16, dtype=torch.uint8, device="cuda")
    rc = lib.llvq_quantize_noalloc(ctypes.byref(desc), ctypes.c_void_p(dummy.data_ptr()),
                                   ctypes.c_void_p(dummy.data_ptr()), ctypes.c_void_p(dummy.data_ptr()), None,
                                   _stream())
    assert rc == -4
    assert b"fixed workspace" in lib.llvq_error_string(rc)
