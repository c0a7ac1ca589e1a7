"""The library built with its in-kernel invariant checks (LLVQ_DEVICE_CHECKS,
libllvq_checks.so) on workloads of every kernel family: the outputs equal the normal
build's byte for byte and no check fails (class and table indices in range, a positive
count for every chosen value slot, queue and ring capacities, codeword index below A).
Also the LLVQ_EHIP path, forced from the host: a HIP error left pending by a refused
allocation is reported by the next call (in a child process)."""

import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import weight_decompression_amd as wd
from oracle import leech
from weight_decompression_amd import synth

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
C10 = leech.index_count(10)


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    if not os.path.exists(wd.CHECKS_LIB_PATH):
        pytest.fail("libllvq_checks.so not built (build_lib.build(device_checks=True))")
    return wd.load_library(), wd.load_library(wd.CHECKS_LIB_PATH)


def _failures(lib, reset=True):
    torch.cuda.synchronize()
    n = ctypes.c_uint32(0)
    assert lib.llvq_device_checks(ctypes.byref(n), 1 if reset else 0) == 0
    return n.value


def _run_both(libs, monkeypatch, fn):
    """fn() with the normal library, then with the checks library (the binding's loader
    patched); returns both results and the checks library's failure count."""
    normal, checked = libs
    _failures(checked)
    a = fn()
    torch.cuda.synchronize()
    monkeypatch.setattr(wd, "load_library", lambda path=None: checked)
    b = fn()
    torch.cuda.synchronize()
    monkeypatch.undo()
    return a, b, _failures(checked)


def _dev(t):
    desc = wd.make_desc(t.mode, t.rows, t.cols, t.max_shell, t.shape_bits, t.gain_bits)
    packed = torch.from_numpy(t.packed).cuda()
    scales = torch.from_numpy(t.scales_f16.copy()).cuda()
    x = None
    if t.x_bits is not None:
        x = torch.from_numpy(t.x_bits.view(np.int16).copy()).cuda().view(torch.bfloat16)
    elif t.x_f32 is not None:
        x = torch.from_numpy(t.x_f32.copy()).cuda()
    return desc, packed, scales, x


def test_normal_build_has_no_checks(libs):
    normal, _ = libs
    n = ctypes.c_uint32(0)
    assert normal.llvq_device_checks(ctypes.byref(n), 0) == -2


@pytest.mark.parametrize("case", ["mlp_b1", "tall_b1", "q_b4", "euclid_b1"])
def test_gemv_with_checks(libs, monkeypatch, case):
    t = {"mlp_b1": lambda: synth.workload3(C10, 1, None),
         "tall_b1": lambda: synth.make_tensor("ck", 40, 1, 3001, 28800, C10),
         "q_b4": lambda: synth.make_tensor("ck", 40, 2, 700, 4096, C10, batch=4),
         "euclid_b1": lambda: synth.workload1(leech.index_count(3))}[case]()
    desc, packed, scales, x = _dev(t)

    def run():
        y = torch.full((x.shape[0], t.rows), float("nan"), dtype=torch.float32, device="cuda")
        wd.gemv(desc, packed, scales, x, y)
        return y.cpu().numpy()

    a, b, fails = _run_both(libs, monkeypatch, run)
    say(f"gemv {case}: {t.rows}x{t.cols}, check failures {fails}")
    assert fails == 0
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("kind", [wd.OUT_POINTS_I8, wd.OUT_BF16])
def test_decode_and_decode_many_with_checks(libs, monkeypatch, kind):
    ts = [synth.make_tensor("ck", 41, j, r, c, C10, batch=0)
          for j, (r, c) in enumerate([(300, 4096), (97, 11008), (2598, 11008), (5, 100)])]
    devs = [_dev(t) for t in ts]

    def outs():
        return [torch.empty((t.rows, t.kb * 24) if kind == wd.OUT_POINTS_I8 else (t.rows, t.cols),
                            dtype=torch.int8 if kind == wd.OUT_POINTS_I8 else torch.bfloat16, device="cuda")
                for t in ts]

    def run():
        o1 = outs()
        for (d, p, s, _), o in zip(devs, o1):
            wd.decode(d, p, s, kind, o)
        o2 = outs()
        wd.decode_many([d for d, _, _, _ in devs], [p for _, p, _, _ in devs], [s for _, _, s, _ in devs], kind, o2)
        return [o.view(torch.int8).cpu().numpy() for o in o1 + o2]

    a, b, fails = _run_both(libs, monkeypatch, run)
    say(f"decode kind {kind}: check failures {fails}")
    assert fails == 0
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_rank_search_and_general_decoder_with_checks(libs, monkeypatch):
    rng = np.random.default_rng(42)
    idx = synth.workload5_roundtrip_indices(C10, 100000, chunk=3)
    t = synth.Tensor("rt", synth.MODE_SHAPEGAIN, idx.size, 24, 10, 44, 4, idx.reshape(-1, 1),
                     np.zeros((idx.size, 1), dtype=np.uint64), np.ones(16, dtype=np.float16),
                     synth.pack_fields(idx, 48))
    d, p, s, _ = _dev(t)
    w3 = synth.make_wide_tensor("ck3", 42, 0, 64, 11008, wd.index_count(42), batch=1)
    d3, p3, s3, x3 = _dev(w3)
    xs = torch.from_numpy((rng.standard_normal((2048, 24)) * 0.02).astype(np.float32)).cuda()

    def run():
        pts = torch.empty((idx.size, 24), dtype=torch.int8, device="cuda")
        wd.decode(d, p, s, wd.OUT_POINTS_I8, pts)
        back = torch.empty(idx.size, dtype=torch.int64, device="cuda")
        wd.encode_ref(pts, 10, back)
        y3 = torch.empty((1, w3.rows), dtype=torch.float32, device="cuda")
        wd.gemv(d3, p3, s3, x3, y3)
        o3 = torch.empty((w3.rows, w3.cols), dtype=torch.bfloat16, device="cuda")
        wd.decode(d3, p3, s3, wd.OUT_BF16, o3)
        sp = torch.empty((2048, 24), dtype=torch.int8, device="cuda")
        si = torch.empty(2048, dtype=torch.int64, device="cuda")
        wd.search(xs, 10, wd.SEARCH_ANGULAR, sp, si)
        return [back.cpu().numpy(), y3.cpu().numpy().view(np.uint32), o3.view(torch.int16).cpu().numpy(),
                si.cpu().numpy()]

    a, b, fails = _run_both(libs, monkeypatch, run)
    say(f"rank / 3-bit decoder / search: check failures {fails}")
    assert fails == 0
    assert np.array_equal(a[0].view(np.uint64), idx)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


_PENDING_ERROR = r"""
import ctypes, sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
import weight_decompression_amd as wd
from weight_decompression_amd import synth
torch.cuda.init()
lib = wd.load_library()
hip = None
for line in open("/proc/self/maps"):
    if "libamdhip64" in line:
        hip = ctypes.CDLL(line.split()[-1])
        break
assert hip is not None
hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
t = synth.make_tensor("pe", 43, 0, 16, 240, wd.index_count(10))
desc = wd.make_desc(t.mode, t.rows, t.cols, t.max_shell, t.shape_bits, t.gain_bits)
packed = torch.from_numpy(t.packed).cuda()
scales = torch.from_numpy(t.scales_f16.copy()).cuda()
x = torch.from_numpy(t.x_bits.view(np.int16).copy()).cuda().view(torch.bfloat16)
y = torch.zeros((1, t.rows), dtype=torch.float32, device="cuda")
torch.cuda.synchronize()
p = ctypes.c_void_p()
e = hip.hipMalloc(ctypes.byref(p), 1 << 50)      # 1 PiB: refused, and left pending
args = (ctypes.byref(desc), ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
        ctypes.c_void_p(x.data_ptr()), wd.X_BF16, 1, ctypes.c_void_p(y.data_ptr()), None,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
rc1 = lib.llvq_gemv(*args)
rc2 = lib.llvq_gemv(*args)
torch.cuda.synchronize()
msg = lib.llvq_error_string(rc1).decode()
print("MALLOC", e, "RC", rc1, rc2, "finite", bool(torch.isfinite(y).all()), "MSG", msg, flush=True)
"""


def test_pending_hip_error_is_reported_once_as_ehip():
    """A HIP error left pending by an earlier call of the thread (an allocation of 1 PiB,
    refused by the runtime) comes back from the next LLVQ call as LLVQ_EHIP, which clears
    it: the call after that returns LLVQ_OK, and the launches of both were made."""
    root = os.path.dirname(HERE)
    p = subprocess.run([sys.executable, "-c", _PENDING_ERROR, root], capture_output=True, text=True, timeout=120)
    say(p.stdout.strip()[-300:])
    assert p.returncode == 0, p.stderr[-2000:]
    f = p.stdout.split()
    assert f[0] == "MALLOC" and int(f[1]) != 0
    assert f[2:6] == ["RC", "-3", "0", "finite"] and f[6] == "True"
    assert "HIP" in p.stdout.split("MSG", 1)[1]
