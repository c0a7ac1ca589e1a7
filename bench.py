#!/usr/bin/env python3
"""Benchmark of the fused LLVQ dequant-GEMV on one MI355X.

Workload: the 2-bit shape-gain MLP down-projection tensor, 4096 rows x 11008 columns
(459 Leech blocks of 24 per row, 48-bit fields = 44-bit shape index over shells 2..10 +
4-bit gain index), batch 1, bf16 activations; the first 64 rows are the stored
fidelity rows (N(0, 0.02^2) weights quantised by the CPU oracle), the rest uniform
random indices.  All inputs are seeded synthetic data (weight_decompression_amd/synth.py).

A step is one llvq_gemv call (decode of every block fused with the dot product).  The
packed tensor is replicated over >= 512 MB of device memory and the copies are used in
turn, so the 256 MB last-level cache cannot hold the weights between steps.

Output: one JSON line.  `value` is compressed-weight GB/s (6 packed bytes per block /
time per step).  `roofline` reports the bound that limits this kernel (VALU, from the
measured VALU instructions per block of the current kernel source) with the HBM figure
beside it; `cpu_baseline` times the CPU oracle on a row sample of the same tensor.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--cpu-rows R] [--no-cpu]
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "compressed-weight GB/s and % roofline, 2-bit LLVQ dequant-GEMV, batch 1, 1 MI355X"
HBM_PEAK_GBS = 8000.0                       # MI355X HBM3E, published
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12  # 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz (lane-ops/s)
ROTATE_BYTES = 512 * 1024 * 1024

# Per-kernel figures taken with rocprofv3 on the GEMV kernel built from the source whose
# sha256 is given (profiles/ holds the summaries).  When the source changes they no longer
# apply and the benchmark reports null for them.
KERNEL_PROFILE = {
    "source_sha256": "0e2b6c48e4dcb0ff5557a159e8798ae3c7a549e4419e51c49a553d867f38e1e4",
    "summary": "profiles/k_gemv_b1_4096x11008_bf16_batch1.md",
    "valu_lane_ops_per_block": 778.9,      # SQ_INSTS_VALU * 64 / blocks
    "fetch_bytes_per_launch": 12212254,    # FETCH_SIZE scaled by the copy-kernel calibration (x 1.9998)
    "write_bytes_per_launch": 32768,       # WRITE_SIZE (x 1.0000)
}


def kernel_source_sha():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_decompression_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def load_fidelity(which):
    import numpy as np
    path = os.path.join(ROOT, "tests", "golden", f"fidelity_c3_{which}.npz")
    if not os.path.exists(path):
        return None
    z = np.load(path)
    return z["shape_idx"], z["gain_idx"].astype(np.uint64)


def cpu_baseline(t, rows):
    from oracle import cpu_baseline as cb
    row_list = list(range(rows))
    x = t.x_as_f64()
    dt, procs = cb.time_gemv_rows(t.packed.tobytes(), t.rows, t.cols, t.max_shell, t.mode, t.shape_bits,
                                  t.gain_bits, t.scales_f16, t.scales_f16, x, row_list)
    nbytes = rows * t.kb * t.field_bits / 8
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": procs, "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of the same tensor ({rows * t.kb} blocks): pure-Python decode "
                      f"+ fp64 GEMV, {procs} processes, {dt:.2f} s wall"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-rows", type=int, default=192)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB mebibytes (HBM counter calibration)")
    a = ap.parse_args()

    if a.copy_calibration:
        import torch
        n = a.copy_calibration * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this LLVQ build runs on exactly one GPU (no sharding or collectives are "
              "built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import weight_decompression_amd as wd
    from weight_decompression_amd import synth

    lib = wd.load_library()
    C10 = wd.index_count(10)
    t = synth.workload3(C10, 1, load_fidelity(1), batch=1)
    desc = wd.make_desc(t.mode, t.rows, t.cols, t.max_shell, t.shape_bits, t.gain_bits)
    blocks = t.rows * t.kb
    dev = torch.device("cuda:0")

    need = wd.packed_bytes(desc)
    stride = (need + 255) // 256 * 256
    ncopies = max(2, math.ceil(ROTATE_BYTES / stride))
    big = torch.empty((ncopies, stride), dtype=torch.uint8, device=dev)
    src = torch.zeros(stride, dtype=torch.uint8)
    src[: t.packed.size] = torch.from_numpy(t.packed)
    big[:] = src.to(dev)
    scales = torch.from_numpy(t.scales_f16.copy()).to(dev)
    x = torch.from_numpy(t.x_bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    y = torch.empty((1, t.rows), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    dref = ctypes.byref(desc)
    args = [(dref, ctypes.c_void_p(big[i].data_ptr()), ctypes.c_void_p(scales.data_ptr()),
             ctypes.c_void_p(x.data_ptr()), wd.X_BF16, 1, ctypes.c_void_p(y.data_ptr()), None, sptr)
            for i in range(ncopies)]
    gemv = lib.llvq_gemv

    rc = 0
    for i in range(a.warmup):
        rc |= gemv(*args[i % ncopies])
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(a.steps):
        rc |= gemv(*args[i % ncopies])
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    if rc != 0:
        raise RuntimeError(f"llvq_gemv returned {rc}")
    ms_total = ev0.elapsed_time(ev1)
    ms = ms_total / a.steps
    sec = ms * 1e-3
    y_h = y.cpu().numpy()
    if not np.all(np.isfinite(y_h)):
        raise RuntimeError("non-finite GEMV output")

    packed_bytes = blocks * t.field_bits / 8
    alg_bytes = packed_bytes + 2 * t.cols + 4 * t.rows
    value = packed_bytes / sec / 1e9
    hbm = {"bound": "hbm", "achieved": alg_bytes / sec / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": alg_bytes / sec / 1e9 / HBM_PEAK_GBS,
           "bytes_per_launch": alg_bytes, "per_unit": "6 B packed index per 24-weight block + x + y"}
    prof_ok = KERNEL_PROFILE["source_sha256"] == kernel_source_sha()
    traffic = None
    if prof_ok and KERNEL_PROFILE["fetch_bytes_per_launch"] is not None:
        traffic = KERNEL_PROFILE["fetch_bytes_per_launch"] + KERNEL_PROFILE["write_bytes_per_launch"]
    if prof_ok and KERNEL_PROFILE["valu_lane_ops_per_block"]:
        ops = KERNEL_PROFILE["valu_lane_ops_per_block"] * blocks
        roof = {"bound": "alu", "achieved": ops / sec / 1e12, "peak": VALU_PEAK_TOPS, "unit": "TOP/s",
                "frac": ops / sec / 1e12 / VALU_PEAK_TOPS, "traffic": traffic,
                "valu_lane_ops_per_block": KERNEL_PROFILE["valu_lane_ops_per_block"],
                "profile": KERNEL_PROFILE["summary"], "hbm": hbm}
    else:
        roof = dict(hbm)
        roof["traffic"] = traffic
        roof["note"] = "VALU instructions per block not profiled for this kernel source"

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_detail": "exact integer/fp64 index decode, fp32 dot-product accumulation, bf16 x, fp16 gains",
        "data": "synthetic",
        "config": {"workload": "llvq_gemv 2-bit shape-gain 4096x11008 (MLP down-proj), batch 1",
                   "rows": t.rows, "cols": t.cols, "blocks": blocks, "field_bits": t.field_bits,
                   "max_shell": t.max_shell, "batch": 1, "rotating_copies": ncopies},
        "roofline": roof,
        "weights_per_s": t.rows * t.cols / sec,
        "wall_s_timed": wall,
    }
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(t, min(a.cpu_rows, t.rows))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
