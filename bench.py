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
       python bench.py --workload {gemv_11008x4096,gemv_4096x4096,gemv_28672x8192} [--batch B]
       python bench.py --workload decode_bf16_7b [--layers 32]
       python bench.py --workload roundtrip [--points 100000000]
       python bench.py --workload search [--cpu-blocks 2048]
       python bench.py --workload fidelity [--fidelity-blocks 262144]
       python bench.py --workload gptq [--cpu-rows-gptq 8]
The other workloads print one line each in the same format (their own metric).
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

# Per-workload figures taken with rocprofv3 on the kernels built from the source whose
# sha256 is given (profiles/ holds the summaries).  When the source changes they no longer
# apply and the benchmark reports null for them.
KERNEL_PROFILES = {
    "gemv_4096x11008_b1": {
        "source_sha256": "8877de305f525f4a766bb6a5487c5916aa86d556825e37247766f369a2b9645e",
        "summary": "profiles/gemv_4096x11008_batch1_k_gemv_b1.md",
        "unit_of_work": "24-weight block (k_gemv_b1)",
        "valu_lane_ops_per_unit": 514.9,       # SQ_INSTS_VALU * 64 / blocks
        "valu_mix_peak_tops": 38.26,           # peak for the executed instruction mix
        "fetch_bytes_per_launch": 13230938,    # FETCH_SIZE scaled by the copy-kernel calibration
        "write_bytes_per_launch": 16384,       # WRITE_SIZE, same calibration
    },
    "gemv_11008x4096_b1": {
        "source_sha256": "8877de305f525f4a766bb6a5487c5916aa86d556825e37247766f369a2b9645e",
        "summary": "profiles/gemv_11008x4096_batch1_k_gemv_b1.md",
        "unit_of_work": "24-weight block (k_gemv_b1)",
        "valu_lane_ops_per_unit": 520.2,
        "valu_mix_peak_tops": 38.32,
        "fetch_bytes_per_launch": 13134686,
        "write_bytes_per_launch": 51200,
    },
    "gemv_4096x4096_b1": {
        "source_sha256": "8877de305f525f4a766bb6a5487c5916aa86d556825e37247766f369a2b9645e",
        "summary": "profiles/gemv_4096x4096_batch1_k_gemv_b1.md",
        "unit_of_work": "24-weight block (k_gemv_b1)",
        "valu_lane_ops_per_unit": 566.4,
        "valu_mix_peak_tops": 38.46,
        "fetch_bytes_per_launch": 6043133,
        "write_bytes_per_launch": 16384,
    },
    "gemv_28672x8192_b1": {
        "source_sha256": "8877de305f525f4a766bb6a5487c5916aa86d556825e37247766f369a2b9645e",
        "summary": "profiles/gemv_28672x8192_batch1_k_gemv_b1.md",
        "unit_of_work": "24-weight block (k_gemv_b1)",
        "valu_lane_ops_per_unit": 502.0,
        "valu_mix_peak_tops": 38.22,
        "fetch_bytes_per_launch": 60834186,
        "write_bytes_per_launch": 131072,
    },
    "gemv_28672x8192_b4": {
        "source_sha256": "8877de305f525f4a766bb6a5487c5916aa86d556825e37247766f369a2b9645e",
        "summary": "profiles/gemv_28672x8192_batch4_k_gemm_mfma.md",
        "unit_of_work": "24-weight block (k_gemm_mfma)",
        "valu_lane_ops_per_unit": 605.3,
        "valu_mix_peak_tops": 37.99,
        "fetch_bytes_per_launch": 61185676,
        "write_bytes_per_launch": 458752,
    },
    "gemv_28672x8192_b8": {
        "source_sha256": "8877de305f525f4a766bb6a5487c5916aa86d556825e37247766f369a2b9645e",
        "summary": "profiles/gemv_28672x8192_batch8_k_gemm_mfma.md",
        "unit_of_work": "24-weight block (k_gemm_mfma)",
        "valu_lane_ops_per_unit": 605.3,
        "valu_mix_peak_tops": 37.99,
        "fetch_bytes_per_launch": 61709903,
        "write_bytes_per_launch": 917504,
    },
    "gemv_28672x8192_b16": {
        "source_sha256": "8877de305f525f4a766bb6a5487c5916aa86d556825e37247766f369a2b9645e",
        "summary": "profiles/gemv_28672x8192_batch16_k_gemm_mfma.md",
        "unit_of_work": "24-weight block (k_gemm_mfma)",
        "valu_lane_ops_per_unit": 605.3,
        "valu_mix_peak_tops": 37.99,
        "fetch_bytes_per_launch": 62758155,
        "write_bytes_per_launch": 1835008,
    },
    "gemv_3bit_b1": {
        "source_sha256": "8877de305f525f4a766bb6a5487c5916aa86d556825e37247766f369a2b9645e",
        "summary": "profiles/gemv_3bit_4096x11008_batch1_k_gemv_wide_tile.md",
        "unit_of_work": "24-weight block (k_gemv_wide_tile)",
        "valu_lane_ops_per_unit": 2011.9,
        "valu_mix_peak_tops": 36.07,
        "fetch_bytes_per_launch": 32999272,
        "write_bytes_per_launch": 16384,
    },
    "decode_3bit": {
        "source_sha256": "8877de305f525f4a766bb6a5487c5916aa86d556825e37247766f369a2b9645e",
        "summary": "profiles/decode_bf16_3bit_4096x11008_k_decode_wide_tile.md",
        "unit_of_work": "24-weight block (k_decode_wide_tile<bf16>)",
        "valu_lane_ops_per_unit": 2022.0,
        "valu_mix_peak_tops": 35.83,
        "fetch_bytes_per_launch": 44150320,
        "write_bytes_per_launch": 90177536,
    },
    "decode_bf16": {
        "source_sha256": "8877de305f525f4a766bb6a5487c5916aa86d556825e37247766f369a2b9645e",
        "summary": "profiles/decode_bf16_7b_k_decode_stream.md",
        "unit_of_work": "24-weight block (k_decode_stream<bf16>)",
        "valu_lane_ops_per_unit": 611.8,
        "valu_mix_peak_tops": 38.42,
        "fetch_bytes_per_launch": 102449744,           # one launch = two layers (14 tensors)
        "write_bytes_per_launch": 1030306424,
    },
    "roundtrip": {
        "source_sha256": "8877de305f525f4a766bb6a5487c5916aa86d556825e37247766f369a2b9645e",
        "summary": "profiles/roundtrip_1e7_k_decode_stream_k_rank.md",
        "unit_of_work": "point: decode to int8 (548.0) + rank (951.2)",
        "valu_lane_ops_per_unit": 1499.2,
        # the two kernels' mix peaks (38.77, 36.48) weighted by their lane-ops
        "valu_mix_peak_tops": 37.32,
        "fetch_bytes_per_launch": None,        # two kernels per step; see the summary
        "write_bytes_per_launch": None,
    },
    "search": {
        "source_sha256": "8877de305f525f4a766bb6a5487c5916aa86d556825e37247766f369a2b9645e",
        "summary": "profiles/search_4096x4096_k_search_k_rank.md",
        # The search issues more VALU instructions per clock than one per CU (mostly fp32
        # fma / max / compares), and more than the harmonic mix of single-instruction
        # rates allows (utilisation 1.27 against it: such classes co-issue), so its peak
        # is the fastest measured single-instruction rate, 1.464 x 39.32 T lane-ops/s.
        "valu_peak_tops": 57.56,
        "unit_of_work": "24-block: search (3375276.2) + rank (955.4)",
        "valu_lane_ops_per_unit": 3376231.6,
        "fetch_bytes_per_launch": None,        # two kernels per step; see the summary
        "write_bytes_per_launch": None,
    },
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
    """The oracle GEMV of rows 0..rows-1 of tensor t, timed on the host cores: the baseline
    dict and the oracle's fp64 (y, sum of |terms|) for the parity check."""
    from oracle import cpu_baseline as cb, parallel
    row_list = list(range(rows))
    x = t.x_as_f64()
    dt, procs, y, mag = cb.time_gemv_rows(t.packed.tobytes(), t.rows, t.cols, t.max_shell, t.mode, t.shape_bits,
                                          t.gain_bits, t.scales_f16, t.scales_f16, x, row_list)
    nbytes = rows * t.kb * t.field_bits / 8
    base = {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": procs, "kind": "oracle",
            "cpu_model": parallel.cpu_model(),
            "sample": f"rows 0..{rows - 1} of the same tensor ({rows * t.kb} blocks): pure-Python decode "
                      f"+ fp64 GEMV, {procs} processes, {dt:.2f} s wall"}
    return base, y, mag


def gemv_parity(y_gpu, y_ref, mag, rows_checked, what):
    """Parity verdict of a GEMV output against the oracle: every checked output within
    1e-4 of the fp64 result, normalised by the sum of |terms| of its row."""
    import numpy as np
    from oracle import reference
    e = reference.normalized_errors(np.asarray(y_gpu, dtype=np.float64), y_ref, mag)
    return {"what": what, "rows_checked": int(rows_checked), "outputs_checked": int(e.size),
            "max_norm_err": float(e.max()), "tol": reference.GEMV_REL_TOL,
            "pass": bool(np.all(reference.gemv_within_tolerance(y_gpu, y_ref, mag)))}


def time_steps(launch, steps, warmup, stream):
    """Run `launch(i)` warmup times, then time `steps` calls with HIP events on `stream`."""
    import torch
    rc = 0
    for i in range(warmup):
        rc |= launch(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        rc |= launch(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    if rc != 0:
        raise RuntimeError(f"llvq call returned {rc}")
    return ev0.elapsed_time(ev1) / steps * 1e-3, wall


def roofline(profile_key, ops_units, sec, alg_bytes, per_unit_text, launches=1):
    """VALU roofline from the profiled lane-op count of the current source, with the HBM figure beside it.
    ops_units and alg_bytes cover one step of `launches` launches."""
    hbm = {"bound": "hbm", "achieved": alg_bytes / sec / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": alg_bytes / sec / 1e9 / HBM_PEAK_GBS, "bytes_per_launch": alg_bytes / launches,
           "per_unit": per_unit_text}
    if launches != 1:
        hbm["launches_per_step"] = launches
    prof = KERNEL_PROFILES.get(profile_key, {})
    prof_ok = prof.get("source_sha256") == kernel_source_sha()
    traffic = None
    if prof_ok and prof.get("fetch_bytes_per_launch") is not None:
        traffic = prof["fetch_bytes_per_launch"] + prof["write_bytes_per_launch"]
    if prof_ok and prof.get("valu_lane_ops_per_unit"):
        ops = prof["valu_lane_ops_per_unit"] * ops_units
        peak = prof.get("valu_peak_tops", VALU_PEAK_TOPS)
        out = {"bound": "alu", "achieved": ops / sec / 1e12, "peak": peak, "unit": "TOP/s",
               "frac": ops / sec / 1e12 / peak, "traffic": traffic,
               "valu_lane_ops_per_unit": prof["valu_lane_ops_per_unit"], "unit_of_work": prof["unit_of_work"],
               "profile": prof["summary"], "hbm": hbm}
        if prof.get("valu_mix_peak_tops"):
            # the peak weighted by the kernel's executed instruction mix (per-type SQ counters,
            # measured issue rates): the same achieved rate against it
            out["mix_peak"] = prof["valu_mix_peak_tops"]
            out["frac_mix"] = ops / sec / 1e12 / prof["valu_mix_peak_tops"]
        return out
    roof = dict(hbm)
    roof["traffic"] = traffic
    roof["note"] = "VALU instructions not profiled for this kernel source"
    return roof


def base_line(metric, value, unit, steps, warmup, sec, dtype, workload, extra_cfg):
    cfg = {"workload": workload}
    cfg.update(extra_cfg)
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": sec * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": dtype, "data": "synthetic", "config": cfg}


def rotating_copies(packed, nbytes_min):
    """Device copies of a packed stream spanning >= nbytes_min bytes (so the LLC cannot hold them)."""
    import torch
    stride = (packed.size + 255) // 256 * 256
    ncopies = max(2, math.ceil(nbytes_min / stride))
    big = torch.empty((ncopies, stride), dtype=torch.uint8, device="cuda:0")
    src = torch.zeros(stride, dtype=torch.uint8)
    src[: packed.size] = torch.from_numpy(packed)
    big[:] = src.to("cuda:0")
    return big


def run_gemv(a, name, t, profile_key, label):
    """Time llvq_gemv on one packed tensor (rotating copies) and build its JSON line."""
    import numpy as np
    import torch
    import weight_decompression_amd as wd

    lib = wd.load_library()
    desc = wd.make_desc(t.mode, t.rows, t.cols, t.max_shell, t.shape_bits, t.gain_bits)
    batch = t.x_bits.shape[0] if t.x_bits is not None else t.x_f32.shape[0]
    blocks = t.rows * t.kb
    big = rotating_copies(t.packed, ROTATE_BYTES)
    ncopies = big.shape[0]
    scales = torch.from_numpy(t.scales_f16.copy()).cuda()
    if t.x_bits is not None:
        x = torch.from_numpy(t.x_bits.view(np.int16).copy()).cuda().view(torch.bfloat16)
        xk, xb = wd.X_BF16, 2
    else:
        x = torch.from_numpy(t.x_f32.copy()).cuda()
        xk, xb = wd.X_F32, 4
    y = torch.empty((batch, t.rows), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    dref = ctypes.byref(desc)
    args = [(dref, ctypes.c_void_p(big[i].data_ptr()), ctypes.c_void_p(scales.data_ptr()),
             ctypes.c_void_p(x.data_ptr()), xk, batch, ctypes.c_void_p(y.data_ptr()), None, sptr)
            for i in range(ncopies)]
    gemv = lib.llvq_gemv
    sec, wall = time_steps(lambda i: gemv(*args[i % ncopies]), a.steps, a.warmup, stream)
    y_host = y.cpu().numpy()
    packed_bytes = blocks * t.field_bits / 8
    alg_bytes = packed_bytes + xb * t.cols * batch + 4 * t.rows * batch
    out = base_line(METRIC if name == DEFAULT_WORKLOAD else
                    f"compressed-weight GB/s, LLVQ dequant-GEMV, batch {batch}, 1 MI355X",
                    packed_bytes / sec / 1e9, "GB/s", a.steps, a.warmup, sec, "f32", label,
                    {"rows": t.rows, "cols": t.cols, "blocks": blocks, "field_bits": t.field_bits,
                     "max_shell": t.max_shell, "batch": batch, "rotating_copies": ncopies})
    out["dtype_detail"] = "exact integer/fp64 index decode, fp32 accumulation, " + \
        ("bf16" if xk == wd.X_BF16 else "fp32") + " x, fp16 scales"
    out["roofline"] = roofline(profile_key, blocks, sec, alg_bytes,
                               f"{t.field_bits / 8:g} B packed index per 24-weight block + x + y")
    out["weights_per_s"] = t.rows * t.cols * batch / sec
    out["wall_s_timed"] = wall
    if name == DEFAULT_WORKLOAD and not a.no_cpu:
        rows = min(a.cpu_rows, t.rows)
        out["cpu_baseline"], y_ref, mag = cpu_baseline(t, rows)
        out["parity"] = gemv_parity(y_host[:, :rows], y_ref, mag, rows,
                                    f"rows 0..{rows - 1} of the timed output vs the fp64 oracle (cpu_baseline leg)")
    else:
        from oracle import parallel
        rng = np.random.default_rng(7)
        k = min(a.parity_rows, t.rows)
        rows = sorted(set([0, t.rows - 1] + [int(r) for r in rng.choice(t.rows, k, replace=False)]))
        y_ref, mag = parallel.gemv_rows(t.packed.tobytes(), t.rows, t.cols, t.max_shell, t.mode, t.shape_bits,
                                        t.gain_bits, t.scales_f16, t.scales_f16, t.x_as_f64(), rows)
        out["parity"] = gemv_parity(y_host[:, rows], y_ref, mag, len(rows),
                                    f"{len(rows)} seeded rows of the timed output vs the fp64 oracle")
    return out


def run_decode_7b(a):
    """Bulk decode-to-bf16 of 32 layers x (4 x 4096x4096 + 3 x 4096x11008)."""
    import torch
    import weight_decompression_amd as wd
    from weight_decompression_amd import synth

    lib = wd.load_library()
    C10 = wd.index_count(10)
    layers = a.layers
    items = []
    host = []
    blocks = 0
    weights = 0
    for L in range(layers):
        for j in range(len(synth.workload5_shapes())):
            t = synth.workload5_tensor(C10, L, j)
            desc = wd.make_desc(t.mode, t.rows, t.cols, t.max_shell, t.shape_bits, t.gain_bits)
            packed = torch.from_numpy(t.packed).cuda()
            scales = torch.from_numpy(t.scales_f16.copy()).cuda()
            out = torch.empty((t.rows, t.cols), dtype=torch.bfloat16, device="cuda:0")
            items.append((desc, packed, scales, out))
            host.append((t.packed.tobytes(), t.rows, t.cols, t.max_shell, t.mode, t.shape_bits, t.gain_bits,
                         t.scales_f16, None))
            blocks += t.rows * t.kb
            weights += t.rows * t.cols
        print(f"bench: layer {L} generated", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    if a.many > 0:
        # llvq_decode_many over groups of a.many tensors (host argument arrays built once)
        calls, keep = [], []
        for g0 in range(0, len(items), a.many):
            grp = items[g0:g0 + a.many]
            n = len(grp)
            darr = (wd.Desc * n)(*[d for d, _, _, _ in grp])
            parr = (ctypes.c_void_p * n)(*[p.data_ptr() for _, p, _, _ in grp])
            sarr = (ctypes.c_void_p * n)(*[s.data_ptr() for _, _, s, _ in grp])
            oarr = (ctypes.c_void_p * n)(*[o.data_ptr() for _, _, _, o in grp])
            calls.append((ctypes.cast(darr, ctypes.c_void_p), n, ctypes.cast(parr, ctypes.c_void_p),
                          ctypes.cast(sarr, ctypes.c_void_p), wd.OUT_BF16, ctypes.cast(oarr, ctypes.c_void_p),
                          None, sptr))
            keep.append((darr, parr, sarr, oarr))
        dec = lib.llvq_decode_many
    else:
        calls = [(ctypes.byref(d), ctypes.c_void_p(p.data_ptr()), ctypes.c_void_p(s.data_ptr()), wd.OUT_BF16,
                  ctypes.c_void_p(o.data_ptr()), None, sptr) for d, p, s, o in items]
        dec = lib.llvq_decode

    def step(_):
        rc = 0
        for c in calls:
            rc |= dec(*c)
        return rc

    sec, wall = time_steps(step, a.steps, a.warmup, stream)
    packed_bytes = blocks * 6
    alg_bytes = packed_bytes + 2 * weights
    out = base_line("bulk LLVQ decode-to-bf16 throughput, 7B-shaped weight set, 1 MI355X",
                    weights / sec, "weights/s", a.steps, a.warmup, sec, "f32",
                    (f"llvq_decode_many bf16, {a.many} tensors per call" if a.many > 0 else "llvq_decode bf16")
                    + f", {layers} layers x (4 x 4096x4096 + 3 x 4096x11008)",
                    {"layers": layers, "tensors": len(items), "tensors_per_call": max(a.many, 1), "blocks": blocks,
                     "weights": weights, "packed_bytes": packed_bytes, "bf16_bytes": 2 * weights})
    out["compressed_GBps"] = packed_bytes / sec / 1e9
    out["bf16_written_GBps"] = 2 * weights / sec / 1e9
    out["roofline"] = roofline("decode_bf16", blocks, sec, alg_bytes,
                               "6 B packed index read + 48 B bf16 written per 24-weight block", launches=len(calls))
    out["wall_s_timed"] = wall
    # parity: two seeded rows of every tensor, bit for bit against the oracle's bf16 decode
    import numpy as np
    from oracle import parallel
    rng = np.random.default_rng(5)
    pairs = [(i, int(r)) for i in range(len(items)) for r in rng.choice(items[i][0].rows, 2, replace=False)]
    want = parallel.decode_rows_bf16_many(host, pairs)
    bad = 0
    for (i, r), ref in zip(pairs, want):
        got = items[i][3][r].view(torch.int16).cpu().numpy().view(np.uint16)
        bad += int(not np.array_equal(got, ref))
    out["parity"] = {"what": "2 seeded rows of each of the tensors, bf16 bit patterns vs the oracle",
                     "rows_checked": len(pairs), "rows_differing": bad, "pass": bad == 0}
    return out


def run_decode_3bit(a):
    """Decode-to-bf16 of a 4096 x 11008 tensor at 3 bits per weight (68 + 4-bit fields,
    shells 2..42), through the general decoder."""
    import torch
    import weight_decompression_amd as wd
    from weight_decompression_amd import synth

    lib = wd.load_library()
    t = synth.make_wide_tensor("dec3", 10, 0, 4096, 11008, wd.index_count(42), batch=0)
    desc = wd.make_desc(t.mode, t.rows, t.cols, t.max_shell, t.shape_bits, t.gain_bits)
    packed = torch.from_numpy(t.packed).cuda()
    scales = torch.from_numpy(t.scales_f16.copy()).cuda()
    out = torch.empty((t.rows, t.cols), dtype=torch.bfloat16, device="cuda:0")
    stream = torch.cuda.current_stream()
    args = (ctypes.byref(desc), ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(scales.data_ptr()), wd.OUT_BF16,
            ctypes.c_void_p(out.data_ptr()), None, ctypes.c_void_p(stream.cuda_stream))
    sec, wall = time_steps(lambda i: lib.llvq_decode(*args), a.steps, a.warmup, stream)
    blocks = t.rows * t.kb
    weights = t.rows * t.cols
    alg_bytes = blocks * t.field_bits / 8 + 2 * weights
    res = base_line("LLVQ decode-to-bf16 throughput at 3 bits per weight, 1 MI355X", weights / sec, "weights/s",
                    a.steps, a.warmup, sec, "f32",
                    "llvq_decode bf16, 4096x11008, 68+4-bit fields (shells 2..42), general decoder",
                    {"rows": t.rows, "cols": t.cols, "blocks": blocks, "field_bits": t.field_bits, "max_shell": 42})
    res["roofline"] = roofline("decode_3bit", blocks, sec, alg_bytes,
                               "9 B packed index read + 48 B bf16 written per 24-weight block")
    res["wall_s_timed"] = wall
    # parity: seeded rows of the timed output, bf16 bit patterns vs the oracle's decode
    import numpy as np
    from oracle import parallel
    rows = sorted(set([0, t.rows - 1] + [int(r) for r in np.random.default_rng(9).choice(t.rows, 14, replace=False)]))
    ref = parallel.decode_rows_bf16(t.packed.tobytes(), t.rows, t.cols, 42, t.mode, t.shape_bits, t.gain_bits,
                                    t.scales_f16, None, rows)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    bad = int(np.sum(np.any(got != ref, axis=1)))
    res["parity"] = {"what": f"{len(rows)} seeded rows of the timed output, bf16 bit patterns vs the oracle",
                     "rows_checked": len(rows), "rows_differing": bad, "pass": bad == 0}
    return res


def run_roundtrip(a):
    """Index -> point -> index round trip on n uniform indices over shells 2..10."""
    import numpy as np
    import torch
    import weight_decompression_amd as wd
    from weight_decompression_amd import synth

    lib = wd.load_library()
    C10 = wd.index_count(10)
    n = a.points
    kb = 1000
    rows = (n + kb - 1) // kb
    n = rows * kb
    idx = synth.workload5_roundtrip_indices(C10, n)
    packed = synth.pack_fields(idx, 48)
    sample = np.random.default_rng(6).choice(n, min(a.parity_points, n), replace=False)
    sample_idx = idx[sample]
    del idx
    desc = wd.make_desc(wd.MODE_SHAPEGAIN, rows, kb * 24, 10, 44, 4)
    pk = torch.from_numpy(packed).cuda()
    ref = torch.from_numpy(packed[: n * 6].view(np.uint8)).cuda()
    del packed
    scales = torch.ones(16, dtype=torch.float16, device="cuda:0")
    pts = torch.empty((n, 24), dtype=torch.int8, device="cuda:0")
    back = torch.empty(n, dtype=torch.int64, device="cuda:0")
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def step(_):
        rc = lib.llvq_decode(ctypes.byref(desc), ctypes.c_void_p(pk.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                             wd.OUT_POINTS_I8, ctypes.c_void_p(pts.data_ptr()), ctypes.c_void_p(err.data_ptr()), sptr)
        rc |= lib.llvq_encode_ref(ctypes.c_void_p(pts.data_ptr()), n, 10, ctypes.c_void_p(back.data_ptr()),
                                  ctypes.c_void_p(err.data_ptr()), sptr)
        return rc

    sec, wall = time_steps(step, a.steps, a.warmup, stream)
    # the round trip must reproduce every index: compare the low 48 bits of the packed field
    b8 = back.view(torch.uint8).view(n, 8)[:, :6].reshape(-1)
    ok = bool(torch.equal(b8, ref)) and int(err.item()) == 0
    out = base_line("LLVQ index->point->index round trip throughput, 1 MI355X", n / sec, "points/s",
                    a.steps, a.warmup, sec, "int64",
                    f"llvq_decode points + llvq_encode_ref, {n} uniform indices over shells 2..10",
                    {"points": n})
    out["round_trip_exact"] = ok
    from oracle import parallel
    want = parallel.unrank_many(sample_idx, 10)
    got = pts[torch.from_numpy(sample).cuda()].cpu().numpy().astype(np.int64)
    out["parity"] = {"what": f"{len(sample)} seeded points of the timed decode vs the oracle's unrank, and every "
                             f"index equal after the rank", "points_checked": int(len(sample)),
                     "round_trip_exact": ok, "pass": bool(ok and np.array_equal(got, want))}
    out["roofline"] = roofline("roundtrip", n, sec, n * (6 + 24 + 24 + 8),
                               "6 B index read + 24 B point written (decode); 24 B read + 8 B written (rank)")
    out["wall_s_timed"] = wall
    if not ok:
        raise RuntimeError("round trip mismatch")
    return out


def run_search(a):
    """Quantise a 4096x4096 tensor of dense N(0, 0.02^2) weights: the exact angular search
    over shells 2..10 for each of its 24-blocks (zero-padded past the last column), then the
    rank of each chosen point (llvq_search)."""
    import numpy as np
    import torch
    import weight_decompression_amd as wd
    from weight_decompression_amd import synth

    lib = wd.load_library()
    rows, cols, M = 4096, 4096, 10
    kb = synth.blocks_per_row(cols)
    W = synth.fidelity_weights(2, 0, rows, cols)
    wpad = np.zeros((rows, kb * 24), dtype=np.float32)
    wpad[:, :cols] = W
    blocks = wpad.reshape(-1, 24)
    n = blocks.shape[0]
    x = torch.from_numpy(blocks).cuda()
    pts = torch.empty((n, 24), dtype=torch.int8, device="cuda:0")
    idx = torch.empty(n, dtype=torch.int64, device="cuda:0")
    err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    args = (ctypes.c_void_p(x.data_ptr()), n, M, wd.SEARCH_ANGULAR, ctypes.c_void_p(pts.data_ptr()),
            ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(err.data_ptr()), sptr)
    sec, wall = time_steps(lambda i: lib.llvq_search(*args), a.steps, a.warmup, stream)
    if int(err.item()) != 0:
        raise RuntimeError("search reported invalid points")
    out = base_line("LLVQ quantisation throughput (exact multi-shell angular search + rank), 1 MI355X",
                    n / sec, "blocks/s", a.steps, a.warmup, sec, "f32",
                    f"llvq_search angular, shells 2..{M}, {rows}x{cols} dense N(0, 0.02^2) weights",
                    {"rows": rows, "cols": cols, "blocks": n, "max_shell": M})
    out["weights_per_s"] = rows * cols / sec
    out["roofline"] = roofline("search", n, sec, n * (96 + 24 + 8),
                               "96 B fp32 block read + 24 B point written + 8 B index written")
    out["wall_s_timed"] = wall
    if not a.no_cpu:
        from oracle import cpu_baseline as cb
        sample = blocks[: a.cpu_blocks].astype(np.float64)
        dt, procs, ref = cb.time_search(sample, M, "angular")
        out["cpu_baseline"] = {"value": len(sample) / dt, "unit": "blocks/s", "cores": procs, "kind": "oracle",
                               "sample": f"the first {len(sample)} blocks of the same tensor: exact class x "
                                         f"codeword search in numpy, {procs} processes, {dt:.2f} s wall"}
        # parity: the GPU's index of each sampled block equals the oracle's, or (a near tie of
        # the fp32 objective) its point scores the same fp64 objective to 1e-6
        gi = idx[: len(sample)].cpu().numpy().astype(np.uint64)
        gp = pts[: len(sample)].cpu().numpy().astype(np.float64)
        same = ties = 0
        for j, (I, v) in enumerate(ref):
            if int(gi[j]) == int(I):
                same += 1
                continue
            vo = np.asarray(v, dtype=np.float64)
            og = float(sample[j] @ gp[j]) / float(np.linalg.norm(gp[j]))
            oo = float(sample[j] @ vo) / float(np.linalg.norm(vo))
            if abs(og - oo) <= 1e-6 * abs(oo):
                ties += 1
        out["parity"] = {"what": f"the first {len(sample)} blocks' indices vs the oracle's exact search",
                         "blocks_checked": len(sample), "equal": same, "near_ties": ties,
                         "pass": same + ties == len(sample)}
    return out


def eff_of(mse, rate):
    """MSE per dimension as effective bits (SQNR / 6.02 dB) and % of the Shannon bound at `rate`."""
    bits = -0.5 * math.log2(mse)
    return {"mse_per_dim": mse, "effective_bits": bits, "rate_bits_per_dim": rate,
            "pct_of_shannon": 100.0 * bits / rate, "shannon_mse": 2.0 ** (-2.0 * rate)}


def run_fidelity(a):
    """Distortion of the quantiser on the memoryless unit Gaussian source: n 24-blocks as a
    [n/128][3072] tensor.  Shape-gain at 2.0 bits/dim (44-bit shape index over shells 2..10 +
    4-bit gain, gain table = chi_24 equal-probability cell means) and Euclidean spherical
    shaping with the same 44-bit shape index (1.83 bits/dim, one scale swept on a subset).
    Reconstruction through llvq_decode to bf16; MSE per dimension against the source."""
    import numpy as np
    import torch
    import weight_decompression_amd as wd
    from weight_decompression_amd import synth

    lib = wd.load_library()
    n = a.fidelity_blocks
    kb = 128
    rows = n // kb
    n = rows * kb
    cols = kb * 24
    x = synth.gaussian_source(6, n)
    W = torch.from_numpy(x.reshape(rows, cols)).cuda()
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def quantize_and_mse(desc, scales, timed):
        packed = torch.empty(wd.packed_bytes(desc), dtype=torch.uint8, device="cuda:0")
        ws = torch.empty(wd.quantize_workspace_bytes(desc), dtype=torch.uint8, device="cuda:0")
        err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        args = (ctypes.byref(desc), ctypes.c_void_p(W.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ctypes.c_void_p(err.data_ptr()),
                sptr)
        if timed:
            sec, _ = time_steps(lambda i: lib.llvq_quantize(*args), a.steps, a.warmup, stream)
        else:
            if lib.llvq_quantize(*args) != 0:
                raise RuntimeError("llvq_quantize failed")
            sec = None
        out = torch.empty((desc.rows, desc.cols), dtype=torch.bfloat16, device="cuda:0")
        if lib.llvq_decode(ctypes.byref(desc), ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                           wd.OUT_BF16, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(err.data_ptr()), sptr) != 0:
            raise RuntimeError("llvq_decode failed")
        torch.cuda.synchronize()
        if int(err.item()) != 0:
            raise RuntimeError("quantiser reported invalid blocks")
        mse = float(((W[: desc.rows].double() - out.double()) ** 2).mean())
        quantize_and_mse.last_packed = packed
        return mse, sec

    # shape-gain, 48 bits per block
    gains = torch.from_numpy(synth.chi_gain_table(16)).cuda()
    dsg = wd.make_desc(wd.MODE_SHAPEGAIN, rows, cols, 10, 44, 4)
    mse_sg, sec = quantize_and_mse(dsg, gains, True)
    packed_sg, gains_sg = quantize_and_mse.last_packed, gains
    # Euclidean, 44 bits per block: the scale that minimises the MSE on a 1/8 subset
    sub = max(1, rows // 8)
    best = None
    for sc in np.arange(0.30, 0.96, 0.05):
        de = wd.make_desc(wd.MODE_EUCLID, sub, cols, 10, 44, 0)
        srow = torch.full((sub,), float(sc), dtype=torch.float16, device="cuda:0")
        m, _ = quantize_and_mse(de, srow, False)
        if best is None or m < best[0]:
            best = (m, float(torch.tensor(float(sc), dtype=torch.float16)))
    de = wd.make_desc(wd.MODE_EUCLID, rows, cols, 10, 44, 0)
    mse_eu, _ = quantize_and_mse(de, torch.full((rows,), best[1], dtype=torch.float16, device="cuda:0"), False)

    # the pages' bit split at 2 bits/dim: a 46- or 47-bit shape (shells 2..11 / 2..12) with a
    # 2- or 1-bit gain, and Euclidean spherical clipping with all 48 bits (shells 2..13)
    split = {}
    for M, sb, gb in ((11, 46, 2), (12, 47, 1)):
        g = torch.from_numpy(synth.chi_gain_table(1 << gb)).cuda()
        m, _ = quantize_and_mse(wd.make_desc(wd.MODE_SHAPEGAIN, rows, cols, M, sb, gb), g, False)
        split[f"shape_gain_{sb}+{gb}"] = dict(max_shell=M, shape_bits=sb, gain_bits=gb, **eff_of(m, 2.0))
        print(f"bench: fidelity shape-gain {sb}+{gb} done", file=sys.stderr, flush=True)
    best13 = None
    for sc in np.arange(0.20, 0.71, 0.025):
        de = wd.make_desc(wd.MODE_EUCLID, sub, cols, 13, 48, 0)
        srow = torch.full((sub,), float(sc), dtype=torch.float16, device="cuda:0")
        m, _ = quantize_and_mse(de, srow, False)
        if best13 is None or m < best13[0]:
            best13 = (m, float(torch.tensor(float(sc), dtype=torch.float16)))
    de = wd.make_desc(wd.MODE_EUCLID, rows, cols, 13, 48, 0)
    m13, _ = quantize_and_mse(de, torch.full((rows,), best13[1], dtype=torch.float16, device="cuda:0"), False)
    split["euclid_48"] = dict(max_shell=13, shape_bits=48, gain_bits=0, scale=best13[1],
                              scale_grid="0.200..0.700 step 0.025 on 1/8 of the blocks", **eff_of(m13, 2.0))

    eff = eff_of

    out = base_line("LLVQ shape-gain distortion on a unit Gaussian source at 2 bits/dim (MSE per dimension), "
                    "1 MI355X", mse_sg, "MSE/dim", a.steps, a.warmup, sec, "f32",
                    f"llvq_quantize + llvq_decode, {n} i.i.d. N(0,1) 24-blocks, shells 2..10",
                    {"blocks": n, "max_shell": 10, "shape_bits": 44, "gain_bits": 4})
    out["higher_is_better"] = False
    out["shape_gain"] = eff(mse_sg, 48 / 24)
    out["euclid"] = dict(eff(mse_eu, 44 / 24), scale=best[1], scale_grid="0.30..0.95 step 0.05 on 1/8 of the blocks")
    out["pages_bit_split"] = split
    out["quantize_blocks_per_s"] = n / sec
    out["roofline"] = roofline("search", n, sec, n * (96 + 24 + 8 + 6),
                               "96 B fp32 block read + 32 B workspace + 6 B packed field per block")
    if not a.no_cpu:
        from oracle import cpu_baseline as cb
        sample = x[: a.cpu_blocks].astype(np.float64)
        dt, procs, ref = cb.time_search(sample, 10, "angular")
        out["cpu_baseline"] = {"value": len(sample) / dt, "unit": "blocks/s", "cores": procs, "kind": "oracle",
                               "sample": f"exact angular search of the first {len(sample)} source blocks in numpy, "
                                         f"{procs} processes, {dt:.2f} s wall (the quantiser's time, not its MSE)"}
        # parity of the shape-gain stream: each sampled block's 44-bit shape index equals the
        # oracle search's (or ties it on the fp64 objective), and its gain index is the table
        # entry nearest to the block's norm (fp64, ties to the lower index)
        raw = packed_sg.cpu().numpy()[: 6 * len(sample)].reshape(-1, 6)
        fv = np.zeros(len(sample), dtype=np.uint64)
        for k in range(6):
            fv |= raw[:, k].astype(np.uint64) << np.uint64(8 * k)
        gtab = gains_sg.cpu().numpy().astype(np.float64)
        from oracle import bijection
        same = ties = gok = 0
        for jb, (I, v) in enumerate(ref):
            gi = int(fv[jb] & np.uint64((1 << 44) - 1))
            gg = int(fv[jb] >> np.uint64(44))
            if gi == int(I):
                same += 1
            else:
                vg = np.asarray(bijection.unrank(gi, 10), dtype=np.float64)
                vo = np.asarray(v, dtype=np.float64)
                og = float(sample[jb] @ vg) / float(np.linalg.norm(vg))
                oo = float(sample[jb] @ vo) / float(np.linalg.norm(vo))
                ties += int(abs(og - oo) <= 1e-6 * abs(oo))
            gok += int(gg == int(np.argmin(np.abs(gtab - np.linalg.norm(sample[jb])))))
        out["parity"] = {"what": f"shape and gain indices of the first {len(sample)} blocks of the shape-gain stream "
                                 f"vs the oracle's exact search and nearest gain",
                         "blocks_checked": len(sample), "shape_equal": same, "near_ties": ties, "gain_equal": gok,
                         "pass": same + ties == len(sample) and gok == len(sample)}
    return out


def run_gptq(a):
    """Spherical GPTQ of a 4096 x 4096 layer: dense N(0, 0.02^2) weights, Hessian of 4096
    correlated activation samples with log-normal channel scales; shells 2..10, 44-bit shape
    + 4-bit gain (gain table 0.02 x the chi_24 cell means).  Reports the relative layer-output
    error tr(dW H dW^T) / tr(W H W^T) of spherical GPTQ, Euclidean-feedback GPTQ and direct
    quantisation (weights decoded through llvq_decode to bf16), and the GPU time."""
    import numpy as np
    import torch
    import weight_decompression_amd as wd
    from weight_decompression_amd import gptq, synth

    lib = wd.load_library()
    N, K, S = 4096, 4096, 4096
    W, X = synth.gptq_layer(34, N, K, S)
    Wt = torch.from_numpy(W).cuda()
    Xt = torch.from_numpy(X).cuda().double()
    H = Xt.T @ Xt / S
    del Xt
    gains = torch.from_numpy((synth.chi_gain_table(16).astype(np.float64) * 0.02).astype(np.float16)).cuda()
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    Wd = Wt.double()
    base = float(((Wd @ H) * Wd).sum())

    def loss(desc, packed):
        out = torch.empty((N, K), dtype=torch.bfloat16, device="cuda:0")
        err = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        if lib.llvq_decode(ctypes.byref(desc), ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(gains.data_ptr()),
                           wd.OUT_BF16, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(err.data_ptr()), sptr) != 0:
            raise RuntimeError("llvq_decode failed")
        D = Wd - out.double()
        return float(((D @ H) * D).sum()) / base

    res = {}
    fields_sph = None
    for variant in ("direct", "euclid", "spherical"):
        desc, packed, fields = gptq.gptq(Wt, H, 10, gains, variant=variant)
        res[variant] = loss(desc, packed)
        if variant == "spherical":
            fields_sph = fields.cpu().numpy().view(np.uint64)
    sec, wall = time_steps(lambda i: (gptq.gptq(Wt, H, 10, gains, variant="spherical"), 0)[1], a.steps, a.warmup,
                           stream)
    kb = synth.blocks_per_row(K)
    out = base_line("LLVQ spherical GPTQ layer-output error (relative, 2 bits/weight), 1 MI355X", res["spherical"],
                    "tr(dW H dW^T)/tr(W H W^T)", a.steps, a.warmup, sec, "f64",
                    f"weight_decompression_amd.gptq (llvq_gptq_factor, then llvq_search + llvq_gptq_column per block column), "
                    f"{N}x{K} N(0, 0.02^2) layer, {S} correlated activation samples",
                    {"rows": N, "cols": K, "samples": S, "max_shell": 10, "shape_bits": 44, "gain_bits": 4})
    out["higher_is_better"] = False
    out["relative_error"] = res
    out["blocks_per_s"] = N * kb / sec
    out["wall_s_timed"] = wall
    if not a.no_cpu:
        import time as _t
        from oracle import gptq as ogptq
        rows = list(range(a.cpu_rows_gptq))
        t0 = _t.perf_counter()
        want_idx, want_g = ogptq.gptq(W, H.cpu().numpy(), 10, gains.cpu().numpy(), variant="spherical", rows=rows)
        dt = _t.perf_counter() - t0
        out["cpu_baseline"] = {"value": len(rows) * kb / dt, "unit": "blocks/s", "cores": 1, "kind": "oracle",
                               "sample": f"oracle spherical GPTQ of rows 0..{len(rows) - 1} of the same layer "
                                         f"(rows do not interact), one process, {dt:.1f} s wall"}
        f = fields_sph.reshape(N, kb)[rows]
        ok = np.logical_and((f & np.uint64((1 << 44) - 1)) == want_idx,
                            (f >> np.uint64(44)).astype(np.int64) == want_g)
        out["parity"] = {"what": f"shape and gain indices of rows 0..{len(rows) - 1} of the spherical GPTQ run vs "
                                 f"the oracle's GPTQ of the same rows", "blocks_checked": int(ok.size),
                         "blocks_differing": int(ok.size - ok.sum()), "pass": bool(ok.all())}
    return out


DEFAULT_WORKLOAD = "gemv_4096x11008"
WORKLOADS = ("gemv_4096x11008", "gemv_11008x4096", "gemv_4096x4096", "gemv_28672x8192", "decode_bf16_7b",
             "roundtrip", "search", "fidelity", "gptq", "gemv_3bit_4096x11008", "decode_3bit_4096x11008")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-rows", type=int, default=4096, help="rows of the tensor the CPU oracle is timed on")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--workload", choices=WORKLOADS, default=DEFAULT_WORKLOAD,
                    help="default: the 4096x11008 batch-1 GEMV (the headline line)")
    ap.add_argument("--batch", type=int, default=1, help="activation rows (GEMV workloads)")
    ap.add_argument("--layers", type=int, default=32, help="layers of the 7B-shaped set (decode_bf16_7b)")
    ap.add_argument("--many", type=int, default=14, metavar="N",
                    help="tensors per llvq_decode_many call (decode_bf16_7b; 0: one llvq_decode per tensor)")
    ap.add_argument("--points", type=int, default=100_000_000, help="indices in the round trip")
    ap.add_argument("--cpu-blocks", type=int, default=2048, help="blocks the CPU oracle search is timed on (search)")
    ap.add_argument("--fidelity-blocks", type=int, default=262144, help="Gaussian source blocks (fidelity)")
    ap.add_argument("--cpu-rows-gptq", type=int, default=8, help="rows the CPU oracle GPTQ is timed on (gptq)")
    ap.add_argument("--parity-rows", type=int, default=256, help="oracle-checked rows (GEMV workloads other than "
                    "the headline, which checks the cpu_baseline rows)")
    ap.add_argument("--parity-points", type=int, default=20000, help="oracle-checked points (roundtrip)")
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
        print("bench.py: this LLVQ library runs on exactly one GPU (no sharding or collectives are "
              "built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import weight_decompression_amd as wd
    from weight_decompression_amd import synth

    C10 = wd.index_count(10)
    w = a.workload
    if w == "gemv_4096x11008":
        t = synth.workload3(C10, 1, load_fidelity(1), batch=a.batch)
        out = run_gemv(a, w, t, f"gemv_4096x11008_b{a.batch}",
                       f"llvq_gemv 2-bit shape-gain 4096x11008 (MLP down-proj), batch {a.batch}")
    elif w == "gemv_11008x4096":
        t = synth.workload3(C10, 0, load_fidelity(0), batch=a.batch)
        out = run_gemv(a, w, t, f"gemv_11008x4096_b{a.batch}",
                       f"llvq_gemv 2-bit shape-gain 11008x4096 (MLP up-proj), batch {a.batch}")
    elif w == "gemv_4096x4096":
        t = synth.workload2(C10, batch=a.batch)
        out = run_gemv(a, w, t, f"gemv_4096x4096_b{a.batch}",
                       f"llvq_gemv 2-bit shape-gain 4096x4096 (q_proj), batch {a.batch}")
    elif w == "gemv_28672x8192":
        t = synth.workload4(C10, a.batch)
        out = run_gemv(a, w, t, f"gemv_28672x8192_b{a.batch}",
                       f"llvq_gemv 2-bit shape-gain 28672x8192, batch {a.batch}")
    elif w == "gemv_3bit_4096x11008":
        # 3 bits per weight: 72-bit fields (68-bit shape index over shells 2..42 + 4-bit gain)
        t = synth.make_wide_tensor("gemv3", 9, 0, 4096, 11008, wd.index_count(42), batch=a.batch)
        out = run_gemv(a, w, t, f"gemv_3bit_b{a.batch}",
                       f"llvq_gemv 3-bit shape-gain 4096x11008 (68+4-bit fields, shells 2..42), batch {a.batch}")
    elif w == "decode_bf16_7b":
        out = run_decode_7b(a)
    elif w == "decode_3bit_4096x11008":
        out = run_decode_3bit(a)
    elif w == "search":
        out = run_search(a)
    elif w == "fidelity":
        out = run_fidelity(a)
    elif w == "gptq":
        out = run_gptq(a)
    else:
        out = run_roundtrip(a)
    print(json.dumps(out), flush=True)
    if "parity" in out and not out["parity"]["pass"]:
        print("bench.py: the timed output does not match the oracle", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
