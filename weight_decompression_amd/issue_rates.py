"""VALU issue rates on gfx950 and the instruction-mix-weighted VALU peak of a kernel.

The VALU roofline of the decode kernels counts lane-operations (SQ_INSTS_VALU x 64) against
256 CUs x 64 lanes x 2.4 GHz = 39.32 T lane-ops/s, i.e. one wave-instruction per CU per clock.
CDNA4 issues some simple instructions faster than that and others slower, so the peak that
fits a kernel depends on its instruction mix.  This module

  1. measures the issue rate of each instruction in `issue_rates.hip` (libissuerates.so):
     wave-instructions per CU per 2.4 GHz clock, 16 waves per CU as in the decode kernels;
  2. optionally counts the VALU instructions of one kernel in the device assembly of the LLVQ
     library (built here with hipcc, device code only) and reports the mix-weighted rate
     N / sum_i(n_i / r_i), instructions without a measured rate taken at the slowest rate.

Usage (from the repository root, on a machine with the GPU):
    python -m weight_decompression_amd.issue_rates [--kernel k_gemv_b1ILb0]
"""

import argparse
import collections
import ctypes
import os
import re
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libissuerates.so")
CLOCK_HZ = 2.4e9
NCU = 256

# same order as kKernels in issue_rates.hip
NAMES = ["v_add_u32", "v_sub_u32", "v_and_b32", "v_or_b32", "v_xor_b32", "v_not_b32", "v_mov_b32",
         "v_lshrrev_b32", "v_lshlrev_b32", "v_cndmask_b32", "v_mul_f32", "v_add_f32", "v_fmac_f32", "v_fma_f32",
         "v_cvt_f32_u32", "v_cvt_f32_ubyte0", "v_xad_u32", "v_ffbl_b32", "v_bfi_b32", "v_bfe_u32", "v_alignbit_b32",
         "v_lshl_or_b32", "v_lshl_add_u32", "v_add3_u32", "v_and_or_b32", "v_or3_b32", "v_mad_u32_u24",
         "v_mul_lo_u32", "v_perm_b32", "v_dot4_u32_u8", "v_bcnt_u32_b32", "v_med3_u32", "v_min_f32", "v_max_f32",
         "v_min_u32", "v_max_u32", "v_max3_f32", "v_fma_f64", "v_mul_f64", "v_add_f64", "v_cvt_u32_f64",
         "v_cvt_f64_u32", "v_dot2c_f32_bf16", "v_cvt_scalef32_pk_bf16_fp8", "v_bitop3_b32", "v_mbcnt_lo_u32_b32",
         "v_cmp_ne_u32"]


def build(verbose=True):
    """Compile issue_rates.hip into libissuerates.so (gfx950)."""
    from . import build_lib
    tmp = LIB_PATH + ".tmp"
    cmd = [build_lib.hipcc_path(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", tmp,
           os.path.join(PKG_DIR, "issue_rates.hip")]
    if verbose:
        print("+ " + " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def measure(blocks=1024, reps=5):
    """{instruction: wave-instructions per CU per clock} at `blocks` x 256 lanes."""
    import torch
    lib = ctypes.CDLL(LIB_PATH)
    lib.ir_run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int]
    n = lib.ir_count()
    if n != len(NAMES):
        raise RuntimeError(f"libissuerates.so has {n} kernels, expected {len(NAMES)}")
    steps = lib.ir_iters()
    out = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")
    rates = {}
    for w, name in enumerate(NAMES):
        if lib.ir_run(w, ctypes.c_void_p(out.data_ptr()), 7, blocks) != 0:
            raise RuntimeError(f"launch of the {name} kernel failed")
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            lib.ir_run(w, ctypes.c_void_p(out.data_ptr()), 7, blocks)
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / reps
        rates[name] = blocks * 256 * steps / 64 / sec / NCU / CLOCK_HZ
    return rates


def device_asm(outdir):
    """Device assembly of the LLVQ library (the in-tree sources), compiled like the library."""
    from . import build_lib
    path = os.path.join(outdir, "llvq_gfx950.s")
    cmd = [build_lib.hipcc_path(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", build_lib.INCLUDE, "-I", build_lib.CSRC, "-I", build_lib.BUILD_DIR,
           "--offload-device-only", "-S", "-o", path, os.path.join(build_lib.CSRC, "llvq.hip")]
    subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL)
    return path


def kernel_mix(asm_path, kernel):
    """Counter of the VALU instructions (suffixes _e32/_e64/_sdwa/_dpp dropped) in the body
    of the first function whose symbol contains `kernel`."""
    mix = collections.Counter()
    inside = False
    with open(asm_path) as f:
        for line in f:
            if not inside:
                label = line.split(";")[0].strip()
                if label.startswith("_Z") and label.endswith(":") and kernel in label:
                    inside = True
                continue
            tok = line.split()
            if not tok:
                continue
            if tok[0] == "s_endpgm":
                break
            if tok[0].startswith("v_"):
                mix[re.sub(r"_(e32|e64|sdwa|dpp)$", "", tok[0])] += 1
    if not mix:
        raise SystemExit(f"kernel {kernel!r} not found in {asm_path}")
    return mix


def weighted_rate(mix, rates):
    slowest = min(rates.values())
    t = sum(c / rates.get(m, slowest) for m, c in mix.items())
    unmeasured = {m: c for m, c in mix.items() if m not in rates}
    return sum(mix.values()) / t, unmeasured


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--kernel", action="append", default=[],
                    help="substring of a kernel symbol whose static VALU mix is weighted (repeatable)")
    ap.add_argument("--blocks", type=int, default=1024)
    a = ap.parse_args(argv)
    if not os.path.exists(LIB_PATH):
        build()
    rates = measure(a.blocks)
    print("| instruction | wave-instr / CU / clock (2.4 GHz) |")
    print("|---|---|")
    for name in NAMES:
        print(f"| {name} | {rates[name]:.3f} |")
    print()
    if a.kernel:
        with tempfile.TemporaryDirectory() as d:
            asm = device_asm(d)
            for k in a.kernel:
                mix = kernel_mix(asm, k)
                r, unm = weighted_rate(mix, rates)
                n = sum(mix.values())
                print(f"{k}: {n} VALU instructions (static), mix-weighted rate {r:.3f} wave-instr/CU/clock = "
                      f"{r * 64 * NCU * CLOCK_HZ / 1e12:.1f} T lane-ops/s; without a measured rate "
                      f"(taken at the slowest): {sum(unm.values())} {dict(unm)}")
                top = ", ".join(f"{m} {c}" for m, c in mix.most_common(12))
                print(f"  most frequent: {top}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
