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

  3. maps each measured instruction to the SQ counter category that counts it (run under
     rocprofv3 with the two passes of MIX_PASSES; `--categories A B` reads those runs);
  4. gives a kernel's **dynamic-mix peak**: the per-category SQ counters of a profiled
     kernel say how many instructions of each category it executed; inside a category (and
     for the instructions no category counts, `other` = SQ_INSTS_VALU minus the categories
     and MFMA) the split between instructions is taken from the kernel's static device
     assembly.  The peak is N / sum_c(N_c / r_c), r_c the static-split harmonic rate of
     category c (`mix_peak`).

Usage (from the repository root, on a machine with the GPU):
    python -m weight_decompression_amd.issue_rates [--kernel k_gemv_b1ILb0] [--json rates.json]
    rocprofv3 --pmc <MIX_PASSES[i]> ... -- python3 -m weight_decompression_amd.issue_rates --reps 1
"""

import argparse
import collections
import csv
import ctypes
import json
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
         "v_cmp_ne_u32", "v_mad_u64_u32", "v_lshl_add_u64", "v_mov_b64", "v_lshrrev_b64", "v_add_co_u32",
         "v_cvt_pk_bf16_f32", "v_fmac_f64", "v_cmp_ge_f64", "v_div_scale_f64", "v_div_fmas_f64", "v_div_fixup_f64",
         "v_rcp_f64", "v_ldexp_f64", "v_readlane_b32", "v_readfirstlane_b32", "v_writelane_b32", "v_rndne_f64",
         "v_rcp_f32", "v_div_scale_f32"]


# The per-type VALU counters of gfx950, in two rocprofv3 passes (at most 8 SQ counters each).
MIX_PASSES = [
    ["SQ_INSTS_VALU", "SQ_INSTS_VALU_INT32", "SQ_INSTS_VALU_INT64", "SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU_FMA_F64",
     "SQ_INSTS_VALU_MUL_F64", "SQ_INSTS_VALU_ADD_F64", "SQ_INSTS_VALU_TRANS_F64"],
    ["SQ_INSTS_VALU", "SQ_INSTS_VALU_FMA_F32", "SQ_INSTS_VALU_ADD_F32", "SQ_INSTS_VALU_MUL_F32",
     "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_BF16"],
]
CATEGORIES = ["SQ_INSTS_VALU_INT32", "SQ_INSTS_VALU_INT64", "SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU_FMA_F64",
              "SQ_INSTS_VALU_MUL_F64", "SQ_INSTS_VALU_ADD_F64", "SQ_INSTS_VALU_TRANS_F64", "SQ_INSTS_VALU_FMA_F32",
              "SQ_INSTS_VALU_ADD_F32", "SQ_INSTS_VALU_MUL_F32", "SQ_INSTS_VALU_TRANS_F32"]
OTHER = "other"

# Instructions of the kernels without a kernel of their own here, timed as the named one
# (same encoding family and functional unit: compares, min/max and shifts of other types,
# the upper-half lane count, the other byte selects of the ubyte conversion, carry forms,
# literal-operand FMAs).
ALIASES = {
    "v_cmp_gt_i32": "v_cmp_ne_u32", "v_cmp_eq_u32": "v_cmp_ne_u32", "v_cmp_lt_i32": "v_cmp_ne_u32",
    "v_cmp_le_i32": "v_cmp_ne_u32", "v_cmp_gt_u32": "v_cmp_ne_u32", "v_cmp_lt_u32": "v_cmp_ne_u32",
    "v_cmp_ge_u32": "v_cmp_ne_u32", "v_cmp_le_u32": "v_cmp_ne_u32", "v_cmp_ge_i32": "v_cmp_ne_u32",
    "v_cmp_ne_i32": "v_cmp_ne_u32", "v_cmp_eq_i32": "v_cmp_ne_u32", "v_cmp_eq_u16": "v_cmp_ne_u32",
    "v_cmp_gt_f32": "v_cmp_ne_u32", "v_cmp_lt_f32": "v_cmp_ne_u32", "v_cmp_eq_f32": "v_cmp_ne_u32",
    "v_cmp_ge_f32": "v_cmp_ne_u32", "v_cmp_le_f32": "v_cmp_ne_u32", "v_cmp_neq_f32": "v_cmp_ne_u32",
    "v_cmp_nlt_f32": "v_cmp_ne_u32", "v_cmp_ngt_f32": "v_cmp_ne_u32", "v_cmp_u_f32": "v_cmp_ne_u32",
    "v_cmp_o_f32": "v_cmp_ne_u32", "v_cmp_class_f32": "v_cmp_ne_u32",
    "v_cmp_ne_u64": "v_cmp_ge_f64", "v_cmp_eq_u64": "v_cmp_ge_f64", "v_cmp_gt_u64": "v_cmp_ge_f64",
    "v_cmp_lt_u64": "v_cmp_ge_f64", "v_cmp_ge_u64": "v_cmp_ge_f64", "v_cmp_le_u64": "v_cmp_ge_f64",
    "v_cmp_gt_f64": "v_cmp_ge_f64", "v_cmp_lt_f64": "v_cmp_ge_f64", "v_cmp_le_f64": "v_cmp_ge_f64",
    "v_cmp_eq_f64": "v_cmp_ge_f64", "v_cmp_neq_f64": "v_cmp_ge_f64", "v_cmp_nlt_f64": "v_cmp_ge_f64",
    "v_cmp_ngt_f64": "v_cmp_ge_f64", "v_cmp_nge_f64": "v_cmp_ge_f64", "v_cmp_class_f64": "v_cmp_ge_f64",
    "v_cmp_u_f64": "v_cmp_ge_f64", "v_cmp_lg_f64": "v_cmp_ge_f64",
    "v_cmpx_ne_u32": "v_cmp_ne_u32", "v_cmpx_eq_u32": "v_cmp_ne_u32", "v_cmpx_gt_u32": "v_cmp_ne_u32",
    "v_cmpx_lt_u32": "v_cmp_ne_u32", "v_cmpx_gt_i32": "v_cmp_ne_u32", "v_cmpx_lt_i32": "v_cmp_ne_u32",
    "v_min_i32": "v_min_u32", "v_max_i32": "v_max_u32", "v_med3_i32": "v_med3_u32", "v_min3_u32": "v_med3_u32",
    "v_max3_u32": "v_med3_u32", "v_min3_i32": "v_med3_u32", "v_max3_i32": "v_med3_u32",
    "v_bfe_i32": "v_bfe_u32", "v_ashrrev_i32": "v_lshrrev_b32", "v_lshlrev_b64": "v_lshrrev_b64",
    "v_ashrrev_i64": "v_lshrrev_b64", "v_mbcnt_hi_u32_b32": "v_mbcnt_lo_u32_b32",
    "v_cvt_f32_ubyte1": "v_cvt_f32_ubyte0", "v_cvt_f32_ubyte2": "v_cvt_f32_ubyte0",
    "v_cvt_f32_ubyte3": "v_cvt_f32_ubyte0", "v_cvt_u32_f32": "v_cvt_f32_u32", "v_cvt_i32_f32": "v_cvt_f32_u32",
    "v_cvt_f32_i32": "v_cvt_f32_u32", "v_cvt_f32_f64": "v_cvt_u32_f64", "v_cvt_i32_f64": "v_cvt_u32_f64",
    "v_cvt_f64_f32": "v_cvt_f64_u32", "v_cvt_f64_i32": "v_cvt_f64_u32",
    "v_sub_co_u32": "v_add_co_u32", "v_subb_co_u32": "v_add_co_u32", "v_addc_co_u32": "v_add_co_u32",
    "v_subrev_co_u32": "v_add_co_u32", "v_subbrev_co_u32": "v_add_co_u32",
    "v_fmamk_f32": "v_fmac_f32", "v_fmaak_f32": "v_fmac_f32", "v_mul_hi_u32": "v_mul_lo_u32",
    "v_mad_i64_i32": "v_mad_u64_u32", "v_subrev_u32": "v_sub_u32", "v_sub_f32": "v_add_f32",
    "v_subrev_f32": "v_add_f32", "v_mul_u32_u24": "v_mad_u32_u24", "v_mul_hi_u32_u24": "v_mad_u32_u24",
    "v_add_lshl_u32": "v_lshl_add_u32", "v_fract_f64": "v_rcp_f64",
    "v_trig_preop_f64": "v_rcp_f64", "v_rsq_f64": "v_rcp_f64", "v_sqrt_f64": "v_rcp_f64",
    "v_floor_f64": "v_rndne_f64", "v_trunc_f64": "v_rndne_f64", "v_ceil_f64": "v_rndne_f64",
    "v_rsq_f32": "v_rcp_f32", "v_sqrt_f32": "v_rcp_f32", "v_exp_f32": "v_rcp_f32", "v_log_f32": "v_rcp_f32",
    "v_div_fmas_f32": "v_fma_f32", "v_div_fixup_f32": "v_fma_f32", "v_ldexp_f32": "v_mul_f32",
    "v_rndne_f32": "v_cvt_f32_u32", "v_floor_f32": "v_cvt_f32_u32", "v_trunc_f32": "v_cvt_f32_u32",
}


def rate_of(name, rates):
    """Measured rate of an instruction (directly or through ALIASES), or None."""
    if name in rates:
        return rates[name]
    a = ALIASES.get(name)
    return rates.get(a) if a else None


def _pmc_means(path):
    """{kernel base name: {counter: mean per dispatch}} of a rocprofv3 CSV run."""
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    grid = {}
    with open(os.path.join(path, "pmc_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            k = r["Kernel_Name"].split("(")[0].split()[-1]
            agg[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            grid[k] = int(r["Grid_Size"])
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in agg.items()}, grid


def categories(pass_dirs, iters):
    """{instruction: (category, share)} from rocprofv3 runs of this module under MIX_PASSES:
    the category whose counter holds at least half of the kernel's timed instructions
    (grid / 64 x iters), else `other`."""
    counts, grid = {}, {}
    for d in pass_dirs:
        c, g = _pmc_means(d)
        for k, v in c.items():
            counts.setdefault(k, {}).update(v)
        grid.update(g)
    out = {}
    for name in NAMES:
        k = "k_" + name[2:]
        if k not in counts:
            continue
        timed = grid[k] / 64 * iters
        best = max(CATEGORIES, key=lambda c: counts[k].get(c, 0.0))
        share = counts[k].get(best, 0.0) / timed
        out[name] = (best, share) if share >= 0.5 else (OTHER, share)
    return out


def category_of(name, cats):
    if name in cats:
        return cats[name][0]
    a = ALIASES.get(name)
    if a and a in cats:
        return cats[a][0]
    return None


def mix_peak(dyn, static_mix, rates, cats):
    """Dynamic-mix VALU peak of a kernel in wave-instructions per CU per clock.

    dyn: the kernel's mean counters per dispatch (SQ_INSTS_VALU, the CATEGORIES, SQ_INSTS_MFMA);
    static_mix: Counter of the VALU instructions in its device assembly.  Returns
    (rate, table) with table rows (category, dynamic count, static-split rate, instructions
    used for the split)."""
    total = dyn["SQ_INSTS_VALU"] - dyn.get("SQ_INSTS_MFMA", 0.0)
    n = {c: dyn.get(c, 0.0) for c in CATEGORIES}
    n[OTHER] = max(0.0, total - sum(n.values()))
    groups = collections.defaultdict(collections.Counter)
    unplaced = collections.Counter()
    for ins, cnt in static_mix.items():
        if ins.startswith("v_mfma") or ins.startswith("v_accvgpr"):
            continue
        r = rate_of(ins, rates)
        c = category_of(ins, cats)
        if r is None or c is None:
            unplaced[ins] += cnt
            continue
        groups[c][ins] += cnt
    slow = min(rates.values())
    table, t = [], 0.0
    for c, nc in n.items():
        if nc <= 0:
            continue
        g = groups.get(c)
        if g:
            rc = sum(g.values()) / sum(k / rate_of(i, rates) for i, k in g.items())
            used = ", ".join(f"{i} {k}" for i, k in g.most_common(4))
        else:
            rc, used = slow, "(none in the assembly: slowest measured rate)"
        t += nc / rc
        table.append((c, nc, rc, used))
    return total / t, table, unplaced


def read_rates_md(path):
    """{instruction: rate}, {instruction: (category, share)} from the issue-rate summary table."""
    rates, cats = {}, {}
    with open(path) as f:
        for line in f:
            p = [x.strip() for x in line.split("|")]
            if len(p) > 3 and p[1].startswith("v_"):
                rates[p[1]] = float(p[2])
                if len(p) > 5 and p[3]:
                    cats[p[1]] = (p[3], float(p[4]))
    return rates, cats


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
    mix = {m: c for m, c in mix.items() if not (m.startswith("v_mfma") or m.startswith("v_accvgpr"))}
    t = sum(c / (rate_of(m, rates) or slowest) for m, c in mix.items())
    unmeasured = {m: c for m, c in mix.items() if rate_of(m, rates) is None}
    return sum(mix.values()) / t, unmeasured


def rates_table(rates, cats=None):
    lines = ["| instruction | wave-instr / CU / clock (2.4 GHz) | counter category | share |", "|---|---|---|---|"]
    for name in NAMES:
        c, sh = (cats or {}).get(name, ("", None))
        lines.append(f"| {name} | {rates[name]:.3f} | {c} | {'' if sh is None else f'{sh:.3f}'} |")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--kernel", action="append", default=[],
                    help="substring of a kernel symbol whose static VALU mix is weighted (repeatable)")
    ap.add_argument("--blocks", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--categories", nargs=2, metavar=("PASS_A", "PASS_B"),
                    help="rocprofv3 output folders of this module run under the two MIX_PASSES")
    ap.add_argument("--json", help="also write the rates (and categories) to this file")
    a = ap.parse_args(argv)
    if not os.path.exists(LIB_PATH):
        build()
    rates = measure(a.blocks, a.reps)
    cats = categories(a.categories, ctypes.CDLL(LIB_PATH).ir_iters()) if a.categories else None
    print(rates_table(rates, cats))
    print()
    if a.json:
        with open(a.json, "w") as f:
            json.dump({"rates": rates, "categories": cats}, f, indent=1)
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
