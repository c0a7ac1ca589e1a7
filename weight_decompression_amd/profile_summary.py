"""Summarise a rocprofv3 run of one LLVQ kernel into a short markdown report.

Reads the CSV output written by profile_gemv.sh (kernel trace + stats, one PMC pass of
SQ counters, FETCH_SIZE and WRITE_SIZE passes, and the same two passes over a plain
device copy of known size) and prints:

* the kernel's average duration from the kernel-trace statistics;
* SQ_INSTS_VALU x 64 / blocks = VALU lane-operations per 24-block, and the VALU
  utilisation against 256 CUs x 64 lanes x 2.4 GHz;
* FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by the factor that maps the
  counter to the known byte count of the copy kernel.

Usage: python -m weight_decompression_amd.profile_summary OUTDIR KERNEL_SUBSTRING BLOCKS
           ALG_BYTES COPY_BYTES "COMMAND"
"""

import csv
import os
import sys
from collections import defaultdict

VALU_PEAK = 256 * 64 * 2.4e9


def _pmc(path, kernel):
    agg = defaultdict(list)
    meta = {}
    with open(os.path.join(path, "pmc_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"]:
                agg[r["Counter_Name"]].append(float(r["Counter_Value"]))
                meta = {k: r[k] for k in ("Grid_Size", "Workgroup_Size", "LDS_Block_Size", "VGPR_Count",
                                          "Accum_VGPR_Count", "SGPR_Count", "Scratch_Size")}
    return {k: sum(v) / len(v) for k, v in agg.items()}, {k: len(v) for k, v in agg.items()}, meta


def _copy_kib(path, counter):
    vals = []
    with open(os.path.join(path, "pmc_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        return None
    return sum(vals) / len(vals)


def summarise(outdir, kernel, blocks, alg_bytes, copy_bytes, command):
    lines = []
    with open(os.path.join(outdir, "trace", "run_kernel_stats.csv")) as f:
        stats = [r for r in csv.DictReader(f) if kernel in r["Name"]]
    if not stats:
        raise SystemExit(f"kernel {kernel!r} not in the trace statistics")
    st = stats[0]
    avg_ns = float(st["AverageNs"])
    lines.append(f"# {kernel}: rocprofv3 summary\n")
    lines.append("Command (from the repository root):\n")
    lines.append(f"    {command}\n")
    lines.append("## Kernel trace (--kernel-trace --stats)\n")
    lines.append("| kernel | calls | average ns | min ns | max ns |")
    lines.append("|---|---|---|---|---|")
    lines.append(f"| {st['Name'][:90]} | {st['Calls']} | {avg_ns:.0f} | {st['MinNs']} | {st['MaxNs']} |\n")

    sq, n, meta = _pmc(os.path.join(outdir, "pmc_valu"), kernel)
    lines.append("## SQ counters (mean per dispatch)\n")
    lines.append("| counter | value |")
    lines.append("|---|---|")
    for k in sorted(sq):
        lines.append(f"| {k} | {sq[k]:.0f} |")
    lines.append("")
    lines.append("Dispatch: " + ", ".join(f"{k}={v}" for k, v in meta.items()) + "\n")
    valu = sq.get("SQ_INSTS_VALU", 0.0)
    per_block = valu * 64 / blocks
    util = valu * 64 / (avg_ns * 1e-9) / VALU_PEAK
    lines.append(f"* VALU lane-ops per 24-block = SQ_INSTS_VALU x 64 / {blocks} = **{per_block:.1f}**")
    lines.append(f"* VALU utilisation at the traced average duration = {valu * 64:.4g} / {avg_ns * 1e-9:.4g} s "
                 f"/ 39.32e12 = **{util:.3f}**\n")

    fetch, _, _ = _pmc(os.path.join(outdir, "pmc_fetch"), kernel)
    write, _, _ = _pmc(os.path.join(outdir, "pmc_write"), kernel)
    cf = _copy_kib(os.path.join(outdir, "copy_fetch"), "FETCH_SIZE")
    cw = _copy_kib(os.path.join(outdir, "copy_write"), "WRITE_SIZE")
    lines.append("## HBM traffic (FETCH_SIZE and WRITE_SIZE passes, KiB per dispatch)\n")
    lines.append(f"Copy calibration: a device copy of {copy_bytes} B reads FETCH_SIZE = {cf:.2f} KiB and "
                 f"writes WRITE_SIZE = {cw:.2f} KiB.")
    ff = copy_bytes / 1024 / cf
    fw = copy_bytes / 1024 / cw
    fb = fetch["FETCH_SIZE"] * 1024 * ff
    wb = write["WRITE_SIZE"] * 1024 * fw
    lines.append(f"Scale factors: fetch {ff:.4f}, write {fw:.4f}.\n")
    lines.append("| | counter KiB | scaled bytes |")
    lines.append("|---|---|---|")
    lines.append(f"| FETCH_SIZE | {fetch['FETCH_SIZE']:.2f} | {fb:.0f} |")
    lines.append(f"| WRITE_SIZE | {write['WRITE_SIZE']:.2f} | {wb:.0f} |")
    lines.append(f"| total | | **{fb + wb:.0f}** |\n")
    lines.append(f"Algorithmic bytes per launch: {alg_bytes}; measured / algorithmic = {(fb + wb) / alg_bytes:.3f}.")
    return "\n".join(lines) + "\n"


def main(argv):
    if len(argv) != 7:
        raise SystemExit(__doc__)
    outdir, kernel, blocks, alg_bytes, copy_bytes, command = argv[1:]
    sys.stdout.write(summarise(outdir, kernel, int(blocks), float(alg_bytes), int(copy_bytes), command))


if __name__ == "__main__":
    main(sys.argv)
