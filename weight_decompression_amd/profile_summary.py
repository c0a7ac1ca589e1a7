"""Summarise a rocprofv3 run of bench.py into a short markdown report.

Reads the CSV output written by profile_kernels.sh (kernel trace + stats, one PMC pass
of SQ counters, FETCH_SIZE and WRITE_SIZE passes, and the same two passes over a plain
device copy of known size) and prints, for each kernel asked for:

* the kernel's average duration from the kernel-trace statistics;
* SQ_INSTS_VALU x 64 / units = VALU lane-operations per work unit (24-block or point),
  and the VALU utilisation against 256 CUs x 64 lanes x 2.4 GHz;
* FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by the factor that maps the
  counter to the known byte count of the copy kernel, next to the algorithmic bytes;
* when the per-type counter passes (mix_a, mix_b) and an issue-rate table are there: the
  kernel's executed VALU instructions per counter category and its dynamic-mix peak
  (issue_rates.mix_peak), and the utilisation against that peak.

Usage: python -m weight_decompression_amd.profile_summary OUTDIR "BENCH ARGS" KERNEL:UNITS:ALG_BYTES [...]
"""

import csv
import os
import sys
import tempfile
from collections import defaultdict

from . import issue_rates

VALU_PEAK = 256 * 64 * 2.4e9
COPY_BYTES = 256 * 1024 * 1024


def _pmc(path, kernel):
    agg = defaultdict(list)
    meta = {}
    with open(os.path.join(path, "pmc_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"]:
                agg[r["Counter_Name"]].append(float(r["Counter_Value"]))
                meta = {k: r[k] for k in ("Grid_Size", "Workgroup_Size", "VGPR_Count", "Accum_VGPR_Count",
                                          "SGPR_Count", "Scratch_Size")}
    return {k: sum(v) / len(v) for k, v in agg.items()}, meta


def _copy_kib(path, counter):
    vals = []
    with open(os.path.join(path, "pmc_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    return sum(vals) / len(vals) if vals else None


def _mix_section(outdir, kernel, symbol, avg_ns, units, rates_md, asm):
    a, _ = _pmc(os.path.join(outdir, "mix_a"), kernel)
    b, _ = _pmc(os.path.join(outdir, "mix_b"), kernel)
    dyn = dict(a)
    dyn.update(b)
    dyn["SQ_INSTS_VALU"] = a["SQ_INSTS_VALU"]
    rates, cats = issue_rates.read_rates_md(rates_md)
    static = issue_rates.kernel_mix(asm, symbol)
    rate, table, unplaced = issue_rates.mix_peak(dyn, static, rates, cats)
    peak = rate * issue_rates.NCU * 64 * issue_rates.CLOCK_HZ
    util = dyn["SQ_INSTS_VALU"] * 64 / (avg_ns * 1e-9) / peak
    lines = [f"Dynamic VALU mix (per dispatch; static split inside a category from `{symbol}`):", "",
             "| category | instructions | share | static-split rate | most frequent in the assembly |",
             "|---|---|---|---|---|"]
    tot = sum(n for _, n, _, _ in table)
    for c, n, r, used in table:
        lines.append(f"| {c} | {n:.0f} | {n / tot:.3f} | {r:.3f} | {used} |")
    lines.append("")
    if dyn.get("SQ_INSTS_MFMA"):
        lines.append(f"MFMA instructions (matrix pipe, left out of the VALU mix): {dyn['SQ_INSTS_MFMA']:.0f}")
    if dyn.get("SQ_ACTIVE_INST_VALU2") is not None:
        lines.append(f"SQ_ACTIVE_INST_VALU2 (quad-cycles with two VALU issues): {dyn['SQ_ACTIVE_INST_VALU2']:.0f}")
    if unplaced:
        lines.append("Static instructions without a measured rate or category (left out of the split): " +
                     ", ".join(f"{i} {k}" for i, k in unplaced.most_common(8)))
    lines.append("")
    lines.append(f"* dynamic-mix VALU peak = **{rate:.3f}** wave-instructions per CU per clock = "
                 f"**{peak / 1e12:.2f} T lane-ops/s**")
    lines.append(f"* VALU utilisation against it at the traced average duration = **{util:.3f}**")
    lines.append("")
    return lines, peak


def summarise(outdir, bench_args, specs):
    lines = ["# rocprofv3 summary: bench.py " + bench_args, ""]
    lines.append("Command (from the repository root):")
    lines.append("")
    lines.append(f"    bash weight_decompression_amd/profile_kernels.sh OUTDIR \"{bench_args}\" " +
                 " ".join(f"'{s}'" for s in specs))
    lines.append("")
    with open(os.path.join(outdir, "trace", "run_kernel_stats.csv")) as f:
        stats = list(csv.DictReader(f))
    cf = _copy_kib(os.path.join(outdir, "copy_fetch"), "FETCH_SIZE")
    cw = _copy_kib(os.path.join(outdir, "copy_write"), "WRITE_SIZE")
    ff = COPY_BYTES / 1024 / cf
    fw = COPY_BYTES / 1024 / cw
    lines.append(f"HBM counter calibration: a device copy of {COPY_BYTES} B reads FETCH_SIZE = {cf:.2f} KiB "
                 f"(factor {ff:.4f}) and WRITE_SIZE = {cw:.2f} KiB (factor {fw:.4f}).")
    lines.append("")
    rates_md = os.environ.get("RATES_MD") or os.path.join(issue_rates.PKG_DIR, "..", "profiles",
                                                          "valu_issue_rates_gfx950.md")
    do_mix = os.path.isdir(os.path.join(outdir, "mix_a")) and os.path.isdir(os.path.join(outdir, "mix_b")) \
        and os.path.exists(rates_md)
    asm = None
    tmp = None
    if do_mix:
        # the library's device assembly (tens of MB) goes to a temporary folder, not the output
        asm = os.environ.get("LLVQ_ASM")
        if not asm:
            tmp = tempfile.TemporaryDirectory()
            asm = issue_rates.device_asm(tmp.name)
        lines.append(f"Issue rates and counter categories: `{os.path.relpath(rates_md, issue_rates.PKG_DIR + '/..')}`.")
        lines.append("")
    for spec in specs:
        f = spec.split(":")
        kernel, units, alg = f[:3]
        symbol = f[3] if len(f) > 3 else kernel
        units = int(units)
        alg = float(alg)
        st = [r for r in stats if kernel in r["Name"]]
        if not st:
            raise SystemExit(f"kernel {kernel!r} not in the trace statistics")
        st = st[0]
        avg_ns = float(st["AverageNs"])
        lines.append(f"## {kernel}")
        lines.append("")
        lines.append("| kernel | calls | average ns | min ns | max ns |")
        lines.append("|---|---|---|---|---|")
        lines.append(f"| {st['Name'][:100]} | {st['Calls']} | {avg_ns:.0f} | {st['MinNs']} | {st['MaxNs']} |")
        lines.append("")
        sq, meta = _pmc(os.path.join(outdir, "pmc_valu"), kernel)
        lines.append("| counter (mean per dispatch) | value |")
        lines.append("|---|---|")
        for k in sorted(sq):
            lines.append(f"| {k} | {sq[k]:.0f} |")
        lines.append("")
        lines.append("Dispatch: " + ", ".join(f"{k}={v}" for k, v in meta.items()))
        lines.append("")
        valu = sq.get("SQ_INSTS_VALU", 0.0)
        per_unit = valu * 64 / units
        util = valu * 64 / (avg_ns * 1e-9) / VALU_PEAK
        lines.append(f"* work units per launch: {units}")
        lines.append(f"* VALU lane-ops per unit = SQ_INSTS_VALU x 64 / units = **{per_unit:.1f}**")
        lines.append(f"* VALU utilisation at the traced average duration = **{util:.3f}**")
        fetch, _ = _pmc(os.path.join(outdir, "pmc_fetch"), kernel)
        write, _ = _pmc(os.path.join(outdir, "pmc_write"), kernel)
        fb = fetch["FETCH_SIZE"] * 1024 * ff
        wb = write["WRITE_SIZE"] * 1024 * fw
        lines.append(f"* FETCH_SIZE {fetch['FETCH_SIZE']:.2f} KiB -> {fb:.0f} B; WRITE_SIZE {write['WRITE_SIZE']:.2f} KiB "
                     f"-> {wb:.0f} B; total **{fb + wb:.0f} B** per launch")
        lines.append(f"* algorithmic bytes per launch {alg:.0f}; measured / algorithmic = {(fb + wb) / alg:.3f}")
        lines.append("")
        mix_peak = None
        if do_mix:
            ml, mix_peak = _mix_section(outdir, kernel, symbol, avg_ns, units, rates_md, asm)
            lines += ml
        mp = "" if mix_peak is None else f" valu_mix_peak_tops={mix_peak / 1e12:.2f}"
        lines.append(f"<!-- profile {kernel} valu_lane_ops_per_unit={per_unit:.1f} fetch={fb:.0f} write={wb:.0f} "
                     f"avg_ns={avg_ns:.0f}{mp} -->")
        lines.append("")
    if tmp is not None:
        tmp.cleanup()
    return "\n".join(lines) + "\n"


def main(argv):
    if len(argv) < 4:
        raise SystemExit(__doc__)
    sys.stdout.write(summarise(argv[1], argv[2], argv[3:]))


if __name__ == "__main__":
    main(sys.argv)
