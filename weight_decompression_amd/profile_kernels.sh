#!/bin/bash
# rocprofv3 profile of one bench.py workload on one GPU.
# Usage (from the repository root, on a machine with the GPU):
#   bash weight_decompression_amd/profile_kernels.sh OUTDIR "BENCH ARGS" KERNEL:UNITS:ALG_BYTES [...]
# Runs, each in its own rocprofv3 process:
#   trace          kernel trace + stats of `bench.py BENCH ARGS`
#   pmc_valu       SQ counters (VALU / LDS / SALU instructions, wave cycles)
#   pmc_fetch      FETCH_SIZE;  pmc_write  WRITE_SIZE
#   copy_fetch, copy_write   the same two counters over a plain 256 MiB device copy
#   mix_a, mix_b   the per-type VALU counters (issue_rates.MIX_PASSES)
# then writes OUTDIR/summary.md with one section per KERNEL (a substring of the kernel
# name), UNITS its work units per launch (24-blocks or points) and ALG_BYTES its
# algorithmic HBM bytes per launch; KERNEL may carry a fourth field, the substring of the
# mangled symbol whose device assembly gives the static split inside each counter category.
# With RATES_MD (default profiles/valu_issue_rates_gfx950.md, written by profile_rates.sh)
# the summary also gives each kernel's dynamic-mix VALU peak (issue_rates.mix_peak).
set -o pipefail
OUT="$(cd "$(dirname "$1")" && pwd)/$(basename "$1")"
ARGS="$2"
shift 2
REPO="$(cd "$(dirname "$0")/.." && pwd)"
mkdir -p "$OUT"
cd /tmp && export TMPDIR=/tmp
run() { echo "== $1 $(date +%T)"; shift; "$@" || exit $?; }
run trace timeout -k 10 600 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/trace" -o run -- \
  python3 "$REPO/bench.py" --no-cpu $ARGS
run valu timeout -s KILL 300 rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_WAVES SQ_ACTIVE_INST_VALU \
  SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_INSTS_MFMA --output-format csv -d "$OUT/pmc_valu" -o pmc -- \
  python3 "$REPO/bench.py" --no-cpu $ARGS
run fetch timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE --output-format csv -d "$OUT/pmc_fetch" -o pmc -- \
  python3 "$REPO/bench.py" --no-cpu $ARGS
run write timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE --output-format csv -d "$OUT/pmc_write" -o pmc -- \
  python3 "$REPO/bench.py" --no-cpu $ARGS
PASS_A="SQ_INSTS_VALU SQ_INSTS_VALU_INT32 SQ_INSTS_VALU_INT64 SQ_INSTS_VALU_CVT SQ_INSTS_VALU_FMA_F64 SQ_INSTS_VALU_MUL_F64 SQ_INSTS_VALU_ADD_F64 SQ_INSTS_VALU_TRANS_F64"
PASS_B="SQ_INSTS_VALU SQ_INSTS_VALU_FMA_F32 SQ_INSTS_VALU_ADD_F32 SQ_INSTS_VALU_MUL_F32 SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_MFMA SQ_INSTS_VALU_MFMA_BF16"
run mix_a timeout -s KILL 300 rocprofv3 --pmc $PASS_A --output-format csv -d "$OUT/mix_a" -o pmc -- \
  python3 "$REPO/bench.py" --no-cpu $ARGS
run mix_b timeout -s KILL 300 rocprofv3 --pmc $PASS_B --output-format csv -d "$OUT/mix_b" -o pmc -- \
  python3 "$REPO/bench.py" --no-cpu $ARGS
run copy_fetch timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d "$OUT/copy_fetch" -o pmc -- \
  python3 "$REPO/bench.py" --copy-calibration 256
run copy_write timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d "$OUT/copy_write" -o pmc -- \
  python3 "$REPO/bench.py" --copy-calibration 256
# the summary compiles the kernels' assembly, which needs the generated table headers
cd "$REPO" || exit 1
if [ ! -f _build/llvq_tables.inc ] || [ ! -f _build/llvq_wide.inc ] || [ ! -f _build/llvq_search.inc ]; then
  python3 -c "from weight_decompression_amd import build_lib; build_lib.build_tables(verbose=False)" || exit $?
fi
python3 -m weight_decompression_amd.profile_summary "$OUT" "$ARGS" "$@" > "$OUT/summary.md" || exit $?
echo "profile done"
