#!/bin/bash
# Profile the batch-1 fused GEMV of bench.py with rocprofv3 on one GPU.
# Usage (from the repository root, on a machine with the GPU):
#   bash weight_decompression_amd/profile_gemv.sh OUTDIR
# Writes OUTDIR/trace (kernel trace + stats), OUTDIR/pmc_valu, OUTDIR/pmc_fetch,
# OUTDIR/pmc_write and OUTDIR/copy_{fetch,write} (plain-copy calibration, 256 MiB), then
# OUTDIR/summary.md (weight_decompression_amd/profile_summary.py).
# Workload: bench.py's 4096 x 11008 batch-1 GEMV, 1,880,064 blocks, 11,318,784 algorithmic
# bytes per launch (6 B per block + 2 B per column of x + 4 B per row of y).
set -o pipefail
OUT="$(cd "$(dirname "$1")" && pwd)/$(basename "$1")"
REPO="$(cd "$(dirname "$0")/.." && pwd)"
mkdir -p "$OUT"
cd /tmp && export TMPDIR=/tmp
run() { echo "== $1"; shift; "$@" || exit $?; }
run trace timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/trace" -o run -- \
  python3 "$REPO/bench.py" --steps 200 --warmup 10 --no-cpu
run valu timeout -s KILL 120 rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_WAVES SQ_ACTIVE_INST_VALU \
  SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE --output-format csv -d "$OUT/pmc_valu" -o pmc -- \
  python3 "$REPO/bench.py" --steps 10 --warmup 2 --no-cpu
run fetch timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d "$OUT/pmc_fetch" -o pmc -- \
  python3 "$REPO/bench.py" --steps 10 --warmup 2 --no-cpu
run write timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d "$OUT/pmc_write" -o pmc -- \
  python3 "$REPO/bench.py" --steps 10 --warmup 2 --no-cpu
run copy_fetch timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d "$OUT/copy_fetch" -o pmc -- \
  python3 "$REPO/bench.py" --copy-calibration 256
run copy_write timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d "$OUT/copy_write" -o pmc -- \
  python3 "$REPO/bench.py" --copy-calibration 256
cd "$REPO" && python3 -m weight_decompression_amd.profile_summary "$OUT" k_gemv_b1 1880064 11318784 268435456 \
  "bash weight_decompression_amd/profile_gemv.sh $1" > "$OUT/summary.md" || exit $?
echo "profile done"
