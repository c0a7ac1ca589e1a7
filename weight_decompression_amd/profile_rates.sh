#!/bin/bash
# VALU issue rates of gfx950 and the SQ counter category of each timed instruction.
# Usage (from the repository root, on a machine with the GPU):
#   bash weight_decompression_amd/profile_rates.sh OUTDIR
# Runs issue_rates.py under the two per-type counter passes (issue_rates.MIX_PASSES), then
# once more for the rates, and writes OUTDIR/rates.md (the table profile_summary.py reads).
set -o pipefail
OUT="$(cd "$(dirname "$1")" && pwd)/$(basename "$1")"
REPO="$(cd "$(dirname "$0")/.." && pwd)"
mkdir -p "$OUT"
cd /tmp && export TMPDIR=/tmp
export PYTHONPATH="$REPO"
PASS_A="SQ_INSTS_VALU SQ_INSTS_VALU_INT32 SQ_INSTS_VALU_INT64 SQ_INSTS_VALU_CVT SQ_INSTS_VALU_FMA_F64 SQ_INSTS_VALU_MUL_F64 SQ_INSTS_VALU_ADD_F64 SQ_INSTS_VALU_TRANS_F64"
PASS_B="SQ_INSTS_VALU SQ_INSTS_VALU_FMA_F32 SQ_INSTS_VALU_ADD_F32 SQ_INSTS_VALU_MUL_F32 SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_MFMA SQ_INSTS_VALU_MFMA_BF16"
run() { echo "== $1 $(date +%T)"; shift; "$@" || exit $?; }
run rates_a timeout -s KILL 120 rocprofv3 --pmc $PASS_A --output-format csv -d "$OUT/rates_a" -o pmc -- \
  python3 -m weight_decompression_amd.issue_rates --reps 1
run rates_b timeout -s KILL 120 rocprofv3 --pmc $PASS_B --output-format csv -d "$OUT/rates_b" -o pmc -- \
  python3 -m weight_decompression_amd.issue_rates --reps 1
run rates timeout -k 10 120 python3 -m weight_decompression_amd.issue_rates --categories "$OUT/rates_a" "$OUT/rates_b" \
  > "$OUT/rates.md"
echo "rates done"
