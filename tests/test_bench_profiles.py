"""The benchmark's per-workload profile figures agree with the rocprofv3 summaries they cite.

bench.py reports a VALU roofline from lane-op counts, executed-mix peaks and HBM counter
bytes copied out of profiles/*.md; a summary refreshed without the table (or the reverse)
would make a bench line quote stale numbers.  CPU only: this reads files.
"""

import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

COMMENT = re.compile(r"<!-- profile (.+?) valu_lane_ops_per_unit=([0-9.]+) fetch=(\d+) write=(\d+) "
                     r"avg_ns=(\d+)(?: valu_mix_peak_tops=([0-9.]+))? -->")


def summary_kernels(path):
    with open(os.path.join(ROOT, path)) as f:
        text = f.read()
    out = []
    for m in COMMENT.finditer(text):
        out.append({"kernel": m.group(1), "ops": float(m.group(2)), "fetch": int(m.group(3)),
                     "write": int(m.group(4)), "mix": float(m.group(6)) if m.group(6) else None})
    return out


def test_every_entry_cites_an_existing_summary_of_one_source():
    shas = {v["source_sha256"] for v in bench.KERNEL_PROFILES.values()}
    assert len(shas) == 1, "profiles of different kernel sources in one table"
    for key, v in bench.KERNEL_PROFILES.items():
        assert os.path.exists(os.path.join(ROOT, v["summary"])), key
        assert summary_kernels(v["summary"]), key


@pytest.mark.parametrize("key", sorted(bench.KERNEL_PROFILES))
def test_entry_matches_its_summary(key):
    v = bench.KERNEL_PROFILES[key]
    ks = summary_kernels(v["summary"])
    ops = sum(k["ops"] for k in ks)
    # one kernel: the figures themselves; two kernels per step: their sum (search, round trip)
    assert abs(v["valu_lane_ops_per_unit"] - ops) <= 0.05 + 1e-9 * ops, (key, ops)
    if len(ks) == 1:
        assert v["fetch_bytes_per_launch"] == ks[0]["fetch"], key
        assert v["write_bytes_per_launch"] == ks[0]["write"], key
    else:
        assert v.get("fetch_bytes_per_launch") is None and v.get("write_bytes_per_launch") is None, key
    if v.get("valu_mix_peak_tops") is not None:
        mixes = [k["mix"] for k in ks]
        assert all(m is not None for m in mixes), key
        want = sum(k["ops"] * k["mix"] for k in ks) / ops     # lane-op weighted for two kernels
        assert abs(v["valu_mix_peak_tops"] - want) <= 0.006, (key, want)
