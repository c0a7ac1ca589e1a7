"""The HIP library's tables come from a C++ generator written separately from the
oracle; its output must equal the oracle's Golay table and class table value for
value (outputs compared, no code shared)."""

import json
import os
import subprocess

import pytest

from oracle import classes, golay, leech
from weight_decompression_amd import build_lib


@pytest.fixture(scope="module")
def gen():
    build_lib.build_tables(verbose=False)
    with open(build_lib.TABLES_JSON) as f:
        return json.load(f)


def test_golay_table_equal(gen):
    assert gen["golay"] == list(golay.table())


def test_class_table_equal(gen):
    ours = classes.class_table(10)
    assert len(gen["classes"]) == len(ours) == 168
    for g, o in zip(gen["classes"], ours):
        assert (g["m"], g["parity"], g["w"], g["A"], g["B"], g["P_S"], g["P_T"], g["pi"]) == \
               (o.m, o.parity, o.w, o.A, o.B, o.P_S, o.P_T, o.pi)
        assert int(g["start"]) == o.start and int(g["size"]) == o.size
        assert tuple(g["leader"]) == o.leader


def test_index_counts_equal(gen):
    for M in range(2, 11):
        assert int(gen["index_count"][str(M)]) == leech.index_count(M)


def test_generator_rejects_bad_usage():
    r = subprocess.run([build_lib.GEN_BIN], capture_output=True)
    assert r.returncode == 2
    assert os.path.exists(build_lib.TABLES_INC)


def test_wide_class_table_equal(gen):
    # the general decoder's records (shells 2..42, 128-bit starts) against the oracle
    with open(build_lib.WIDE_JSON) as f:
        wide = json.load(f)
    M = wide["max_shell"]
    assert M == 42
    ours = classes.class_table(M)
    assert len(wide["classes"]) == len(ours)
    for g, o in zip(wide["classes"], ours):
        assert (g["m"], g["parity"], g["w"], g["A"], g["B"], g["P_S"], g["P_T"], g["pi"]) == \
               (o.m, o.parity, o.w, o.A, o.B, o.P_S, o.P_T, o.pi)
        assert int(g["start"]) == o.start and int(g["size"]) == o.size
        sup = sorted(set(o.support_values))
        comp = sorted(set(o.complement_values))
        assert g["support"] == [[v, o.support_values.count(v)] for v in sup]
        assert g["complement"] == [[v, o.complement_values.count(v)] for v in comp]
    counts = leech.cumulative_counts(M + 1)
    for m in range(2, M + 2):
        assert int(wide["shell_start"][m]) == counts[m - 1]
        first = wide["shell_first"][m]
        assert first == len(ours) or (ours[first].m == m and (first == 0 or ours[first - 1].m == m - 1))
