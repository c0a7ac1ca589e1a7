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


def _inc_array(text, name):
    """Initialiser of array `name` in the generated include: a list of the numbers, or of
    brace groups of numbers."""
    import re
    start = text.index(name + "[")
    body = text[text.index("{", start) + 1:text.index("};", start)]
    if "{" in body:
        return [[float(v.strip().rstrip("fu")) for v in g.split(",") if v.strip()]
                for g in re.findall(r"\{([^}]*)\}", body)]
    return [int(v.strip().rstrip("u"), 0) for v in body.replace("\n", "").split(",") if v.strip()]


@pytest.mark.parametrize("n", [6, 7])
def test_tail_tables_are_the_sorted_arrangements(gen, n):
    # the table of the last n value slots: every composition's group holds its distinct
    # arrangements in lexicographic order (brute force over itertools), and the record
    # holds Q / n and the group's offset
    import itertools
    with open(build_lib.TABLES_INC) as f:
        text = f.read()
    tail = _inc_array(text, "kTail%d" % n)
    comp = _inc_array(text, "kTailComp%d" % n)
    b = n + 1
    assert len(tail) == 4 ** n and len(comp) == b ** 3
    seen = 0
    for c0 in range(n + 1):
        for c1 in range(n + 1 - c0):
            for c2 in range(n + 1 - c0 - c1):
                c3 = n - c0 - c1 - c2
                seq = [0] * c0 + [1] * c1 + [2] * c2 + [3] * c3
                arr = sorted(set(itertools.permutations(seq)))
                q_over_n, off = comp[c0 + b * c1 + b * b * c2]
                assert q_over_n == pytest.approx(len(arr) / n, rel=1e-7)
                got = tail[int(off):int(off) + len(arr)]
                assert got == [sum(s << (2 * i) for i, s in enumerate(a)) for a in arr]
                seen += len(arr)
    assert seen == 4 ** n


@pytest.mark.parametrize("name,scale", [("kEvenIdx", 1), ("kEvenPos", 2)])
def test_even_position_table_is_the_even_decode_order(gen, name, scale):
    # for every codeword of the (oracle's) sorted Golay table: its positions ascending, then
    # the other positions ascending, as bytes p (kEvenIdx) or 2 p (kEvenPos)
    with open(build_lib.TABLES_INC) as f:
        text = f.read()
    words = _inc_array(text, name)
    table = list(golay.table())
    assert len(words) == 6 * len(table) == 6 * 4096
    for i, c in enumerate(table):
        order = [p for p in range(24) if (c >> p) & 1] + [p for p in range(24) if not (c >> p) & 1]
        got = [(words[6 * i + q // 4] >> (8 * (q % 4))) & 0xFF for q in range(24)]
        assert got == [scale * p for p in order], i
