"""The nearest-point search kernel runs device code that the C++ table generator writes
(`gen_tables --search`): a 24-element sorting network and, per class, the objective of
the class's best point for one codeword as an expression in prefix sums of sorted
coordinates.  These tests read that generated file and check it against the oracle
(outputs compared, no code shared):

* the network sorts (random floats, and the generator's own 0-1 check passed);
* each class's record (ascending values, shell, coset, weight, sign parity) equals the
  oracle's class table;
* each class's objective expression, evaluated on prefix sums of a random block, equals
  the oracle's objective of the best point of that class for that codeword, for
  codewords of every weight, both objectives;
* the expressions appear shell by shell, so a search limited to shells <= M sees exactly
  the classes of those shells (shells 2..13).
"""

import re

import numpy as np
import pytest

from oracle import classes, golay, search
from weight_decompression_amd import build_lib

M_SEARCH = 13          # the search covers shells 2..13 (383 classes)

FN_RE = re.compile(r"__device__ __forceinline__ (?:float|int) (llvq_\w+)\(.*?\) \{\n(.*?)\n\}\n", re.S)


@pytest.fixture(scope="module")
def inc():
    build_lib.build_tables(verbose=False)
    with open(build_lib.SEARCH_INC) as f:
        return f.read()


def _network(inc):
    body = inc[inc.index("void llvq_sort24"):inc.index("struct LlvqSearchClass")]
    ces = [(int(a), int(b)) for a, b in re.findall(r"const T a = v\[(\d+)\], b = v\[(\d+)\];", body)]
    final = [int(v) for v in re.findall(r"v\[(\d+)\]", body[body.index("const T s[24]"):])[:24]]
    return ces, final


def _run_network(ces, final, v):
    v = list(v)
    for a, b in ces:
        lo, hi = min(v[a], v[b]), max(v[a], v[b])
        v[a], v[b] = lo, hi
    return [v[i] for i in final]


def test_sorting_network_sorts(inc):
    ces, final = _network(inc)
    assert sorted(final) == list(range(24))
    rng = np.random.default_rng(1)
    for _ in range(300):
        x = rng.normal(size=24)
        if rng.random() < 0.3:
            x = np.round(x * 2) / 2    # repeated values
        assert _run_network(ces, final, x) == sorted(x)


def _class_records(inc):
    body = inc[inc.index("kSearchClass["):]
    body = body[:body.index("};")]
    recs = []
    for vals, rest in re.findall(r"\{\{([-\d,]+)\}, ([\d, ]+)\}", body):
        recs.append((tuple(int(v) for v in vals.split(",")), tuple(int(v) for v in rest.split(","))))
    return recs


def test_class_records_match_oracle(inc):
    recs = _class_records(inc)
    ours = classes.class_table(M_SEARCH)
    assert len(recs) == len(ours) == 383
    assert f"#define LLVQ_SEARCH_MAX_SHELL {M_SEARCH}" in inc
    for (vals, (m, parity, w, pi)), c in zip(recs, ours):
        assert (m, parity, w, pi) == (c.m, c.parity, c.w, c.pi)
        if c.parity:
            want = sorted(a if a % 4 == 1 else -a for a in c.complement_values)
        else:
            want = list(c.support_values) + list(c.complement_values)
        assert list(vals) == want


def _py(expr):
    """C expression of the generated code -> Python (fp64 evaluation of the same terms)."""
    e = expr.replace("__builtin_fmaf", "_fma")
    return re.sub(r"(-?\d\.\d+e[+-]\d+)f", r"\1", e)


def _fma(a, b, c):
    return a * b + c


def _argmax_bodies(inc):
    """{function name: [(class k, python expr or None for a shell break (M < m))]}"""
    out = {}
    for name, body in FN_RE.findall(inc):
        if "_argmax_" not in name:
            continue
        items = []
        for line in body.split("\n"):
            mb = re.match(r"\s*if \(M < (\d+)\) goto done;", line)
            if mb:
                items.append((None, int(mb.group(1))))
                continue
            mo = re.match(r"\s*\{ const float o = (.*); if \(o > best\) \{ best = o; k = (\d+); \} \}", line)
            if mo:
                items.append((int(mo.group(2)), _py(mo.group(1))))
        out[name] = items
    return out


def _objective(x, v, m, euclid):
    s = float(np.dot(x, v))
    return 2.0 * s - 16.0 * m if euclid else s / (4.0 * np.sqrt(m))


@pytest.mark.parametrize("euclid", [False, True])
def test_class_objectives_match_oracle_points(inc, euclid):
    fns = _argmax_bodies(inc)
    cls = classes.class_table(M_SEARCH)
    T = golay.table()
    rng = np.random.default_rng(7 + euclid)
    suffix = "_euclid" if euclid else "_angular"
    by_weight = {}
    for pos, c in enumerate(T):
        by_weight.setdefault(bin(c).count("1"), []).append(c)
    seen = set()
    for trial in range(6):
        x = rng.normal(size=24) * (3.0 if euclid else 1.0)
        # odd coset: every odd class against a few codewords of any weight
        for c in [T[int(i)] for i in rng.integers(0, 4096, size=3)]:
            inc_c = np.array([(c >> i) & 1 for i in range(24)], dtype=bool)
            y = np.where(inc_c, x, -x)
            S = np.concatenate([[0.0], np.cumsum(np.sort(y))])
            for k, expr in fns["llvq_odd_argmax" + suffix]:
                if k is None:
                    continue
                got = eval(expr, {"_fma": _fma, "S": S})
                v = search._odd_point(x, cls[k], c)
                want = _objective(x, v, cls[k].m, euclid)
                assert abs(got - want) <= 1e-6 * (1.0 + abs(want)), (k, c, got, want)
                seen.add(k)
        # even coset: every weight, a few codewords each
        for w, words in by_weight.items():
            name = f"llvq_even{w}_argmax" + suffix
            for c in [words[int(i)] for i in rng.integers(0, len(words), size=2)]:
                sup = [i for i in range(24) if (c >> i) & 1]
                comp = [i for i in range(24) if not (c >> i) & 1]
                ax = np.abs(x)
                Ss = np.concatenate([[0.0], np.cumsum(np.sort(ax[sup]))])
                Sc = np.concatenate([[0.0], np.cumsum(np.sort(ax[comp]))])
                wrong1 = (sum(1 for i in sup if x[i] < 0) % 2) != 1
                m2 = -2.0 * (np.sort(ax[sup])[0] if sup else 0.0)
                pen = {"pen0": 0.0 if wrong1 else m2, "pen1": m2 if wrong1 else 0.0}
                for k, expr in fns[name]:
                    if k is None:
                        continue
                    got = eval(expr, {"_fma": _fma, "Ss": Ss, "Sc": Sc, **pen})
                    v = search._even_point(x, cls[k], c)
                    want = _objective(x, v, cls[k].m, euclid)
                    assert abs(got - want) <= 1e-6 * (1.0 + abs(want)), (k, w, c, got, want)
                    seen.add(k)
    assert seen == set(range(383))


def test_shell_breaks_follow_class_shells(inc):
    # each class is preceded by the limit check of its own shell (shell 2 needs none)
    cls = classes.class_table(M_SEARCH)
    for name, items in _argmax_bodies(inc).items():
        shell = 2
        for k, item in items:
            if k is None:
                assert item > shell, (name, item, shell)
                shell = item
            else:
                assert cls[k].m == shell, (name, k, cls[k].m, shell)
                want_parity = 1 if name.startswith("llvq_odd") else 0
                assert cls[k].parity == want_parity
                if want_parity == 0:
                    assert f"llvq_even{cls[k].w}_" in name
