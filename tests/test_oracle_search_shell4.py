"""Pins for the oracle search's per-codeword closed forms past shell 2 (papernotes.org
page, 关键设计 1: multi-shell angular / Euclidean search; gist.science page, Methodik /
2. Multi-Shell Search).

Inside one (class, codeword) pair the oracle does not enumerate points: it pairs sorted
coordinates with sorted values (rearrangement inequality) and, for even classes whose
sign parity comes out wrong, subtracts 2 * min|x| * min(support value).  Shell 2 has no
class where these shortcuts can go wrong, so two classes of shell 4 are enumerated here
point by point, straight from the lattice's definition, and the best <x, v> per codeword
is compared with oracle.search.codeword_scores:

* even class 6 2^7 0^16 (777,216 points): two distinct support values, so the parity
  fix has a choice of which entry to flip and what value it carries;
* odd class 5 3^2 1^21 (24,870,912 points): three distinct absolute values, whose signed
  images 5, -3, 1 must be paired in sorted order.

The points are built from the Golay code alone (support = an octad, or the odd-coset
sign rule) and checked for membership by an independent vectorised test (common parity,
coordinate sum mod 8, residue pattern in a 2^24 codeword bitmap); the oracle's bijection
is used only to map the search's winner back to its index.
"""

import itertools

import numpy as np
import pytest

from oracle import bijection, golay, search

M = 4


def _membership(P):
    """Lattice membership of integer points P [n][24] without the oracle's leech module."""
    P = P.astype(np.int64)
    p = P[:, :1] & 1
    same = ((P & 1) == p).all(axis=1)
    sum_ok = ((P.sum(axis=1) - 4 * p[:, 0]) % 8) == 0
    want = np.where(p == 1, 1, 2)
    bits = (((P % 4) == want).astype(np.int64) << np.arange(24)).sum(axis=1)
    bitmap = np.zeros(1 << 24, dtype=bool)
    bitmap[np.array(golay.table(), dtype=np.int64)] = True
    return same & sum_ok & bitmap[bits]


def _class_of(leader, parity):
    for cl, base, _ in search.codeword_scores(np.ones(24), M):
        if cl.leader == tuple(leader) and cl.parity == parity:
            return cl, base
    raise AssertionError("class not in the table")


def _bits(mask):
    return np.array([(mask >> i) & 1 for i in range(24)], dtype=bool)


# ---------------------------------------------------------------------------
# even class 6 2^7 0^16

@pytest.fixture(scope="module")
def even_class():
    """Points [759][1024][24] of the class, grouped by octad in table order."""
    T = golay.table()
    off8 = golay.weight_offset()[8]
    octads = T[off8:off8 + 759]
    signs = np.array([[1 - 2 * ((s >> k) & 1) for k in range(8)] for s in range(256)], dtype=np.int64)
    groups = []
    for c in octads:
        sup = np.nonzero(_bits(c))[0]
        pts = []
        for p6 in range(8):
            mag = np.full(8, 2, dtype=np.int64)
            mag[p6] = 6
            vals = signs * mag[None, :]                      # [256][8]
            keep = (vals.sum(axis=1) % 8) == 0                # the even coset's sum rule
            full = np.zeros((int(keep.sum()), 24), dtype=np.int64)
            full[:, sup] = vals[keep]
            pts.append(full)
        groups.append(np.concatenate(pts))
    P = np.stack(groups).astype(np.int8)
    return P


def test_even_class_enumeration_is_the_class(even_class):
    P = even_class.reshape(-1, 24)
    assert P.shape[0] == 777216
    assert _membership(P).all()
    assert ((P.astype(np.int64) ** 2).sum(axis=1) == 16 * M).all()
    assert len({row.tobytes() for row in P[::97]}) == len(P[::97])
    cl, _ = _class_of((6,) + (2,) * 7 + (0,) * 16, 0)
    assert cl.size == 777216 and cl.w == 8
    # the oracle's unrank of sampled indices of the class lands in the enumerated set
    have = {row.tobytes() for row in P}
    rng = np.random.default_rng(40)
    for J in rng.integers(0, cl.size, size=300):
        v = np.array(bijection.unrank(cl.start + int(J), M), dtype=np.int8)
        assert v.tobytes() in have


def test_even_class_per_codeword_scores_match_enumeration(even_class):
    cl, base = _class_of((6,) + (2,) * 7 + (0,) * 16, 0)
    rng = np.random.default_rng(41)
    X = rng.standard_normal((24, 20)) * rng.choice([0.5, 1.0, 3.0], size=20)[None, :]
    dots = even_class.astype(np.float64) @ X                     # [759][1024][20]
    brute = dots.max(axis=1)                                     # best per codeword
    arg = dots.argmax(axis=1)
    fixed = 0
    for t in range(X.shape[1]):
        x = X[:, t]
        got = [s for c, b, s in search.codeword_scores(x, M) if c is cl][0]
        assert got.shape == (759,)
        assert np.allclose(got, brute[:, t], rtol=1e-12, atol=1e-12), t
        # the best point of a codeword whose signs cannot follow x on the support
        best_pts = even_class[np.arange(759), arg[:, t]].astype(np.int64)
        sup = best_pts != 0
        fixed += int((((np.sign(best_pts) != np.sign(x)[None, :]) & sup).any(axis=1)).sum())
        # and the class maximum with its codeword(s)
        best, winners = search.class_scores(x, M)[[c for c, _, _ in search.codeword_scores(x, M)].index(cl)]
        assert np.isclose(best, brute[:, t].max(), rtol=1e-12, atol=1e-12)
        assert winners == [base + int(j) for j in np.nonzero(np.isclose(brute[:, t], brute[:, t].max(),
                                                                          rtol=1e-12, atol=1e-12))[0]]
    # the parity fix was on the path of many (codeword, x) pairs
    assert fixed > 759 * X.shape[1] // 4


# ---------------------------------------------------------------------------
# odd class 5 3^2 1^21

@pytest.fixture(scope="module")
def odd_arrangements():
    """Absolute-value arrangements [6072][24] of 5 3^2 1^21."""
    out = []
    for p5 in range(24):
        rest = [i for i in range(24) if i != p5]
        for a, b in itertools.combinations(rest, 2):
            v = np.ones(24, dtype=np.int64)
            v[p5] = 5
            v[a] = v[b] = 3
            out.append(v)
    return np.array(out)


def _odd_points(A, masks):
    """Points [len(masks)][len(A)][24] of the odd coset: x_i = a_i if (a_i = 1 mod 4) equals
    (i in the codeword), else -a_i (the residue-1 positions form the codeword)."""
    inc = np.array([_bits(c) for c in masks])                     # [k][24]
    one = (A % 4) == 1                                            # [n][24]
    pos = one[None, :, :] == inc[:, None, :]
    return np.where(pos, A[None, :, :], -A[None, :, :])


def test_odd_class_enumeration_is_the_class(odd_arrangements):
    A = odd_arrangements
    assert A.shape == (6072, 24)
    T = golay.table()
    total = 0
    rng = np.random.default_rng(42)
    for k0 in range(0, 4096, 512):
        P = _odd_points(A, T[k0:k0 + 512]).reshape(-1, 24)
        ok = ((P.sum(axis=1) - 4) % 8) == 0
        assert ok.all()                       # the class is valid for every codeword
        total += P.shape[0]
        samp = P[rng.choice(P.shape[0], 4000, replace=False)]
        assert _membership(samp).all()
    assert total == 24870912
    cl, _ = _class_of((5, 3, 3) + (1,) * 21, 1)
    assert cl.size == total
    for J in rng.integers(0, cl.size, size=200):
        v = np.array(bijection.unrank(cl.start + int(J), M), dtype=np.int64)
        assert sorted(np.abs(v).tolist()) == sorted(A[0].tolist()) and _membership(v[None, :]).all()


def test_odd_class_per_codeword_scores_match_enumeration(odd_arrangements):
    cl, base = _class_of((5, 3, 3) + (1,) * 21, 1)
    assert base == 0
    A = odd_arrangements
    T = golay.table()
    rng = np.random.default_rng(43)
    X = rng.standard_normal((24, 12)) * rng.choice([0.5, 1.0, 3.0], size=12)[None, :]
    brute = np.empty((4096, X.shape[1]))
    for k0 in range(0, 4096, 128):
        P = _odd_points(A, T[k0:k0 + 128]).astype(np.float64)     # [128][6072][24]
        brute[k0:k0 + 128] = (P @ X).max(axis=1)
    for t in range(X.shape[1]):
        got = [s for c, b, s in search.codeword_scores(X[:, t], M) if c is cl][0]
        assert got.shape == (4096,)
        assert np.allclose(got, brute[:, t], rtol=1e-12, atol=1e-12), t


# ---------------------------------------------------------------------------
# search() against the enumerated classes

def _objective(dots, m, mode):
    return dots / (4.0 * np.sqrt(m)) if mode == "angular" else 2.0 * dots - 16.0 * m


@pytest.mark.parametrize("mode", ["angular", "euclid"])
def test_search_winner_is_never_beaten_by_the_enumerated_classes(even_class, odd_arrangements, mode):
    # For random x the search's winner over shells 2..4 must score at least the best point
    # of each enumerated class, and for x next to a point of one of them it must return
    # that point (the nearest lattice point, whose direction is also the closest) with
    # the point's own index.
    T = golay.table()
    ev = even_class.reshape(-1, 24).astype(np.float64)
    rng = np.random.default_rng(44 if mode == "angular" else 45)
    odd_pts = _odd_points(odd_arrangements, [T[k] for k in rng.choice(4096, 64, replace=False)]).reshape(-1, 24)
    for t in range(6):
        x = rng.standard_normal(24) * (1.0 if t % 2 else 3.0)
        I, v = search.search(x, M, mode)
        v = np.asarray(v, dtype=np.float64)
        top = _objective(v @ x, (v @ v) / 16.0, mode)
        assert top >= _objective((ev @ x).max(), M, mode) - 1e-9
        assert top >= _objective((odd_pts @ x).max(), M, mode) - 1e-9
    for src in (ev, odd_pts.astype(np.float64)):
        for j in rng.choice(src.shape[0], 4, replace=False):
            p = src[j]
            x = p + rng.normal(0.0, 0.15, size=24)
            I, v = search.search(x, M, mode)
            assert v == [int(a) for a in p]
            assert I == bijection.rank([int(a) for a in p], M)
            d = src @ x
            assert int(np.argmax(_objective(d, M, mode))) == j
