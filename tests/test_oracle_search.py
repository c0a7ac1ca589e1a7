"""Pins for the oracle's exact search: literal enumeration of whole shells on tiny
random inputs must pick the same point (the method's angular and Euclidean objectives,
papernotes.org page 关键设计 1; gist.science page Methodik / 2. Multi-Shell Search)."""

import multiprocessing as mp

import numpy as np
import pytest

from oracle import bijection, leech, search


def _points(args):
    lo, hi, M = args
    return np.array([bijection.unrank(I, M) for I in range(lo, hi)], dtype=np.int8)


def _enumerate(M):
    hi = leech.index_count(M)
    step = 100000
    chunks = [(a, min(a + step, hi), M) for a in range(0, hi, step)]
    with mp.get_context("fork").Pool(min(8, mp.cpu_count())) as pool:
        return np.concatenate(pool.map(_points, chunks))


@pytest.fixture(scope="module")
def shell2_points():
    return _enumerate(2)


def _brute(P, norms2, x, mode):
    dots = P.astype(np.float64) @ x
    if mode == "angular":
        obj = dots / np.sqrt(norms2)
    else:
        obj = 2 * dots - norms2
    return int(np.argmax(obj))   # first maximum = smallest index


def test_angular_and_euclid_match_bruteforce_on_shell2(shell2_points):
    P = shell2_points
    n2 = (P.astype(np.int64) ** 2).sum(axis=1).astype(np.float64)
    rng = np.random.default_rng(1)
    for t in range(12):
        x = rng.standard_normal(24) * (3.0 if t % 2 else 0.7)
        for mode in ("angular", "euclid"):
            I, v = search.search(x, 2, mode)
            assert I == _brute(P, n2, x, mode), (t, mode)
            assert list(P[I]) == v


@pytest.mark.slow
def test_angular_and_euclid_match_bruteforce_on_shells_2_3():
    P = _enumerate(3)
    assert P.shape[0] == 16969680
    n2 = (P.astype(np.int64) ** 2).sum(axis=1).astype(np.float64)
    rng = np.random.default_rng(2)
    for t in range(6):
        x = rng.standard_normal(24) * (4.0 if t % 2 else 1.0)
        for mode in ("angular", "euclid"):
            I, _ = search.search(x, 3, mode)
            assert I == _brute(P, n2, x, mode), (t, mode)


def test_search_beats_random_lattice_points():
    rng = np.random.default_rng(3)
    C = leech.index_count(10)
    for _ in range(3):
        x = rng.standard_normal(24)
        I, v = search.search(x, 10, "angular")
        assert leech.in_leech(v)
        best = np.dot(x, v) / np.linalg.norm(v)
        for _ in range(200):
            u = bijection.unrank(int(rng.integers(0, C)), 10)
            assert np.dot(x, u) / np.linalg.norm(u) <= best + 1e-12


def test_shape_gain_fidelity_band():
    # Loose context, not an exact pin: the pages report MSE 0.078 for LLVQ shape-gain on
    # a unit Gaussian at 2 bit/dim (with a 1-2 bit gain).  Here the shape alone (the
    # exact block norm as gain, shells 2..10, 44-bit shape index) must land near
    # 0.08-0.09; a random 16-entry gain table adds error that depends on the draw.
    rng = np.random.default_rng(4)
    err = 0.0
    n = 40
    for _ in range(n):
        w = rng.standard_normal(24)
        _, v = search.search(w, 10, "angular")
        v = np.asarray(v, dtype=np.float64)
        w_hat = np.linalg.norm(w) * v / np.linalg.norm(v)
        err += np.sum((w - w_hat) ** 2)
    mse = err / (24 * n)
    assert 0.06 < mse < 0.11, mse


def test_nearest_gain_ties_go_low():
    assert search.nearest_gain(1.5, [1.0, 2.0, 3.0]) == 0
    assert search.nearest_gain(2.9, [1.0, 2.0, 3.0]) == 2


def test_angular_collinear_tie_goes_to_the_shell2_point(shell2_points):
    # The angular objective ignores |v|: u (shell 2) and 2u (shell 8) tie exactly, and the
    # smaller index is u's.  x = u (and x = 2u) must come back as u with M = 10.
    rng = np.random.default_rng(3)
    C2 = leech.index_count(2)
    for I in rng.integers(0, C2, size=6):
        u = [int(a) for a in shell2_points[int(I)]]
        for x in (np.array(u, dtype=np.float64), 2.0 * np.array(u, dtype=np.float64)):
            J, v = search.search(x, 10, "angular")
            assert (J, v) == (int(I), u)
        assert search.smallest_on_ray([2 * a for a in u]) == u


def test_smallest_on_ray_only_for_halvable_shell8_points(shell2_points):
    # a shell-8 point with even coordinates halves to a lattice point exactly when its half
    # is one of the enumerated shell-2 points
    s2 = {tuple(int(a) for a in p) for p in shell2_points}
    rng = np.random.default_rng(4)
    lo, hi = leech.index_count(7), leech.index_count(8)
    seen_even = 0
    for I in rng.integers(lo, hi, size=4000):
        v = bijection.unrank(int(I), 8)
        h = search.smallest_on_ray(v)
        if all(a % 2 == 0 for a in v):
            seen_even += 1
            half = tuple(a // 2 for a in v)
            assert (h is not None) == (half in s2)
            if h is not None:
                assert tuple(h) == half
        else:
            assert h is None
    assert seen_even > 0
    assert search.smallest_on_ray(bijection.unrank(5, 10)) is None      # a shell-2 point


def test_angular_collinear_tie_shell12_goes_to_the_shell3_point():
    # up to shell 13 the other collinear pair: u in shell 3 and 2u in shell 12 tie exactly
    # under the angular objective; x = u and x = 2u come back as u at M = 12 and 13
    rng = np.random.default_rng(12)
    lo, hi = leech.index_count(2), leech.index_count(3)
    for I in rng.integers(lo, hi, size=4):
        u = bijection.unrank(int(I), 3)
        assert search.smallest_on_ray([2 * a for a in u]) == u
        assert search.smallest_on_ray(u) is None
        for M in (12, 13):
            for x in (np.array(u, dtype=np.float64), 2.0 * np.array(u, dtype=np.float64)):
                J, v = search.search(x, M, "angular")
                assert (J, v) == (int(I), u)


def test_smallest_on_ray_rejects_non_lattice_fractions():
    # 2w for a shell-2 point w is in shell 8; 4w (shell 32) halves twice, to w
    w = bijection.unrank(777, 2)
    assert search.smallest_on_ray([4 * a for a in w]) == w
    # a shell-12 point with all coordinates even whose half is not a lattice point
    rng = np.random.default_rng(13)
    lo, hi = leech.index_count(11), leech.index_count(12)
    found = 0
    for I in rng.integers(lo, hi, size=3000):
        v = bijection.unrank(int(I), 12)
        if all(a % 2 == 0 for a in v):
            h = search.smallest_on_ray(v)
            half = [a // 2 for a in v]
            assert (h == half) == leech.in_leech(half)
            found += 1
    assert found > 0
