"""Pins for the oracle's index <-> point bijection.

* exhaustive on shell 2: 196,560 indices decode to 196,560 distinct lattice points of
  the right norm, and rank inverts unrank on each (injective + count = bijective);
* random indices on every shell 3..10 (and exhaustive shell 3 with -m slow);
* the lexicographic multiset rank agrees with sorting the distinct permutations by
  brute force (itertools), the textbook definition of lexicographic order;
* regression vectors for the conventions (values worked out by hand from the stated
  conventions: the first index of a class is its lexicographically smallest arrangement
  with the first codeword of the weight slice and no free negative signs).
"""

import itertools
import multiprocessing as mp
import random

import numpy as np
import pytest

from oracle import bijection, classes, golay, leech

M = 10


def test_multiset_rank_matches_bruteforce_lex_order():
    for values in ([0, 0, 4, 4, 8], [1, 1, 1, 3, 5, 5], [2, 2, 6], [1, 3, 3, 3, 5, 7, 7], [0] * 5 + [4]):
        perms = sorted(set(itertools.permutations(values)))
        for r, p in enumerate(perms):
            assert bijection.multiset_unrank(r, values) == list(p)
            assert bijection.multiset_rank(list(p)) == r


def _chunk_check(args):
    lo, hi = args
    pts = []
    for I in range(lo, hi):
        x = bijection.unrank(I, 2)
        if not leech.in_leech(x) or leech.norm2(x) != 32:
            return ("bad point", I)
        if bijection.rank(x, 2) != I:
            return ("rank mismatch", I)
        pts.append(bytes((v + 16) for v in x))
    return pts


def _exhaustive(lo, hi, max_shell):
    n = hi - lo
    step = max(1, n // 64)
    chunks = [(a, min(a + step, hi)) for a in range(lo, hi, step)]
    with mp.get_context("fork").Pool(min(8, mp.cpu_count())) as pool:
        seen = set()
        for res in pool.imap_unordered(_chunk_check, chunks):
            assert isinstance(res, list), res
            seen.update(res)
    return seen


def test_exhaustive_shell2_bijection():
    seen = _exhaustive(0, 196560, 2)
    assert len(seen) == 196560


def _chunk_check3(args):
    lo, hi = args
    out = []
    for I in range(lo, hi):
        x = bijection.unrank(I, 3)
        if not leech.in_leech(x) or leech.norm2(x) != 48:
            return ("bad point", I)
        if bijection.rank(x, 3) != I:
            return ("rank mismatch", I)
        out.append(hash(tuple(x)))
    return out


@pytest.mark.slow
def test_exhaustive_shell3_bijection():
    lo, hi = 196560, 16969680
    step = 50000
    chunks = [(a, min(a + step, hi)) for a in range(lo, hi, step)]
    with mp.get_context("fork").Pool(min(8, mp.cpu_count())) as pool:
        total = 0
        hashes = set()
        for res in pool.imap_unordered(_chunk_check3, chunks):
            assert isinstance(res, list), res
            total += len(res)
            hashes.update(res)
    assert total == 16773120
    assert len(hashes) == 16773120


@pytest.mark.parametrize("m", range(3, 11))
def test_random_round_trip_per_shell(m):
    rnd = random.Random(100 + m)
    C = leech.cumulative_counts(M)
    for _ in range(400):
        I = rnd.randrange(C[m - 1], C[m])
        x = bijection.unrank(I, M)
        assert leech.in_leech(x)
        assert leech.norm2(x) == 16 * m
        assert bijection.rank(x, M) == I


def test_every_class_boundary_round_trips():
    for c in classes.class_table(M):
        for I in (c.start, c.start + 1, c.end - 2, c.end - 1):
            if c.start <= I < c.end:
                x = bijection.unrank(I, M)
                assert leech.in_leech(x) and leech.norm2(x) == 16 * c.m
                assert bijection.rank(x, M) == I


def test_index_radix_follows_the_page():
    # I_class = r + A * (s + 2^B * I''): r picks the codeword, s the signs, I'' the order.
    rnd = random.Random(9)
    T = golay.table()
    off = golay.weight_offset()
    for c in classes.class_table(M)[::5]:
        J = rnd.randrange(c.size)
        r, Ip = J % c.A, J // c.A
        s, R = Ip % (1 << c.B), Ip >> c.B
        x = bijection.unrank(c.start + J, M)
        if c.parity == 1:
            mask = sum(1 << i for i, v in enumerate(x) if v % 4 == 1)
            assert mask == T[r]
            assert bijection.multiset_rank([abs(v) for v in x]) == R
        else:
            mask = sum(1 << i for i, v in enumerate(x) if v % 4 == 2)
            assert mask == T[off[c.w] + r]


def test_regression_vectors():
    cases = {
        0: [2, 2, 2, 2, 2, 0, 0, 2, 0, 0, 2, 0, 2, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0],
        97152: [0] * 22 + [4, 4],
        98256: [-1] * 23 + [3],
        196560: [2, 0, 2, 2, 2, 0, 2, 2, 2, 2, 2, 2, 0, 2, 2, 0, 0, 0, 0, 0, 0, 0, 0, 0],
        13503934538639: [-11, -3, -3] + [1] * 21,
        12345678901234: [-1, -1, 3, 3, 1, -1, -1, 1, 1, -1, -3, -7, 5, 1, -1, 3, 3, 1, 3, -3, 3, 1, 1, 1],
    }
    for I, x in cases.items():
        assert bijection.unrank(I, M) == x
        assert bijection.rank(x, M) == I


def test_even_class_sign_bit_order():
    # Worked by hand from the stated conventions.  Class 4.2^8.0^15 of shell 3 starts at
    # 5,472,208 (w = 8, A = 759, B = 8, P_S = 1, P_T = 16, pi = (8*2 + 4)/4 mod 2 = 1).
    # Take r = 0 (codeword T[1] = 0x00149f: positions 0,1,2,3,4,7,10,12; q = 12),
    # s = 2^5 and I'' = 15: the complement arrangement of rank 15 puts the 4 on the first
    # complement position (5).  Free positions in order: support 0,1,2,3,4,7,10 then the
    # nonzero complement position 5, so bit 5 makes position 7 negative; one negative on
    # the support already has parity pi, so q stays positive.
    I = 5472208 + 0 + 759 * ((1 << 5) + 256 * 15)
    x = [2, 2, 2, 2, 2, 4, 0, -2, 0, 0, 2, 0, 2] + [0] * 11
    assert bijection.unrank(I, 10) == x
    assert bijection.rank(x, 10) == I
    # bit 7 is the complement position: -4 there, and q flips to restore parity pi
    I2 = 5472208 + 759 * ((1 << 7) + 256 * 15)
    x2 = [2, 2, 2, 2, 2, -4, 0, 2, 0, 0, 2, 0, -2] + [0] * 11
    assert bijection.unrank(I2, 10) == x2
    assert bijection.rank(x2, 10) == I2


def test_rank_rejects_bad_points():
    with pytest.raises(ValueError):
        bijection.rank([1] * 24, M)                 # norm 24 is not a lattice point here
    with pytest.raises(ValueError):
        bijection.rank([0] * 24, M)                 # origin is outside the shell union
    x = bijection.unrank(leech.index_count(M) - 1, M)
    with pytest.raises(ValueError):
        bijection.rank(x, 9)                        # shell 10 point, union only up to 9
    with pytest.raises(ValueError):
        bijection.unrank(leech.index_count(M), M)   # index past C_M


def test_values_bounded_by_12():
    rnd = random.Random(4)
    for _ in range(2000):
        x = bijection.unrank(rnd.randrange(leech.index_count(M)), M)
        assert max(abs(v) for v in x) <= 12
    assert max(max(c.leader) for c in classes.class_table(M)) == 12


def test_uniform_indices_split_even_odd_about_evenly():
    C = leech.index_count(M)
    odd = sum(c.size for c in classes.class_table(M) if c.parity == 1)
    assert abs(odd / C - 0.5) < 0.02
    _ = np  # numpy imported for pool workers' environment
