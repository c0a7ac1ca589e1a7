"""Pins for the oracle's lattice, shells and class table.

Fixed numbers come from the pages (kissing number 196,560; about 0.75 bit/dim for the
first shell; 4096 codewords), from the workload statement (shell sizes 196,560 /
16,773,120 / 398,034,000 and the 25-bit index range [0, 16,969,680)), and from
textbook facts (the Leech theta series).  Every count is reached by at least two
independent routes."""

import math
import random

import pytest

from oracle import classes, golay, leech
from oracle.bijection import unrank


def test_published_shell_sizes():
    assert leech.shell_size_closed_form(2) == 196560      # kissing number
    assert leech.shell_size_closed_form(3) == 16773120
    assert leech.shell_size_closed_form(4) == 398034000
    assert leech.shell_size_closed_form(1) == 0           # no vectors of norm 2


def test_first_shell_rate_about_three_quarter_bit():
    rate = math.log2(196560) / 24
    assert abs(rate - 0.75) < 0.02


def test_tau_known_values():
    t = leech.tau_table(6)
    assert t[1:7] == (1, -24, 252, -1472, 4830, -6048)


@pytest.mark.parametrize("m", range(1, 12))
def test_closed_form_equals_coordinate_dp(m):
    assert leech.shell_size_dp(m) == leech.shell_size_closed_form(m)


def test_class_sums_equal_shell_sizes():
    sizes = classes.class_sizes_by_shell(10)
    for m in range(2, 11):
        assert sizes[m] == leech.shell_size_closed_form(m)


def test_index_range_and_max_shell():
    assert leech.index_count(3) == 16969680          # the 25-bit workload's range
    assert leech.index_count(3) <= (1 << 25)
    assert leech.max_shell_for_bits(44) == 10
    assert leech.index_count(10) == 13503934538640
    assert leech.index_count(10) <= (1 << 44) < leech.cumulative_counts(11)[11]


def test_class_table_shape():
    T = classes.class_table(10)
    assert len(T) == 168
    assert T[0].start == 0
    for a, b in zip(T, T[1:]):
        assert a.end == b.start
    assert T[-1].end == leech.index_count(10)
    # every class's I' = floor(I_class / A) fits in 32 bits (the GPU relies on it)
    assert max(c.size // c.A for c in T) < (1 << 32)
    # at most four distinct values in any multiset that gets unranked
    for c in T:
        assert len(set(c.complement_values)) <= 4
        assert len(set(c.support_values)) <= 4


def test_class_leaders_are_lattice_points():
    # the leader with the right signs and a codeword of matching weight is in the lattice
    T = golay.table()
    off = golay.weight_offset()
    for c in classes.class_table(10):
        x = unrank(c.start, 10)
        assert leech.in_leech(x)
        assert sorted((abs(v) for v in x), reverse=True) == list(c.leader)
        assert leech.norm2(x) == 16 * c.m
        if c.parity == 0 and c.w:
            assert golay.popcount(T[off[c.w]]) == c.w


def test_membership_rejects_perturbations():
    rnd = random.Random(11)
    M = 10
    for _ in range(300):
        I = rnd.randrange(leech.index_count(M))
        x = unrank(I, M)
        assert leech.in_leech(x)
        y = list(x)
        i = rnd.randrange(24)
        y[i] += rnd.choice([1, 2, 4, -1, -2, -4])
        # changing one coordinate by 1 breaks parity, by 2 or 4 breaks the residue/sum rule
        assert not leech.in_leech(y)


def test_lattice_closed_under_addition():
    rnd = random.Random(5)
    M = 10
    for _ in range(300):
        a = unrank(rnd.randrange(leech.index_count(M)), M)
        b = unrank(rnd.randrange(leech.index_count(M)), M)
        assert leech.in_leech([p + q for p, q in zip(a, b)])
        assert leech.in_leech([p - q for p, q in zip(a, b)])
        # integral lattice scaled by 8: inner products are multiples of 8
        assert sum(p * q for p, q in zip(a, b)) % 8 == 0
