"""Pins for the oracle beyond shell 10 (other rates): shells up to 42, where a 68-bit shape
field plus a 4-bit gain is 3 bits per weight.

Shell sizes are reached by two independent routes (the theta-series closed form and the
class table's sums, the coordinate count for the first shells past 10); the bijection is
pinned by lattice membership, the shell norm and the inverse map on random indices,
including indices past 2^64."""

import random

import pytest

from oracle import classes, leech
from oracle.bijection import rank, unrank

M_WIDE = 42


@pytest.fixture(scope="module")
def table42():
    return classes.class_table(M_WIDE)


def test_class_sums_equal_closed_form_to_shell_42(table42):
    sizes = {}
    for c in table42:
        sizes[c.m] = sizes.get(c.m, 0) + c.size
    for m in range(2, M_WIDE + 1):
        assert sizes[m] == leech.shell_size_closed_form(m), m


@pytest.mark.parametrize("m", [12, 13])
def test_closed_form_equals_coordinate_dp_past_shell_11(m):
    assert leech.shell_size_dp(m) == leech.shell_size_closed_form(m)


def test_rates_and_index_widths():
    # 2 bits per weight with a 1- or 2-bit gain: 47 or 46 shape bits reach shells 12 and 11
    assert leech.max_shell_for_bits(46) == 11
    assert leech.max_shell_for_bits(47) == 12
    # 3 bits per weight: 72-bit fields, 68 shape bits + 4 gain bits reach shell 42
    assert leech.max_shell_for_bits(68) == 42
    assert (1 << 67) < leech.index_count(42) <= (1 << 68)
    assert leech.max_shell_for_bits(64) == 33           # past shell 33 the index needs > 64 bits
    assert leech.index_count(33) < (1 << 64) < leech.index_count(34)


def test_contiguous_intervals_and_fixed_width_bounds(table42):
    assert table42[0].start == 0
    for a, b in zip(table42, table42[1:]):
        assert a.end == b.start
    assert table42[-1].end == leech.index_count(42)
    # bounds the general GPU decoder is sized for
    assert max(c.size for c in table42) < (1 << 63)
    assert max(max(c.P_S, c.P_T) for c in table42) < (1 << 58)
    assert max(len(set(c.support_values)) for c in table42) <= 8
    assert max(len(set(c.complement_values)) for c in table42) <= 8
    assert max(c.leader[0] for c in table42) == 25


def test_bisection_equals_linear_scan():
    T = classes.class_table(16)
    rnd = random.Random(5)
    probes = [c.start for c in T] + [c.end - 1 for c in T]
    probes += [rnd.randrange(leech.index_count(16)) for _ in range(300)]
    for I in probes:
        assert classes.find_class(I, 16) is classes.find_class_linear(I, 16)
    with pytest.raises(ValueError):
        classes.find_class(leech.index_count(16), 16)


@pytest.mark.parametrize("M", [11, 12, 16, 24, 42])
def test_random_round_trip_membership_and_norm(M):
    from oracle.leech import in_leech, norm2
    rnd = random.Random(M)
    C = leech.index_count(M)
    T = classes.class_table(M)
    idx = [rnd.randrange(C) for _ in range(60)]
    idx += [T[-1].start, T[-1].end - 1, C - 1]              # the last class of shell M
    for I in idx:
        x = unrank(I, M)
        m = classes.find_class(I, M).m
        assert in_leech(x) and norm2(x) == 16 * m, I
        assert rank(x, M) == I
