"""Pins for the oracle's Golay code: properties the extended binary Golay code must have
whatever generator is used (size 4096 per the papernotes.org page, 关键设计 2; the
weight enumerator 1/759/2576/759/1; linearity; self-duality; minimum distance 8)."""

import itertools
import random

from oracle import golay


def test_size_and_weight_distribution():
    T = golay.table()
    assert len(T) == 4096
    assert len(set(T)) == 4096
    assert golay.weight_count() == {0: 1, 8: 759, 12: 2576, 16: 759, 24: 1}
    assert all(0 <= c < (1 << 24) for c in T)


def test_sorted_by_weight_then_mask_with_offsets():
    T = golay.table()
    keys = [(golay.popcount(c), c) for c in T]
    assert keys == sorted(keys)
    assert golay.weight_offset() == {0: 0, 8: 1, 12: 760, 16: 3336, 24: 4095}


def test_linear_closed_under_xor():
    S = set(golay.table())
    rnd = random.Random(7)
    T = golay.table()
    for _ in range(20000):
        a, b = rnd.choice(T), rnd.choice(T)
        assert (a ^ b) in S


def test_minimum_distance_8():
    # linear code: minimum distance = minimum nonzero weight
    assert min(golay.popcount(c) for c in golay.table() if c) == 8


def test_self_dual_even_overlaps():
    # G24 is self-dual: any two codewords meet in an even number of positions
    T = golay.table()
    basis = [T[i] for i in range(1, 4096, 331)]
    for a, b in itertools.product(basis, T[::17]):
        assert golay.popcount(a & b) % 2 == 0


def test_punctured_code_is_cyclic():
    # the first 23 coordinates form a cyclic code: rotating them keeps a codeword
    S = set(golay.table())
    full = (1 << 23) - 1
    for c in golay.table()[::7]:
        c23 = c & full
        rot = ((c23 << 1) | (c23 >> 22)) & full
        parity = golay.popcount(rot) & 1
        assert (rot | (parity << 23)) in S


def test_every_weight8_word_is_an_octad_covering_5_sets():
    # Steiner system S(5,8,24): every 5-subset lies in exactly one octad
    octads = [c for c in golay.table() if golay.popcount(c) == 8]
    rnd = random.Random(3)
    for _ in range(200):
        five = rnd.sample(range(24), 5)
        m = sum(1 << i for i in five)
        assert sum(1 for o in octads if o & m == m) == 1
