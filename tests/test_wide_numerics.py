"""The general decoder finishes each multiset unranking in fp64 once fewer than 2^38
arrangements are left (arithmetic decoding: u = (rank + 1/2) / rem, u' = (u n - C_k) / c_k,
the batch-1 tile kernel multiplying by a rounded 1/c_k instead of dividing).  Its exactness
rests on an error bound, not on integer arithmetic, so this CPU test replays both forms of
the scheme in IEEE fp64 (numpy) on the classes with the most arrangements at shell 42 and on
ranks at the interval edges, against the oracle's integer unranking."""

import random

import numpy as np
import pytest

from oracle import bijection, classes

FP_REM = 1 << 38


def hybrid_unrank(rank, values, recip=False):
    """Exact integer steps while rem >= 2^38, then fp64 arithmetic decoding (recip: the
    step multiplies by fp64(1 / c_k) rather than dividing by c_k)."""
    distinct = sorted(set(values))
    cnt = [values.count(v) for v in distinct]
    n = len(values)
    rem = classes.multinomial(cnt)
    out = []
    fp = rem < FP_REM
    u = (np.float64(rank) + np.float64(0.5)) / np.float64(rem) if fp else None
    while n:
        if fp:
            y = u * np.float64(n)
            fy = int(y)
            run = np.cumsum(cnt)
            k = int(np.sum(run <= fy))
            below = int(run[k - 1]) if k else 0
            if recip:
                u = (y - np.float64(below)) * (np.float64(1.0) / np.float64(cnt[k]))
            else:
                u = (y - np.float64(below)) / np.float64(cnt[k])
        else:
            t = rank * n
            k, below = 0, 0
            while t >= below + rem * cnt[k]:
                below += rem * cnt[k]
                k += 1
            rank = (t - below) // n
            rem = rem * cnt[k] // n
            if rem < FP_REM:
                fp = True
                u = (np.float64(rank) + np.float64(0.5)) / np.float64(rem)
        out.append(distinct[k])
        cnt[k] -= 1
        n -= 1
    return out


@pytest.fixture(scope="module")
def big_parts():
    T = classes.class_table(42)
    parts = [c.complement_values for c in T] + [c.support_values for c in T if c.support_values]
    parts.sort(key=lambda vs: classes.arrangements(vs), reverse=True)
    return parts[:40]


@pytest.mark.parametrize("recip", [False, True])
def test_hybrid_unrank_equals_integer_unrank(big_parts, recip):
    rnd = random.Random(38)
    checked = 0
    for vs in big_parts:
        P = classes.arrangements(vs)
        ranks = [0, 1, P - 1, P - 2, P // 2, P // 3] + [rnd.randrange(P) for _ in range(60)]
        for R in ranks:
            assert hybrid_unrank(R, list(vs), recip) == bijection.multiset_unrank(R, vs), (vs, R)
            checked += 1
    assert checked > 2000
    assert classes.arrangements(big_parts[0]) > 2 ** 47        # the scheme starts exact here


@pytest.mark.parametrize("recip", [False, True])
def test_hybrid_unrank_at_every_rank_of_a_small_part(recip):
    # a part below the threshold from the start: every one of its ranks
    vs = (1, 1, 3, 3, 3, 5, 5, 7, 9, 9)
    P = classes.arrangements(vs)
    for R in range(P):
        assert hybrid_unrank(R, list(vs), recip) == bijection.multiset_unrank(R, vs)
