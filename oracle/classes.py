"""Class table: shell -> class partition of the index space (oracle).

The index hierarchy on the pages (papernotes.org page, 关键设计 2; gist.science page,
Methodik / 3. Indexierungsschema): shells are laid out in ascending order by
cumulative offsets; inside a shell the points are grouped into classes, a class being
a leader (the multiset of coordinate absolute values) together with its even or odd
coset, and each class owns one contiguous index interval.  Inside a class the free
choices are a Golay codeword, a sign pattern obeying the congruence rule, and a
permutation of the leader.

Readings taken here (the pages do not spell these out):

Even classes (p = 0; all values even).  w = number of values = 2 mod 4 must be the
weight of a Golay codeword (0, 8, 12, 16 or 24); those values sit on the codeword's
support, the others (= 0 mod 4) on its complement.  If w = 0 the sum of the values
must also be 0 mod 8.
  A = number of codewords of weight w,
  B = (number of nonzero values) - 1 if w > 0, else the number of nonzero values,
  P = P_S * P_T with P_S the number of distinct arrangements of the support values on
      w slots and P_T that of the complement values on 24 - w slots,
  pi = (sum of values / 4) mod 2, the required parity of the number of negative
      signs on the support.
Odd classes (p = 1; all values odd).  Valid iff sum(floor(a/4)) + #{a = 3 mod 4} is
odd.  A = 4096, B = 0, P = number of distinct arrangements over 24 slots.

Class size = A * 2^B * P.  Order inside a shell: even classes first, then odd ones;
inside each parity, by the leader written as a non-increasing 24-tuple, ascending
lexicographically.  Class starts are cumulative in that order over shells 2..M.
"""

from dataclasses import dataclass
from functools import lru_cache
from math import factorial

from . import golay

DIM = 24


def multinomial(counts) -> int:
    n = sum(counts)
    out = factorial(n)
    for c in counts:
        out //= factorial(c)
    return out


def arrangements(values) -> int:
    """Number of distinct arrangements of a multiset."""
    cnt = {}
    for v in values:
        cnt[v] = cnt.get(v, 0) + 1
    return multinomial(cnt.values())


@dataclass(frozen=True)
class LeechClass:
    m: int                  # shell
    parity: int             # 0 even coset, 1 odd coset
    leader: tuple           # non-increasing 24-tuple of absolute values
    w: int                  # even: codeword weight; odd: 0 (unused)
    A: int
    B: int
    P_S: int                # even: support arrangements; odd: 1
    P_T: int                # even: complement arrangements; odd: full arrangements
    pi: int                 # even: required parity of negatives on the support
    start: int              # first global index of the class
    support_values: tuple   # even: ascending multiset on the codeword support
    complement_values: tuple  # even: ascending multiset on the complement; odd: all 24

    @property
    def P(self) -> int:
        return self.P_S * self.P_T

    @property
    def size(self) -> int:
        return self.A * (1 << self.B) * self.P

    @property
    def end(self) -> int:
        return self.start + self.size


def _leaders(target: int, parity: int):
    """All non-increasing 24-tuples of non-negative integers of the given parity whose
    squares sum to target."""
    vmax = 0
    while (vmax + 1) ** 2 <= target:
        vmax += 1
    values = [v for v in range(vmax, -1, -1) if v % 2 == parity]
    out = []

    def rec(idx, remaining_slots, remaining_norm, acc):
        if remaining_slots == 0:
            if remaining_norm == 0:
                out.append(tuple(acc))
            return
        if idx == len(values):
            return
        v = values[idx]
        # try every multiplicity of v, largest first
        max_k = remaining_slots if v == 0 else min(remaining_slots, remaining_norm // (v * v))
        for k in range(max_k, -1, -1):
            rec(idx + 1, remaining_slots - k, remaining_norm - k * v * v, acc + [v] * k)

    rec(0, DIM, target, [])
    return out


def _even_class_fields(leader):
    sup = sorted(a for a in leader if a % 4 == 2)
    comp = sorted(a for a in leader if a % 4 == 0)
    w = len(sup)
    if w not in golay.weight_count():
        return None
    if w == 0 and sum(leader) % 8 != 0:
        return None
    nnz = sum(1 for a in leader if a != 0)
    A = golay.weight_count()[w]
    B = nnz - 1 if w > 0 else nnz
    pi = (sum(leader) // 4) % 2
    return dict(w=w, A=A, B=B, P_S=arrangements(sup), P_T=arrangements(comp), pi=pi,
                support_values=tuple(sup), complement_values=tuple(comp))


def _odd_class_fields(leader):
    q = sum(a // 4 for a in leader) + sum(1 for a in leader if a % 4 == 3)
    if q % 2 != 1:
        return None
    return dict(w=0, A=4096, B=0, P_S=1, P_T=arrangements(leader), pi=0,
                support_values=(), complement_values=tuple(sorted(leader)))


@lru_cache(maxsize=None)
def class_table(M: int) -> tuple:
    """All classes of shells 2..M in index order, with their global starts."""
    out = []
    start = 0
    for m in range(2, M + 1):
        target = 16 * m
        for parity in (0, 1):
            leaders = sorted(_leaders(target, parity))
            for leader in leaders:
                f = _even_class_fields(leader) if parity == 0 else _odd_class_fields(leader)
                if f is None:
                    continue
                c = LeechClass(m=m, parity=parity, leader=leader, start=start, **f)
                out.append(c)
                start = c.end
    return tuple(out)


def class_sizes_by_shell(M: int) -> dict:
    sizes = {}
    for c in class_table(M):
        sizes[c.m] = sizes.get(c.m, 0) + c.size
    return sizes


@lru_cache(maxsize=None)
def _starts(M: int) -> tuple:
    return tuple(c.start for c in class_table(M))


def find_class(I: int, M: int) -> LeechClass:
    """The class whose interval holds global index I: the last class starting at or
    before I (the intervals are contiguous and ascending), checked to contain I."""
    import bisect
    table = class_table(M)
    k = bisect.bisect_right(_starts(M), I) - 1
    if k < 0 or not table[k].start <= I < table[k].end:
        raise ValueError(f"shape index {I} outside the shell union 2..{M}")
    return table[k]


def find_class_linear(I: int, M: int) -> LeechClass:
    """The same by a plain scan of every interval (a pin for find_class)."""
    for c in class_table(M):
        if c.start <= I < c.end:
            return c
    raise ValueError(f"shape index {I} outside the shell union 2..{M}")
