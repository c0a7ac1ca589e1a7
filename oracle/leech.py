"""Leech lattice in integer coordinates (oracle).

The pages construct the Leech lattice from the extended Golay code and split it into
an even and an odd coset, using an integer embedding (papernotes.org page, 关键设计 2;
gist.science page, Methodik / 1. Struktur des Leech-Gitters).  Shells are the sets
of points of equal squared norm 2m in the standard scaling, and the codebook is the
union of shells m = 2..M (papernotes.org page, 关键设计 1).

Reading taken (the pages give no coordinates): integer coordinates are sqrt(8) times
the standard ones.  Then x in Z^24 is a lattice point iff for some p in {0, 1}

* every x_i is congruent to p mod 2,
* sum(x) is congruent to 4p mod 8,
* the set {i : x_i = 2 mod 4} (p = 0), or {i : x_i = 1 mod 4} (p = 1), is a Golay
  codeword.

Every "mod" here is the non-negative residue.  Shell m (standard norm 2m) is the set
x.x = 16 m.

Shell sizes are computed two independent ways:

* closed form: the Leech theta series is E_12 - (65520/691) Delta, so the number of
  vectors of standard norm 2m is (65520/691) (sigma_11(m) - tau(m)) with tau the
  Ramanujan tau function (textbook modular-forms fact, not from the pages);
* a coordinate dynamic programme that uses only the Golay weight enumerator and the
  residue rules above.
"""

from functools import lru_cache

from . import golay

DIM = 24


def norm2(x) -> int:
    return sum(int(v) * int(v) for v in x)


def in_leech(x) -> bool:
    """Membership test, straight from the residue definition above."""
    x = [int(v) for v in x]
    if len(x) != DIM:
        return False
    p = x[0] & 1
    if any((v & 1) != p for v in x):
        return False
    if (sum(x) - 4 * p) % 8 != 0:
        return False
    want = 2 if p == 0 else 1
    mask = 0
    for i, v in enumerate(x):
        if v % 4 == want:
            mask |= 1 << i
    return golay.is_codeword(mask)


def shell_of(x) -> int:
    """m with x.x = 16 m (x must be a lattice point)."""
    n = norm2(x)
    assert n % 16 == 0
    return n // 16


# ---------------------------------------------------------------------------
# closed form

def sigma(k: int, m: int) -> int:
    return sum(d ** k for d in range(1, m + 1) if m % d == 0)


@lru_cache(maxsize=None)
def tau_table(n_max: int) -> tuple:
    """Ramanujan tau(1..n_max) from Delta = q * prod_{n>=1} (1 - q^n)^24."""
    coef = [0] * (n_max + 1)
    coef[0] = 1
    for n in range(1, n_max + 1):
        for _ in range(24):
            # multiply the truncated series by (1 - q^n)
            for e in range(n_max, n - 1, -1):
                coef[e] -= coef[e - n]
    # Delta = q * prod -> tau(m) = coef[m - 1]
    return tuple([0] + [coef[m - 1] for m in range(1, n_max + 1)])


def shell_size_closed_form(m: int) -> int:
    t = tau_table(max(m, 1))[m]
    num = 65520 * (sigma(11, m) - t)
    assert num % 691 == 0
    return num // 691


# ---------------------------------------------------------------------------
# coordinate dynamic programme

def _count_coordinate_patterns(target: int, allowed_in, allowed_out, w: int, sum_res: int) -> int:
    """Number of integer vectors (x_0..x_23) with x_0..x_{w-1} drawn from allowed_in,
    x_w..x_23 from allowed_out, x.x = target and sum(x) = sum_res mod 8."""
    # state: (partial norm, partial sum mod 8) -> count
    state = {(0, 0): 1}
    for pos in range(DIM):
        allowed = allowed_in if pos < w else allowed_out
        nxt = {}
        for (nrm, sm), cnt in state.items():
            for v in allowed:
                n2 = nrm + v * v
                if n2 > target:
                    continue
                key = (n2, (sm + v) % 8)
                nxt[key] = nxt.get(key, 0) + cnt
        state = nxt
    return state.get((target, sum_res), 0)


def shell_size_dp(m: int) -> int:
    """Shell size by counting coordinate vectors per Golay weight (independent of the
    class table and of the closed form)."""
    target = 16 * m
    vmax = 1
    while (vmax + 1) ** 2 <= target:
        vmax += 1
    ints = range(-vmax, vmax + 1)
    res2 = [v for v in ints if v % 4 == 2]
    res0 = [v for v in ints if v % 4 == 0]
    res1 = [v for v in ints if v % 4 == 1]
    res3 = [v for v in ints if v % 4 == 3]
    total = 0
    for w, a_w in golay.weight_count().items():
        # even coset: codeword positions = 2 mod 4, others = 0 mod 4, sum = 0 mod 8
        total += a_w * _count_coordinate_patterns(target, res2, res0, w, 0)
        # odd coset: codeword positions = 1 mod 4, others = 3 mod 4, sum = 4 mod 8
        total += a_w * _count_coordinate_patterns(target, res1, res3, w, 4)
    return total


@lru_cache(maxsize=None)
def cumulative_counts(m_max: int) -> tuple:
    """(C_1, C_2, ..., C_{m_max}) with C_1 = 0 and C_m = C_{m-1} + |Shell(m)|.
    Returned as a tuple indexed by m (entries 0 and 1 are 0)."""
    out = [0, 0]
    for m in range(2, m_max + 1):
        out.append(out[-1] + shell_size_closed_form(m))
    return tuple(out)


def max_shell_for_bits(bits: int) -> int:
    """Largest M with C_M <= 2^bits (the shell union an index field of that width
    can address in full)."""
    m = 2
    while cumulative_counts(m + 1)[m + 1] <= (1 << bits):
        m += 1
    return m


def index_count(M: int) -> int:
    """C_M = |Lambda24(M)|, the number of valid shape indices for shells 2..M."""
    return cumulative_counts(M)[M]
