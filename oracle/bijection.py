"""Index <-> lattice point bijection (oracle).

The inverse map on the pages (papernotes.org page, 关键设计 2): with I_class the index
inside its class,
    r  = I_class mod A       (Golay codeword choice)
    I' = floor(I_class / A)
    s  = I' mod 2^B          (sign pattern obeying the congruence rule)
    I''= floor(I' / 2^B)     (rank in the lexicographic order of the permutations)
The gist.science page (Methodik / 3. Indexierungsschema, 4. Dequantisierungskernel)
describes the same walk: shell -> class -> local symmetries, undone with integer
division and modulo.

Readings taken (the pages leave these open):
* codeword: c = T[offset(w) + r] for even classes, c = T[r] for odd classes (T sorted
  by weight then mask, see golay.py);
* permutation rank: lexicographic rank among the distinct arrangements of the
  multiset, values in ascending order, position 0 most significant.  For even classes
  the support values and the complement values are ranked separately,
  I'' = rank_S * P_T + rank_T; the support values fill the codeword's positions in
  ascending position order, the complement values the other positions likewise;
* signs, odd classes: x_i > 0 iff (|x_i| = 1 mod 4) == (i in c), i.e. the positions
  = 1 mod 4 are exactly the codeword;
* signs, even classes: the free positions are, in this order, the codeword's positions
  in ascending order without q = its highest position, then the nonzero positions off
  the codeword in ascending order (the order in which the two parts are unranked); bit
  j of s (LSB first) is the sign of the j-th free position, 1 meaning negative; x_q
  takes the sign that makes the number of negative support entries = pi mod 2 (this is
  the sum = 0 mod 8 rule).
"""

from . import golay
from .classes import class_table, find_class, multinomial

DIM = 24


# ---------------------------------------------------------------------------
# lexicographic rank of multiset arrangements

def multiset_unrank(rank: int, values) -> list:
    """The arrangement of the multiset `values` with the given lexicographic rank
    (values compared in ascending order, position 0 most significant)."""
    distinct = sorted(set(values))
    cnt = {v: 0 for v in distinct}
    for v in values:
        cnt[v] += 1
    n = len(values)
    total = multinomial(cnt.values())
    if not 0 <= rank < total:
        raise ValueError("permutation rank out of range")
    out = []
    remaining = total  # number of arrangements of what is left
    for pos in range(len(values)):
        for v in distinct:
            if cnt[v] == 0:
                continue
            # arrangements of the rest that start with v
            starting_with_v = remaining * cnt[v] // n
            if rank < starting_with_v:
                out.append(v)
                cnt[v] -= 1
                remaining = starting_with_v
                break
            rank -= starting_with_v
        n -= 1
    return out


def multiset_rank(seq) -> int:
    """Inverse of multiset_unrank."""
    cnt = {}
    for v in seq:
        cnt[v] = cnt.get(v, 0) + 1
    n = len(seq)
    remaining = multinomial(cnt.values())
    rank = 0
    for v_here in seq:
        for v in sorted(cnt):
            if cnt[v] == 0:
                continue
            starting_with_v = remaining * cnt[v] // n
            if v == v_here:
                cnt[v] -= 1
                remaining = starting_with_v
                break
            rank += starting_with_v
        n -= 1
    return rank


# ---------------------------------------------------------------------------
# unrank: global shape index -> lattice point

def bits_of(mask: int) -> list:
    return [i for i in range(DIM) if (mask >> i) & 1]


def unrank(I: int, M: int) -> list:
    """Lattice point (integer coordinates, x.x = 16 m) of global shape index I in the
    shell union 2..M."""
    cl = find_class(I, M)
    J = I - cl.start
    r = J % cl.A
    Ip = J // cl.A
    s = Ip % (1 << cl.B)
    R = Ip >> cl.B
    T = golay.table()

    if cl.parity == 1:
        c = T[r]
        absx = multiset_unrank(R, cl.complement_values)
        x = []
        for i, a in enumerate(absx):
            in_c = bool((c >> i) & 1)
            x.append(a if ((a % 4 == 1) == in_c) else -a)
        return x

    c = T[golay.weight_offset()[cl.w] + r]
    support = bits_of(c)
    complement = [i for i in range(DIM) if not (c >> i) & 1]
    rank_S, rank_T = divmod(R, cl.P_T)
    absx = [0] * DIM
    for pos, a in zip(support, multiset_unrank(rank_S, cl.support_values)):
        absx[pos] = a
    for pos, a in zip(complement, multiset_unrank(rank_T, cl.complement_values)):
        absx[pos] = a

    q = support[-1] if cl.w > 0 else None
    free = [i for i in support if i != q] + [i for i in complement if absx[i] != 0]
    negative = set(free[j] for j in range(len(free)) if (s >> j) & 1)
    if q is not None:
        neg_on_support = sum(1 for i in support if i in negative)
        if neg_on_support % 2 != cl.pi:
            negative.add(q)
    return [-a if i in negative else a for i, a in enumerate(absx)]


# ---------------------------------------------------------------------------
# rank: lattice point -> global shape index

def rank(x, M: int) -> int:
    """Inverse of unrank.  Raises ValueError for a non-lattice point or a point outside
    shells 2..M."""
    from .leech import in_leech, norm2  # local import keeps module order simple

    x = [int(v) for v in x]
    if len(x) != DIM or not in_leech(x):
        raise ValueError("not a Leech lattice point")
    n2 = norm2(x)
    m = n2 // 16
    if n2 % 16 or not 2 <= m <= M:
        raise ValueError("point outside the shell union")
    p = x[0] & 1
    leader = tuple(sorted((abs(v) for v in x), reverse=True))
    cl = None
    for c in class_table(M):
        if c.m == m and c.parity == p and c.leader == leader:
            cl = c
            break
    if cl is None:
        raise ValueError("no class for this point")
    absx = [abs(v) for v in x]
    T_pos = golay.position_of()

    if p == 1:
        c = 0
        for i, v in enumerate(x):
            if v % 4 == 1:
                c |= 1 << i
        r = T_pos[c]
        s = 0
        R = multiset_rank(absx)
    else:
        c = 0
        for i, v in enumerate(x):
            if v % 4 == 2:
                c |= 1 << i
        r = T_pos[c] - golay.weight_offset()[cl.w]
        support = bits_of(c)
        complement = [i for i in range(DIM) if not (c >> i) & 1]
        rank_S = multiset_rank([absx[i] for i in support])
        rank_T = multiset_rank([absx[i] for i in complement])
        R = rank_S * cl.P_T + rank_T
        q = support[-1] if cl.w > 0 else None
        free = [i for i in support if i != q] + [i for i in complement if absx[i] != 0]
        s = 0
        for j, i in enumerate(free):
            if x[i] < 0:
                s |= 1 << j
    return cl.start + r + cl.A * (s + (R << cl.B))
