"""Exact nearest-point search over the shell union (oracle only).

The pages extend a single-shell Leech search to the union of shells 2..M and give two
objectives (papernotes.org page, 关键设计 1; gist.science page, Methodik / 2.
Multi-Shell Search):

* angular (shape-gain): maximise <x/|x|, v/|v|> over v in Lambda24(M);
* Euclidean (spherical shaping / clipping): minimise |x - v|^2 over the same set.

This module is the plain exhaustive version: every class of shells 2..M is paired with
every Golay codeword it can use, and inside one (class, codeword) pair the best sign
pattern and permutation follow in closed form:

* odd class, codeword c: v_i = b(a) for i in c and -b(a) otherwise, where
  b(a) = a if a = 1 mod 4 else -a.  With y_i = x_i (i in c) or -x_i (i not in c),
  <x, v> = sum_i y_i b(a_i), maximised by pairing sorted y with sorted b
  (rearrangement inequality);
* even class, codeword c: sorted |x| on the support paired with the sorted support
  values, likewise on the complement, signs following x.  If the number of negative
  support entries has the wrong parity (pi), the best fix flips the entry with the
  smallest |x_i| on the support, costing 2 * min|x_i| * min(support value).

Both objectives reduce to max <x, v> inside one class because the norm is constant on
a class.  Exact ties between candidates are broken towards the smaller global index.
The angular objective does not see the scale of v, so a point k u (k >= 2) whose
fraction u is a lattice point ties exactly with u; the fp64 objectives of the two are
computed along different paths and need not come out equal, so that tie is resolved
explicitly: the winner is replaced by the smallest lattice point on its ray, whose index
is smallest (indices ascend with the shell).  k u lies in shell k^2 m, so up to shell 13
this concerns 2u in shell 8 (u in shell 2) and in shell 12 (u in shell 3).  The tests
pin this against literal enumeration of whole shells.
"""

import numpy as np

from . import golay
from .bijection import rank
from .classes import class_table
from .leech import in_leech

DIM = 24


def _codeword_matrix(words):
    """0/1 matrix [len(words)][24] of codeword bits."""
    arr = np.array(words, dtype=np.int64)
    return ((arr[:, None] >> np.arange(DIM)[None, :]) & 1).astype(bool)


class _Prepared:
    def __init__(self, M):
        self.M = M
        self.classes = class_table(M)
        T = golay.table()
        self.all_masks = _codeword_matrix(T)  # [4096][24]
        off = golay.weight_offset()
        cnt = golay.weight_count()
        self.by_weight = {}
        for w in cnt:
            words = T[off[w]:off[w] + cnt[w]]
            bits = _codeword_matrix(words)
            sup_idx = np.array([np.nonzero(b)[0] for b in bits], dtype=np.int64).reshape(len(words), w)
            comp_idx = np.array([np.nonzero(~b)[0] for b in bits], dtype=np.int64).reshape(len(words), DIM - w)
            self.by_weight[w] = (words, sup_idx, comp_idx)


_PREP = {}


def _prep(M):
    if M not in _PREP:
        _PREP[M] = _Prepared(M)
    return _PREP[M]


def _odd_point(x, cl, c):
    in_c = np.array([(c >> i) & 1 for i in range(DIM)], dtype=bool)
    y = np.where(in_c, x, -x)
    b = np.array([a if a % 4 == 1 else -a for a in cl.complement_values], dtype=np.int64)
    order_y = np.argsort(y, kind="stable")
    b_sorted = np.sort(b, kind="stable")
    signed_b = np.empty(DIM, dtype=np.int64)
    signed_b[order_y] = b_sorted
    return [int(v) if in_c[i] else -int(v) for i, v in enumerate(signed_b)]


def _even_point(x, cl, c):
    sup = [i for i in range(DIM) if (c >> i) & 1]
    comp = [i for i in range(DIM) if not (c >> i) & 1]
    v = [0] * DIM
    for idx, vals in ((sup, cl.support_values), (comp, cl.complement_values)):
        if not idx:
            continue
        ax = np.abs(x[idx])
        order = np.argsort(ax, kind="stable")
        for rank_pos, j in enumerate(order):
            i = idx[j]
            a = vals[rank_pos]
            v[i] = -a if x[i] < 0 else a
    if cl.w > 0:
        neg = sum(1 for i in sup if v[i] < 0)
        if neg % 2 != cl.pi:
            ax = np.abs(x[sup])
            j = int(np.argsort(ax, kind="stable")[0])
            i = sup[j]
            v[i] = -v[i]
    return v


def codeword_scores(x, M):
    """For every class of shells 2..M: (class, position in T of its first usable codeword,
    array of the best <x, v> over the class's points that use each usable codeword, in
    table order).  Odd classes use all 4096 codewords, even classes the A codewords of
    weight w."""
    P = _prep(M)
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    # odd coset: one sorted y per codeword, shared by all odd classes
    Y = np.where(P.all_masks, x[None, :], -x[None, :])
    Ys = np.sort(Y, axis=1)
    # even coset, per weight: sorted |x| on support / complement, negative counts
    even_pre = {}
    for w, (words, sup_idx, comp_idx) in P.by_weight.items():
        sup_abs = np.sort(ax[sup_idx], axis=1) if w else np.zeros((len(words), 0))
        comp_abs = np.sort(ax[comp_idx], axis=1) if w < DIM else np.zeros((len(words), 0))
        negs = (x[sup_idx] < 0).sum(axis=1) if w else np.zeros(len(words), dtype=np.int64)
        min_sup = sup_abs[:, 0] if w else np.zeros(len(words))
        even_pre[w] = (sup_abs, comp_abs, negs, min_sup)

    out = []
    for cl in P.classes:
        if cl.parity == 1:
            b = np.sort(np.array([a if a % 4 == 1 else -a for a in cl.complement_values], dtype=np.float64))
            scores = Ys @ b
            base = 0
        else:
            sup_abs, comp_abs, negs, min_sup = even_pre[cl.w]
            scores = np.zeros(sup_abs.shape[0])
            if cl.w:
                scores = scores + sup_abs @ np.array(cl.support_values, dtype=np.float64)
                wrong = (negs % 2) != cl.pi
                scores = scores - wrong * (2.0 * min_sup * min(cl.support_values))
            if cl.w < DIM:
                scores = scores + comp_abs @ np.array(cl.complement_values, dtype=np.float64)
            base = golay.weight_offset()[cl.w]
        out.append((cl, base, scores))
    return out


def class_scores(x, M):
    """For every class of shells 2..M: (best <x,v> in the class, list of codeword
    positions in T attaining it).  Exhaustive over codewords."""
    out = []
    for _cl, base, scores in codeword_scores(x, M):
        best = scores.max()
        winners = [int(base + j) for j in np.nonzero(scores == best)[0]]
        out.append((float(best), winners))
    return out


def search(x, M, mode="angular"):
    """Best point of Lambda24(M) for input block x (24 floats).

    mode 'angular': maximise <x, v> / |v|;  mode 'euclid': minimise |x - v|^2 with x in
    the lattice's integer-coordinate units.  Returns (global index, point)."""
    x = np.asarray(x, dtype=np.float64)
    T = golay.table()
    scored = []
    for cl, (best, winners) in zip(_prep(M).classes, class_scores(x, M)):
        if mode == "angular":
            obj = best / (4.0 * np.sqrt(cl.m))
        elif mode == "euclid":
            obj = 2.0 * best - 16.0 * cl.m
        else:
            raise ValueError(mode)
        scored.append((obj, cl, winners))
    top = max(s[0] for s in scored)
    candidates = []
    for obj, cl, winners in scored:
        if obj != top:
            continue
        for pos in winners:
            c = T[pos]
            v = _odd_point(x, cl, c) if cl.parity == 1 else _even_point(x, cl, c)
            candidates.append((rank(v, M), v))
    I, v = min(candidates, key=lambda t: t[0])
    if mode == "angular":
        u = smallest_on_ray(v)
        if u is not None:
            return rank(u, M), u
    return I, v


def smallest_on_ray(v):
    """The lattice point of smallest norm on the ray through v other than v itself: v / k
    for the largest k >= 2 with v / k in the lattice (norm >= 32, so in a shell >= 2), or
    None when there is none.  Such a point ties with v under the angular objective."""
    import math
    v = [int(a) for a in v]
    g = 0
    for a in v:
        g = math.gcd(g, abs(a))
    best = None
    for k in range(2, g + 1):
        if g % k:
            continue
        u = [a // k for a in v]
        if sum(a * a for a in u) >= 32 and in_leech(u):
            best = u
    return best


def nearest_gain(norm, gains):
    """Index of the gain table entry closest to `norm` (ties -> lower index)."""
    g = np.asarray(gains, dtype=np.float64)
    d = np.abs(g - norm)
    return int(np.nonzero(d == d.min())[0][0])
