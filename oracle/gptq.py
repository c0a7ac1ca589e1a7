"""Spherical GPTQ: quantisation with Hessian error feedback on the product of spheres
(oracle only; test infrastructure).

papernotes.org notes, 关键设计 3 (and 整体框架): shape-gain quantisation is combined with
GPTQ's curvature compensation.  A block's candidate (the lattice direction) is rescaled to
the block's own norm, which is a retraction onto the product of spheres,
    w_hat = (|w| / |w_tilde|) w_tilde,
and the residual E = w - w_hat, now purely angular, is spread over the not yet quantised
weights through the Cholesky factor of the inverse Hessian, U = chol(H^-1)^T.  The gain
(the norm) is quantised by itself.

Steps, for a weight matrix W [N][K] (K a multiple of 24; see gptq() for padding) and a layer
Hessian H [K][K]:
  1. H_d = H + damp * mean(diag H) I;  U upper triangular with H_d^-1 = U^T U;
  2. for each 24-column block S in order (F = the columns after S):
       per row: v = the angular nearest point of shells 2..M to W[r, S] (oracle/search.py),
                w_hat = |W[r, S]| v / |v|   (the retraction; the Euclidean variant instead
                takes the gain-quantised reconstruction G[g] v / |v|),
                the row's norm is kept for the gain;
       E = W[:, S] - W_hat[:, S];  W[:, F] -= (E U_SS^-1) U_SF;
  3. gain index per block = the table entry nearest to the kept norm (ties to the lower).
The update in step 2 is the optimal (OBS) correction of the remaining weights for fixing
the block, -E [H_R^-1]_SS^-1 [H_R^-1]_SF with H_R the Hessian of the remaining columns,
written with the rows of U (tests check the two forms agree).  Rows do not interact.
"""

import numpy as np

from . import search


def inverse_hessian_factor(H, damp=0.01):
    """Upper triangular U with (H + damp mean(diag H) I)^-1 = U^T U."""
    H = np.asarray(H, dtype=np.float64)
    Hd = H + damp * np.mean(np.diag(H)) * np.eye(H.shape[0])
    L = np.linalg.cholesky(np.linalg.inv(Hd))     # inverse = L L^T
    return L.T


def obs_update(E, Hd, start, stop):
    """The optimal correction of the columns after [start, stop) for fixing that block with
    error E, from plain inverses of the remaining columns' Hessian (no Cholesky)."""
    R = slice(start, Hd.shape[0])
    Hinv_R = np.linalg.inv(Hd[R, R])
    n = stop - start
    return -E @ np.linalg.inv(Hinv_R[:n, :n]) @ Hinv_R[:n, n:]


def gptq(W, H, M, gains, damp=0.01, variant="spherical", rows=None):
    """Quantise W [N][K]: shape indices [N][Kb] (uint64) and gain indices [N][Kb].
    variant: 'spherical' (retraction), 'euclid' (gain-quantised feedback) or 'direct' (no
    feedback).  rows: optional subset of rows (rows do not interact).  When K is not a
    multiple of 24 the last block is zero-padded and the pad columns get an uncoupled unit
    Hessian (scaled to the mean diagonal), so they stay zero."""
    W = np.asarray(W, dtype=np.float64)
    H = np.asarray(H, dtype=np.float64)
    if rows is not None:
        W = W[list(rows)]
    N, K0 = W.shape
    kb = (K0 + 23) // 24
    K = 24 * kb
    if K != K0:
        Wp = np.zeros((N, K))
        Wp[:, :K0] = W
        Hp = np.eye(K) * np.mean(np.diag(H))
        Hp[:K0, :K0] = H
        W, H = Wp, Hp
    U = inverse_hessian_factor(H, damp)
    g = np.asarray(gains, dtype=np.float64)
    Wq = W.copy()
    idx = np.zeros((N, kb), dtype=np.uint64)
    gidx = np.zeros((N, kb), dtype=np.int64)
    for b in range(kb):
        s0, s1 = 24 * b, 24 * b + 24
        E = np.zeros((N, 24))
        for r in range(N):
            w = Wq[r, s0:s1]
            I, v = search.search(w, M, "angular")
            vhat = np.asarray(v, dtype=np.float64) / np.linalg.norm(v)
            nrm = float(np.linalg.norm(w))
            gi = search.nearest_gain(nrm, g)
            what = (g[gi] if variant == "euclid" else nrm) * vhat
            E[r] = w - what
            idx[r, b] = I
            gidx[r, b] = gi
        if variant != "direct" and s1 < K:
            Ep = np.linalg.solve(U[s0:s1, s0:s1].T, E.T).T      # E U_SS^-1
            Wq[:, s1:] -= Ep @ U[s0:s1, s1:]
    return idx, gidx


def reconstruct(idx, gidx, M, gains):
    """W_hat [N][K] = G[g] v / |v| per block."""
    from .bijection import unrank
    N, kb = idx.shape
    out = np.zeros((N, kb * 24))
    g = np.asarray(gains, dtype=np.float64)
    for r in range(N):
        for b in range(kb):
            v = np.asarray(unrank(int(idx[r, b]), M), dtype=np.float64)
            out[r, 24 * b:24 * b + 24] = g[gidx[r, b]] * v / np.linalg.norm(v)
    return out


def proxy_loss(W, W_hat, H):
    """Relative layer-output error tr(dW H dW^T) / tr(W H W^T)."""
    W = np.asarray(W, dtype=np.float64)
    D = W - W_hat
    return float(np.trace(D @ H @ D.T) / np.trace(W @ H @ W.T))
