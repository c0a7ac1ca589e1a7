"""Spherical GPTQ on the GPU: the quantiser with Hessian error feedback (papernotes.org
notes, 关键设计 3 and 整体框架).

For each 24-column block S in order, every row's block gets its angular nearest point of
shells 2..M from llvq_search (the HIP search kernel); the block is replaced by its
retraction onto the sphere of its own norm, w_hat = |w| v / |v|, and the residual
E = w - w_hat is spread over the later columns F through U = chol(H^-1)^T:
W[:, F] -= (E U_SS^-1) U_SF (the optimal correction for fixing the block).  The gain
index of each block is the table entry nearest to the norm it had when it was quantised;
the fields go to the packed stream through llvq_pack_fields.  The 'euclid' variant feeds
back the gain-quantised reconstruction G[g] v / |v| instead, 'direct' feeds back nothing.

The search and the packing run in the library's kernels; the per-block feedback is a
triangular solve and a matrix product (torch.linalg / torch.matmul on the device, fp64).
"""

import ctypes

from . import SEARCH_ANGULAR, load_library, make_desc, packed_bytes, MODE_SHAPEGAIN, _check


def inverse_hessian_factor(H, damp=0.01):
    """Upper triangular U (fp64, on H's device) with (H + damp mean(diag H) I)^-1 = U^T U."""
    import torch
    H = H.to(torch.float64)
    Hd = H + damp * torch.mean(torch.diagonal(H)) * torch.eye(H.shape[0], dtype=H.dtype, device=H.device)
    Hinv = torch.cholesky_inverse(torch.linalg.cholesky(Hd))
    return torch.linalg.cholesky(Hinv).mT    # Hinv = L L^T, U = L^T


def gptq(W, H, max_shell, gains, shape_bits=44, damp=0.01, variant="spherical", stream=None):
    """Quantise W [N][K] (torch fp32/fp64 on the GPU) with Hessian H [K][K].  When K is not a
    multiple of 24 the last block is zero-padded (the pad columns get an uncoupled unit
    Hessian, so they stay zero).  gains: fp16 gain table (torch, 2^gain_bits entries).
    Returns (descriptor, packed uint8 stream, shape indices int64 [N][Kb], gain indices
    int64 [N][Kb])."""
    import torch
    if variant not in ("spherical", "euclid", "direct"):
        raise ValueError(variant)
    lib = load_library()
    dev = W.device
    N, K0 = W.shape
    kb = (K0 + 23) // 24
    K = 24 * kb
    if K != K0:
        Wp = torch.zeros((N, K), dtype=W.dtype, device=dev)
        Wp[:, :K0] = W
        Hp = torch.eye(K, dtype=torch.float64, device=dev) * torch.mean(torch.diagonal(H.to(torch.float64)))
        Hp[:K0, :K0] = H
        W, H = Wp, Hp
    gain_bits = int(gains.numel()).bit_length() - 1
    if (1 << gain_bits) != gains.numel():
        raise ValueError("the gain table needs 2^gain_bits entries")
    U = inverse_hessian_factor(H.to(dev), damp)
    G = gains.to(torch.float64)
    Wq = W.to(torch.float64).clone()
    idx = torch.empty((N, kb), dtype=torch.int64, device=dev)
    gidx = torch.empty((N, kb), dtype=torch.int64, device=dev)
    pts = torch.empty((N, 24), dtype=torch.int8, device=dev)
    ind = torch.empty(N, dtype=torch.int64, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    sptr = ctypes.c_void_p(stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream)
    for b in range(kb):
        s0, s1 = 24 * b, 24 * b + 24
        blk = Wq[:, s0:s1]
        xs = blk.to(torch.float32).contiguous()
        _check(lib.llvq_search(ctypes.c_void_p(xs.data_ptr()), N, max_shell, SEARCH_ANGULAR,
                               ctypes.c_void_p(pts.data_ptr()), ctypes.c_void_p(ind.data_ptr()),
                               ctypes.c_void_p(err.data_ptr()), sptr), "llvq_search")
        v = pts.to(torch.float64)
        vhat = v / torch.linalg.vector_norm(v, dim=1, keepdim=True)
        nrm = torch.linalg.vector_norm(blk, dim=1)
        gi = torch.argmin(torch.abs(G[None, :] - nrm[:, None]), dim=1)    # first minimum: ties to the lower
        idx[:, b] = ind
        gidx[:, b] = gi
        if variant != "direct" and s1 < K:
            what = (G[gi] if variant == "euclid" else nrm)[:, None] * vhat
            E = blk - what
            Ep = torch.linalg.solve_triangular(U[s0:s1, s0:s1], E, upper=True, left=False)   # E U_SS^-1
            Wq[:, s1:] -= Ep @ U[s0:s1, s1:]
    if int(err.item()) != 0:
        raise RuntimeError("search returned invalid points (non-finite weights?)")
    desc = make_desc(MODE_SHAPEGAIN, N, K0, max_shell, shape_bits, gain_bits)
    fields = idx | (gidx << shape_bits)
    packed = torch.empty(packed_bytes(desc), dtype=torch.uint8, device=dev)
    _check(lib.llvq_pack_fields(ctypes.byref(desc), ctypes.c_void_p(fields.data_ptr()),
                                ctypes.c_void_p(packed.data_ptr()), sptr), "llvq_pack_fields")
    return desc, packed, idx, gidx
