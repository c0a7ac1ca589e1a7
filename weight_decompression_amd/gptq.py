"""Spherical GPTQ on the GPU: the quantiser with Hessian error feedback (papernotes.org
notes, 关键设计 3 and 整体框架).

For each 24-column block S in order, every row's block gets its angular nearest point of
shells 2..M from llvq_search; the block is replaced by its retraction onto the sphere of
its own norm, w_hat = |w| v / |v|, and the residual E = w - w_hat is spread over the later
columns F through U = chol(H^-1)^T: W[:, F] -= (E U_SS^-1) U_SF (the optimal correction for
fixing the block).  The gain index of each block is the table entry nearest to the norm it
had when it was quantised; the fields go to the packed stream through llvq_pack_fields.
The 'euclid' variant feeds back the gain-quantised reconstruction G[g] v / |v| instead,
'direct' feeds back nothing.

Every step runs in the library's kernels (llvq_gptq_factor for U, llvq_gptq_begin,
llvq_search and llvq_gptq_column per block column, llvq_pack_fields); this module only
allocates the device buffers and runs the loop.
"""

import ctypes

from . import (SEARCH_ANGULAR, MODE_SHAPEGAIN, _check, _packed_nbytes, _tensor, load_library, make_desc)

VARIANTS = {"spherical": 0, "euclid": 1, "direct": 2}


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def gptq(W, H, max_shell, gains, shape_bits=44, damp=0.01, variant="spherical", stream=None):
    """Quantise W [N][K] (fp32 on the GPU) with the layer Hessian H [K][K] (fp64 on the
    GPU).  When K is not a multiple of 24 the last block is zero-padded (the pad columns get
    an uncoupled Hessian diagonal, so they stay zero).  gains: fp16 gain table (2^gain_bits
    entries).  Returns (descriptor, packed uint8 stream, fields int64 [N][Kb] with
    shape index | gain index << shape_bits)."""
    import torch
    if variant not in VARIANTS:
        raise ValueError(variant)
    N, K = W.shape
    kb = (K + 23) // 24
    kp = 24 * kb
    gain_bits = int(gains.numel()).bit_length() - 1
    if (1 << gain_bits) != gains.numel():
        raise ValueError("the gain table needs 2^gain_bits entries")
    _tensor(W, "gptq: W", (torch.float32,), 4 * N * K)
    _tensor(H, "gptq: H", (torch.float64,), 8 * K * K)
    _tensor(gains, "gptq: gains", (torch.float16,), 2 * gains.numel())
    lib = load_library()
    dev = W.device
    sp = ctypes.c_void_p(stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    U = torch.empty((kp, kp), dtype=torch.float64, device=dev)
    ws = torch.empty(int(lib.llvq_gptq_workspace_bytes(K)), dtype=torch.uint8, device=dev)
    _check(lib.llvq_gptq_factor(K, _p(H), float(damp), _p(U), _p(ws), _p(err), sp), "llvq_gptq_factor")
    del ws
    Wq = torch.empty((N, kp), dtype=torch.float64, device=dev)
    xs = [torch.empty((N, 24), dtype=torch.float32, device=dev) for _ in range(2)]
    _check(lib.llvq_gptq_begin(N, K, _p(W), _p(Wq), _p(xs[0]), sp), "llvq_gptq_begin")
    desc = make_desc(MODE_SHAPEGAIN, N, K, max_shell, shape_bits, gain_bits)
    pts = torch.empty((N, 24), dtype=torch.int8, device=dev)
    ind = torch.empty(N, dtype=torch.int64, device=dev)
    fields = torch.empty((N, kb), dtype=torch.int64, device=dev)
    ework = torch.empty((N, 24), dtype=torch.float64, device=dev)
    v = VARIANTS[variant]
    for b in range(kb):
        x, x_next = xs[b & 1], xs[(b + 1) & 1]
        _check(lib.llvq_search(_p(x), N, max_shell, SEARCH_ANGULAR, _p(pts), _p(ind), _p(err), sp), "llvq_search")
        _check(lib.llvq_gptq_column(ctypes.byref(desc), b, v, _p(gains), _p(Wq), _p(U), _p(pts), _p(ind),
                                    _p(fields), _p(ework), None if b == kb - 1 else _p(x_next), sp),
               "llvq_gptq_column")
    packed = torch.empty(_packed_nbytes(desc), dtype=torch.uint8, device=dev)
    _check(lib.llvq_pack_fields(ctypes.byref(desc), _p(fields), _p(packed), sp), "llvq_pack_fields")
    if int(err.item()) != 0:
        raise RuntimeError("GPTQ: Hessian not positive definite after damping, or non-finite weights")
    return desc, packed, fields
