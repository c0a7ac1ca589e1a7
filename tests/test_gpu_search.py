"""GPU parity of the nearest-point search (llvq_search) against the CPU oracle's exact
class x codeword search (oracle/search.py).

The search picks a maximum of a float objective, so the bar is: the GPU's index equals
the oracle's; where it does not, both candidates are optimal up to rounding (their
objectives, recomputed in fp64 from the two points, agree to 1e-6 relative), which can
only happen on a near-tie such as collinear points of different shells under the angular
objective.  Every GPU index must rank its GPU point (checked with the oracle's bijection)
and lie in shells 2..M.  Inputs: seeded Gaussian blocks, the fidelity rows of the
MLP-shaped workload (dense N(0, 0.02^2) weights, whose oracle search results are stored
under tests/golden/), and perturbed lattice points.
"""

import ctypes
import os
import random

import numpy as np
import pytest
import torch

import weight_decompression_amd as wd
from oracle import bijection, classes, leech, search
from weight_decompression_amd import synth

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
MODES = {"angular": wd.SEARCH_ANGULAR, "euclid": wd.SEARCH_EUCLID}


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    wd.load_library()
    torch.cuda.init()
    yield


def gpu_search(x, M, mode):
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    n = xt.shape[0]
    pts = torch.empty((n, 24), dtype=torch.int8, device="cuda")
    idx = torch.empty(n, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.search(xt, M, MODES[mode], pts, idx, err)
    torch.cuda.synchronize()
    return pts.cpu().numpy().astype(np.int64), idx.cpu().numpy().view(np.uint64), int(err.item())


def objective(x, v, mode):
    v = np.asarray(v, dtype=np.float64)
    s = float(np.dot(np.asarray(x, dtype=np.float64), v))
    m = float(np.dot(v, v)) / 16.0
    return s / (4.0 * np.sqrt(m)) if mode == "angular" else 2.0 * s - 16.0 * m


def check_against(x, want_idx, M, mode, label):
    """GPU search of blocks x against the oracle's indices want_idx."""
    pts, idx, err = gpu_search(x, M, mode)
    assert err == 0, label
    C = leech.index_count(M)
    assert np.all(idx < C), label
    diff = np.nonzero(idx != np.asarray(want_idx, dtype=np.uint64))[0]
    for i in diff:
        gv = bijection.unrank(int(idx[i]), M)
        ov = bijection.unrank(int(want_idx[i]), M)
        assert list(pts[i]) == gv, (label, i)
        og, oo = objective(x[i], gv, mode), objective(x[i], ov, mode)
        assert og >= oo - 1e-6 * (1.0 + abs(oo)), (label, i, og, oo)
    # the GPU point of a sample of agreeing blocks is the unranked index
    for i in range(0, len(x), max(1, len(x) // 16)):
        assert list(pts[i]) == bijection.unrank(int(idx[i]), M), (label, i)
    say(f"{label}: {len(x)} blocks, {len(diff)} near-tie differences from the oracle")
    assert len(diff) <= len(x) // 1000, label   # fp32 vs fp64 near-ties are rare
    return pts, idx


@pytest.mark.parametrize("mode,M,scale", [("angular", 10, 1.0), ("euclid", 10, 2.2), ("angular", 2, 1.0),
                                          ("euclid", 3, 1.6), ("angular", 6, 0.3), ("euclid", 5, 1.9)])
def test_search_matches_oracle_on_gaussian_blocks(mode, M, scale):
    rng = np.random.default_rng(100 + M + (mode == "euclid"))
    x = (rng.standard_normal((96, 24)) * scale).astype(np.float32)
    want = [search.search(x[i].astype(np.float64), M, mode)[0] for i in range(len(x))]
    check_against(x, want, M, mode, f"{mode} M={M}")


@pytest.mark.parametrize("which", [0, 1])
def test_search_reproduces_fidelity_fixture(which):
    # the stored oracle results of the MLP-shaped workload's first 64 rows (angular, M = 10)
    rows, cols = ((11008, 4096), (4096, 11008))[which]
    fx = np.load(os.path.join(HERE, "golden", f"fidelity_c3_{which}.npz"))
    want = fx["shape_idx"]
    nrows, kb = want.shape
    W = synth.fidelity_weights(3, which, nrows, cols)
    wpad = np.zeros((nrows, kb * 24), dtype=np.float32)
    wpad[:, :cols] = W
    x = wpad.reshape(-1, 24)
    check_against(x, want.reshape(-1), 10, "angular", f"fidelity rows {rows}x{cols}")


def test_search_recovers_perturbed_lattice_points():
    # Euclidean: a point plus noise well inside its Voronoi cell comes back exactly
    rng = np.random.default_rng(5)
    C = leech.index_count(10)
    I = rng.integers(0, C, size=200, dtype=np.uint64)
    v = np.array([bijection.unrank(int(i), 10) for i in I], dtype=np.float64)
    x = (v + rng.uniform(-0.4, 0.4, size=v.shape)).astype(np.float32)
    pts, idx, err = gpu_search(x, 10, "euclid")
    assert err == 0
    assert np.array_equal(idx, I.astype(np.uint64))
    assert np.array_equal(pts, v.astype(np.int64))


def test_search_many_blocks_grid_stride_and_edge_inputs():
    # more vectors than workgroups in the grid, plus a zero vector (every angular objective
    # ties at 0: any point is optimal) and a vector with a NaN coordinate
    rng = np.random.default_rng(9)
    n = 20000
    x = rng.standard_normal((n, 24)).astype(np.float32)
    x[7] = 0.0
    x[11, 3] = np.nan
    pts, idx, err = gpu_search(x, 10, "angular")
    assert err == 1
    assert idx[11] == np.uint64(2**64 - 1) and not pts[11].any()
    ok = np.ones(n, dtype=bool)
    ok[11] = False
    assert np.all(idx[ok] < leech.index_count(10))
    assert list(pts[7]) == bijection.unrank(int(idx[7]), 10)
    for i in rng.choice(np.nonzero(ok)[0], size=24, replace=False):
        if i == 7:
            continue
        I, _ = search.search(x[i].astype(np.float64), 10, "angular")
        if I != idx[i]:
            og = objective(x[i], bijection.unrank(int(idx[i]), 10), "angular")
            oo = objective(x[i], bijection.unrank(int(I), 10), "angular")
            assert og >= oo - 1e-6 * (1.0 + abs(oo)), i


def gpu_quantize(desc, w, scales):
    n_ws = wd.quantize_workspace_bytes(desc)
    wt = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).cuda()
    st = torch.from_numpy(np.ascontiguousarray(scales, dtype=np.float16)).cuda()
    packed = torch.full((wd.packed_bytes(desc),), 0xA5, dtype=torch.uint8, device="cuda")
    ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.quantize(desc, wt, st, packed, ws, err)
    torch.cuda.synchronize()
    return packed.cpu().numpy(), int(err.item())


def oracle_fields(w, scales, M, mode, gain_bits, shape_bits):
    rows, cols = w.shape
    kb = synth.blocks_per_row(cols)
    fields = np.zeros(rows * kb, dtype=np.uint64)
    for r in range(rows):
        wpad = np.zeros(kb * 24)
        wpad[:cols] = w[r]
        for b in range(kb):
            blk = wpad[b * 24:(b + 1) * 24]
            if mode == wd.MODE_SHAPEGAIN:
                I, _ = search.search(blk, M, "angular")
                g = search.nearest_gain(np.linalg.norm(blk), scales.astype(np.float64))
                fields[r * kb + b] = np.uint64(I) | (np.uint64(g) << np.uint64(shape_bits))
            else:
                I, _ = search.search(blk / float(scales[r]), M, "euclid")
                fields[r * kb + b] = np.uint64(I)
    return fields


def test_quantize_shapegain_stream_matches_oracle():
    # 13 x 226 N(0, 0.02^2) weights (10 blocks per row, the last of 10 columns), 44 + 4 bits
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((13, 226)) * 0.02).astype(np.float32)
    gains = synth.draw_gain_table(3, 0, 16, 0.02)
    desc = wd.make_desc(wd.MODE_SHAPEGAIN, 13, 226, 10, 44, 4)
    got, err = gpu_quantize(desc, w, gains)
    assert err == 0
    want = synth.pack_fields(oracle_fields(w, gains, 10, wd.MODE_SHAPEGAIN, 4, 44), 48)
    assert got.size == want.size and np.array_equal(got, want)


def test_quantize_euclid_stream_matches_oracle():
    # shells 2..3, 25-bit fields (not byte aligned), per-row fp16 scales
    rng = np.random.default_rng(22)
    rows, cols = 9, 24 * 7 + 3
    s = rng.uniform(0.5, 2.0, size=rows).astype(np.float16)
    w = (rng.standard_normal((rows, cols)) * 1.6 * s.astype(np.float32)[:, None]).astype(np.float32)
    desc = wd.make_desc(wd.MODE_EUCLID, rows, cols, 3, 25, 0)
    got, err = gpu_quantize(desc, w, s)
    assert err == 0
    want = synth.pack_fields(oracle_fields(w, s, 3, wd.MODE_EUCLID, 0, 25), 25)
    assert got.size == want.size and np.array_equal(got, want)


def test_quantize_then_decode_and_gemv():
    # the quantiser's stream decodes to its search points; a non-finite block is written
    # as an invalid field (zero block, counted by the decoder)
    rng = np.random.default_rng(23)
    rows, cols = 40, 24 * 20
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w[5, 30] = np.inf
    gains = synth.draw_gain_table(3, 1, 16, 0.02)
    desc = wd.make_desc(wd.MODE_SHAPEGAIN, rows, cols, 10, 44, 4)
    packed, err = gpu_quantize(desc, w, gains)
    assert err == 1
    pk = torch.from_numpy(packed).cuda()
    out = torch.empty((rows, cols), dtype=torch.int8, device="cuda")
    derr = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.decode(desc, pk, torch.from_numpy(gains).cuda(), wd.OUT_POINTS_I8, out, derr)
    torch.cuda.synchronize()
    assert int(derr.item()) == 1
    pts = out.cpu().numpy().reshape(rows, 20, 24).astype(np.int64)
    assert not pts[5, 1].any()
    xt = torch.from_numpy(w.reshape(-1, 24).copy())
    xt[5 * 20 + 1] = 0.0
    spts, _, _ = gpu_search(xt.numpy(), 10, "angular")
    sp = spts.reshape(rows, 20, 24)
    sp[5, 1] = 0
    assert np.array_equal(pts, sp)



@pytest.mark.parametrize("K", [72, 240, 1001])
def test_gptq_factor_matches_oracle(K):
    # U = chol(Hd^-1)^T from the library's blocked kernels (reversed Cholesky + triangular
    # inverse) against the oracle's plain inverse + Cholesky; K = 1001 pads to 1008
    from oracle import gptq as ogptq
    from weight_decompression_amd import gptq as ggptq  # noqa: F401  (binding loaded)
    rng = np.random.default_rng(K)
    X = rng.standard_normal((2 * K, K)) * np.exp(0.5 * rng.standard_normal(K))
    H = X.T @ X / (2 * K)
    kp = 24 * ((K + 23) // 24)
    Hp = np.eye(kp) * np.mean(np.diag(H))
    Hp[:K, :K] = H
    want = ogptq.inverse_hessian_factor(Hp, 0.01)
    lib = wd.load_library()
    Ht = torch.from_numpy(H).cuda()
    U = torch.full((kp, kp), float("nan"), dtype=torch.float64, device="cuda")
    ws = torch.empty(lib.llvq_gptq_workspace_bytes(K), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.llvq_gptq_factor(K, ctypes.c_void_p(Ht.data_ptr()), 0.01, ctypes.c_void_p(U.data_ptr()),
                                ctypes.c_void_p(ws.data_ptr()), ctypes.c_void_p(err.data_ptr()), sp) == 0
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = U.cpu().numpy()
    rel = np.abs(got - want).max() / np.abs(want).max()
    say(f"gptq factor K={K}: max |dU| / max |U| = {rel:.2e}")
    assert rel < 1e-10
    assert np.array_equal(got, np.triu(got))


def test_gptq_factor_reports_an_indefinite_hessian():
    # -I damped by 0.01 * mean(diag) stays negative definite: every pivot is counted; with
    # no counter the call still completes (the pivots are replaced, nothing is written)
    lib = wd.load_library()
    K = 48
    H = torch.from_numpy(-np.eye(K)).cuda()
    U = torch.empty((K, K), dtype=torch.float64, device="cuda")
    ws = torch.empty(lib.llvq_gptq_workspace_bytes(K), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.llvq_gptq_factor(K, ctypes.c_void_p(H.data_ptr()), 0.01, ctypes.c_void_p(U.data_ptr()),
                                ctypes.c_void_p(ws.data_ptr()), ctypes.c_void_p(err.data_ptr()), sp) == 0
    assert lib.llvq_gptq_factor(K, ctypes.c_void_p(H.data_ptr()), 0.01, ctypes.c_void_p(U.data_ptr()),
                                ctypes.c_void_p(ws.data_ptr()), None, sp) == 0
    torch.cuda.synchronize()
    assert int(err.item()) == K
    assert lib.llvq_gptq_factor(K, ctypes.c_void_p(H.data_ptr()), -1.0, ctypes.c_void_p(U.data_ptr()),
                                ctypes.c_void_p(ws.data_ptr()), None, sp) == -1


def _gptq_fields(W, H, gains, variant):
    from weight_decompression_amd import gptq as ggptq
    desc, packed, fields = ggptq.gptq(torch.from_numpy(W).cuda(), torch.from_numpy(H).cuda(), 10,
                                      torch.from_numpy(gains).cuda(), variant=variant)
    torch.cuda.synchronize()
    f = fields.cpu().numpy().view(np.uint64)
    return packed.cpu().numpy(), f & np.uint64((1 << 44) - 1), (f >> np.uint64(44)).astype(np.int64)


@pytest.mark.parametrize("variant", ["spherical", "euclid", "direct"])
def test_gptq_matches_oracle(variant):
    # spherical GPTQ on a seeded 12 x 240 layer (10 block columns) with a correlated Hessian
    from oracle import gptq as ogptq
    W, H = synth.gptq_problem(33, 12, 240, 1024)
    gains = (synth.chi_gain_table(16).astype(np.float64) * 0.02).astype(np.float16)
    want_idx, want_g = ogptq.gptq(W, H, 10, gains, variant=variant)
    packed, idx, gidx = _gptq_fields(W, H, gains, variant)
    assert np.array_equal(idx, want_idx)
    assert np.array_equal(gidx, want_g)
    fields = want_idx | (want_g.astype(np.uint64) << np.uint64(44))
    assert np.array_equal(packed, synth.pack_fields(fields.reshape(-1), 48))
    say(f"gptq {variant}: 120 blocks equal to the oracle")


def test_gptq_layer_spanning_every_workgroup_matches_oracle_rows():
    # 512 x 1000 (42 block columns, the last ragged): every kernel runs on many workgroups;
    # rows do not interact, so the oracle runs on a sample of them
    from oracle import gptq as ogptq
    W, H = synth.gptq_problem(35, 512, 1000, 2048)
    gains = (synth.chi_gain_table(16).astype(np.float64) * 0.02).astype(np.float16)
    _, idx, gidx = _gptq_fields(W, H, gains, "spherical")
    rows = [0, 1, 255, 256, 511]
    want_idx, want_g = ogptq.gptq(W, H, 10, gains, variant="spherical", rows=rows)
    assert np.array_equal(idx[rows], want_idx)
    assert np.array_equal(gidx[rows], want_g)
    say(f"gptq 512x1000: rows {rows} ({len(rows) * 42} blocks) equal to the oracle")


# ---------------------------------------------------------------------------
# shells past 10: the search up to shell 13 (2 bits per weight with 46..48 shape bits) and
# the general rank

@pytest.mark.parametrize("mode,M,scale", [("angular", 11, 1.0), ("angular", 12, 1.0), ("angular", 13, 0.7),
                                          ("euclid", 12, 2.4), ("euclid", 13, 2.5)])
def test_search_past_shell_10_matches_oracle(mode, M, scale):
    rng = np.random.default_rng(200 + M + (mode == "euclid"))
    x = (rng.standard_normal((64, 24)) * scale).astype(np.float32)
    want = [search.search(x[i].astype(np.float64), M, mode)[0] for i in range(len(x))]
    check_against(x, want, M, mode, f"{mode} M={M}")


def test_search_shell12_collinear_tie_goes_to_shell3():
    # u (shell 3) and 2u (shell 12) tie under the angular objective; u has the smaller index
    rng = np.random.default_rng(31)
    lo, hi = leech.index_count(2), leech.index_count(3)
    I = [int(i) for i in rng.integers(lo, hi, size=8)]
    u = np.array([bijection.unrank(i, 3) for i in I], dtype=np.float32)
    x = np.concatenate([u, 2.0 * u])
    for M in (12, 13):
        pts, idx, err = gpu_search(x, M, "angular")
        assert err == 0
        assert list(idx) == I + I, M


@pytest.mark.parametrize("M", [11, 13, 24, 33])
def test_rank_past_shell_10_matches_oracle(M):
    rng = random.Random(M)
    C = leech.index_count(M)
    T = classes.class_table(M)
    I = [rng.randrange(C) for _ in range(400)]
    for k in rng.sample(range(len(T)), min(len(T), 300)):
        I += [T[k].start, T[k].end - 1]
    pts = np.array([bijection.unrank(i, M) for i in I], dtype=np.int8)
    bad = pts[:6].copy()
    bad[0, 0] += 2          # one coordinate's residue mod 4 changes: not a codeword pattern
    bad[1, :] = 0           # the zero vector
    bad[2, 0] += 1          # mixed parity
    bad[3, :] = 2 * pts[3]  # shell 4m: beyond M, or a member the oracle ranks
    bad[4, [0, 5]] = bad[4, [5, 0]]   # two coordinates swapped: usually not a member
    bad[5, 7] = -bad[5, 7] if bad[5, 7] else bad[5, 7] + 4
    allp = np.concatenate([pts, bad])
    d = torch.from_numpy(allp.copy()).cuda()
    out = torch.empty(len(allp), dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.encode_ref(d, M, out, err)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint64)
    assert [int(g) for g in got[:len(I)]] == I
    nbad = 0
    for j, p in enumerate(bad):
        try:
            want = bijection.rank([int(a) for a in p], M)
        except ValueError:
            want = None
        g = int(got[len(I) + j])
        if want is None:
            assert g == 2**64 - 1, j
            nbad += 1
        else:
            assert g == want, j
    assert int(err.item()) == nbad and nbad >= 3
    say(f"general rank M={M}: {len(I)} points, {nbad} rejected")


@pytest.mark.parametrize("M,sb,gb", [(11, 46, 2), (12, 47, 1)])
def test_quantize_past_shell_10_stream_matches_oracle(M, sb, gb):
    # 2 bits per weight with the pages' split: 46 + 2 (shell 11) and 47 + 1 (shell 12)
    rng = np.random.default_rng(40 + M)
    w = rng.standard_normal((6, 100)).astype(np.float32)
    gains = synth.chi_gain_table(1 << gb)
    desc = wd.make_desc(wd.MODE_SHAPEGAIN, 6, 100, M, sb, gb)
    got, err = gpu_quantize(desc, w, gains)
    assert err == 0
    want = synth.pack_fields(oracle_fields(w, gains, M, wd.MODE_SHAPEGAIN, gb, sb), sb + gb)
    assert got.size == want.size and np.array_equal(got, want)
    # the stream decodes (general decoder) to the search points
    pk = torch.from_numpy(got).cuda()
    out = torch.empty((6, 5 * 24), dtype=torch.int8, device="cuda")
    wd.decode(desc, pk, torch.from_numpy(gains).cuda(), wd.OUT_POINTS_I8, out)
    torch.cuda.synchronize()
    fields = oracle_fields(w, gains, M, wd.MODE_SHAPEGAIN, gb, sb).reshape(6, 5)
    for r in (0, 5):
        for b in range(5):
            I = int(fields[r, b]) & ((1 << sb) - 1)
            assert list(out[r, 24 * b:24 * b + 24].cpu().numpy().astype(int)) == bijection.unrank(I, M)


def test_quantize_euclid_48bit_shell13_stream_matches_oracle():
    # Euclidean spherical shaping with all 48 bits on the shape (shells 2..13), row scales
    rng = np.random.default_rng(45)
    rows, cols = 5, 24 * 4 + 7
    s = rng.uniform(0.3, 0.45, size=rows).astype(np.float16)
    w = rng.standard_normal((rows, cols)).astype(np.float32)
    desc = wd.make_desc(wd.MODE_EUCLID, rows, cols, 13, 48, 0)
    got, err = gpu_quantize(desc, w, s)
    assert err == 0
    want = synth.pack_fields(oracle_fields(w, s, 13, wd.MODE_EUCLID, 0, 48), 48)
    assert got.size == want.size and np.array_equal(got, want)
