"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bar: decoded lattice points and bf16 weights bit-exact; GEMV outputs within 1e-4 of the
fp64 oracle, normalised by sum_k |W_hat[r,k] x[k]|; indices bit-exact in the rank
round trip.  Inputs are the seeded synthetic workloads of weight_decompression_amd/synth.py.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

import weight_decompression_amd as wd
from oracle import bijection, classes, golay, leech, reference
from weight_decompression_amd import synth

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
C3 = leech.index_count(3)
C10 = leech.index_count(10)


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    wd.load_library()
    torch.cuda.init()
    yield


def dev(t: synth.Tensor):
    packed = torch.from_numpy(t.packed).cuda()
    scales = torch.from_numpy(t.scales_f16.copy()).cuda()
    x = None
    if t.x_bits is not None:
        x = torch.from_numpy(t.x_bits.view(np.int16).copy()).cuda().view(torch.bfloat16)
    elif t.x_f32 is not None:
        x = torch.from_numpy(t.x_f32.copy()).cuda()
    desc = wd.make_desc(t.mode, t.rows, t.cols, t.max_shell, t.shape_bits, t.gain_bits)
    assert packed.numel() >= wd.packed_bytes(desc)
    return desc, packed, scales, x


def gpu_points(t):
    desc, packed, scales, _ = dev(t)
    out = torch.empty((t.rows, t.kb * 24), dtype=torch.int8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.decode(desc, packed, scales, wd.OUT_POINTS_I8, out, err)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(err.item())


def gpu_gemv(t, repeat=1):
    desc, packed, scales, x = dev(t)
    batch = x.shape[0]
    outs = []
    for _ in range(repeat):
        y = torch.full((batch, t.rows), float("nan"), dtype=torch.float32, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        wd.gemv(desc, packed, scales, x, y, err)
        torch.cuda.synchronize()
        outs.append((y.cpu().numpy(), int(err.item())))
    return outs


def oracle_gemv(t, rows):
    x = t.x_as_f64()
    return reference.gemv(t.packed.tobytes(), t.rows, t.cols, t.max_shell, t.mode, t.shape_bits, t.gain_bits,
                          t.scales_f16, t.scales_f16, x, rows)


def check_gemv(t, rows, label):
    (y, err), = gpu_gemv(t)
    assert err == 0
    assert np.all(np.isfinite(y)), label
    y_ref, mag = oracle_gemv(t, rows)
    got = y[:, rows].astype(np.float64)
    e = reference.normalized_errors(got, y_ref, mag)
    say(f"{label}: max normalised error {e.max():.3e} over {e.size} outputs")
    assert np.all(reference.gemv_within_tolerance(got, y_ref, mag)), (label, e.max())
    return y


def sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, n - 1), size=min(k, n - 2), replace=False)
    return sorted(set([0, n - 1] + [int(v) for v in mid]))


# ---------------------------------------------------------------------------
# decode -> int8 points

def test_decode_points_tiny_workload_full():
    t = synth.workload1(C3)
    say(f"decode points {t.name}")
    pts, err = gpu_points(t)
    assert err == 0
    for r in range(t.rows):
        ref = reference.decode_row_points(t.packed.tobytes(), t.rows, t.cols, 3, 25, 0, r)
        assert np.array_equal(pts[r].astype(np.int64), ref), r


def point_list_tensor(indices, max_shell=10, shape_bits=44, gain_bits=4):
    idx = np.asarray(indices, dtype=np.uint64).reshape(-1, 1)
    packed = synth.pack_fields(idx, shape_bits + gain_bits)
    return synth.Tensor("points", synth.MODE_SHAPEGAIN, idx.shape[0], 24, max_shell, shape_bits, gain_bits, idx,
                        np.zeros_like(idx), np.ones(1 << gain_bits, dtype=np.float16), packed)


def test_decode_points_every_class_boundary_and_shell():
    rng = np.random.default_rng(7)
    idx = []
    for c in classes.class_table(10):
        idx += [c.start, c.end - 1, c.start + int(rng.integers(0, c.size))]
    Cm = leech.cumulative_counts(10)
    for m in range(2, 11):
        idx += [int(v) for v in rng.integers(Cm[m - 1], Cm[m], size=300, dtype=np.uint64)]
    idx += [0, C10 - 1]
    say(f"decode points: {len(idx)} indices over all classes")
    t = point_list_tensor(idx)
    pts, err = gpu_points(t)
    assert err == 0
    for j, I in enumerate(idx):
        assert list(pts[j].astype(int)) == bijection.unrank(int(I), 10), I


def test_decode_points_uniform_sample_matches_oracle():
    t = synth.make_tensor("u", 11, 0, 64, 24 * 40, C10, batch=0)
    pts, err = gpu_points(t)
    assert err == 0
    for r in range(0, 64, 7):
        ref = reference.decode_row_points(t.packed.tobytes(), t.rows, t.cols, 10, 44, 4, r)
        assert np.array_equal(pts[r].astype(np.int64), ref), r


def test_out_of_range_index_gives_zero_block_and_counts():
    idx = [5, C10, C10 + 12345, (1 << 44) - 1, 7]
    t = point_list_tensor(idx)
    pts, err = gpu_points(t)
    assert err == 3
    assert list(pts[0]) == bijection.unrank(5, 10)
    assert not pts[1:4].any()
    assert list(pts[4]) == bijection.unrank(7, 10)


def _with_invalid_blocks(t, positions):
    """Copy of tensor t whose blocks at (row, block) positions hold shape indices past the
    shell union (they must decode to zero and be counted)."""
    import dataclasses
    shape = t.shape_idx.copy()
    for j, (r, b) in enumerate(positions):
        shape[r, b] = np.uint64(C10 + 1000 * j)
    packed = synth.pack_fields(shape | (t.gain_idx << np.uint64(t.shape_bits)), t.shape_bits + t.gain_bits)
    return dataclasses.replace(t, shape_idx=shape, packed=packed)


def test_decode_two_buffer_pipeline_with_invalid_blocks():
    # 2598 x 11008 (Kb = 459): a workgroup's rows do not fit one LDS tile, so the decode runs
    # 4-row tiles (3 per workgroup, the last tile 2 rows) with the next tile classified during
    # the decode of the current one; invalid blocks are spread over the tensor.
    t0 = synth.make_tensor("dpipe", 19, 1, 2598, 11008, C10, batch=0)
    rng = np.random.default_rng(19)
    pos = [(0, 0), (0, 458), (2597, 458), (2596, 3), (1300, 200)]
    pos += [(int(r), int(b)) for r, b in zip(rng.integers(0, 2598, 35), rng.integers(0, 459, 35))]
    pos = sorted(set(pos))
    t = _with_invalid_blocks(t0, pos)
    bad = {}
    for r, b in pos:
        bad.setdefault(r, set()).add(b)
    rows = sorted(set(sample_rows(t.rows, 10, 19)) | set(bad) | {2596, 2597})
    pts, err = gpu_points(t)
    assert err == len(pos)
    raw = t.packed.tobytes()
    for r in rows:
        ref = reference.decode_row_points(raw, t.rows, t.cols, 10, 44, 4, r) if r not in bad else None
        if ref is None:
            for b in range(t.kb):
                blk = pts[r, 24 * b:24 * b + 24]
                if b in bad[r]:
                    assert not blk.any(), (r, b)
                else:
                    assert list(blk.astype(int)) == bijection.unrank(int(t.shape_idx[r, b]), 10), (r, b)
        else:
            assert np.array_equal(pts[r].astype(np.int64), ref), r
    desc, packed, scales, _ = dev(t)
    out = torch.empty((t.rows, t.cols), dtype=torch.bfloat16, device="cuda")
    err_t = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.decode(desc, packed, scales, wd.OUT_BF16, out, err_t)
    torch.cuda.synchronize()
    assert int(err_t.item()) == len(pos)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    ok_rows = [r for r in rows if r not in bad]
    for r in ok_rows:
        ref = reference.decode_row_bf16(raw, t.rows, t.cols, 10, t.mode, 44, 4, t.scales_f16, None, r)
        assert np.array_equal(got[r], ref), r
    for r in bad:
        for b in bad[r]:
            assert not got[r, 24 * b:min(24 * b + 24, t.cols)].any(), (r, b)


# ---------------------------------------------------------------------------
# decode -> bf16

def test_decode_bf16_shapegain_bit_exact():
    t = synth.make_tensor("bf", 12, 0, 48, 4096, C10, batch=0)
    desc, packed, scales, _ = dev(t)
    out = torch.empty((t.rows, t.cols), dtype=torch.bfloat16, device="cuda")
    wd.decode(desc, packed, scales, wd.OUT_BF16, out)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for r in sample_rows(t.rows, 10, 1):
        ref = reference.decode_row_bf16(t.packed.tobytes(), t.rows, t.cols, 10, t.mode, 44, 4, t.scales_f16, None, r)
        assert np.array_equal(got[r], ref), r


def test_decode_bf16_euclid_ragged_bit_exact():
    t = synth.make_tensor("bfe", 13, 0, 37, 100, C3, mode=synth.MODE_EUCLID, max_shell=3, shape_bits=25,
                          gain_bits=0, batch=0)
    desc, packed, scales, _ = dev(t)
    out = torch.empty((t.rows, t.cols), dtype=torch.bfloat16, device="cuda")
    wd.decode(desc, packed, scales, wd.OUT_BF16, out)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for r in range(t.rows):
        ref = reference.decode_row_bf16(t.packed.tobytes(), t.rows, t.cols, 3, t.mode, 25, 0, None, t.scales_f16, r)
        assert np.array_equal(got[r], ref), r


# ---------------------------------------------------------------------------
# several tensors in one call

def _decode_one(t, kind):
    desc, packed, scales, _ = dev(t)
    shape = (t.rows, t.kb * 24) if kind == wd.OUT_POINTS_I8 else (t.rows, t.cols)
    out = torch.empty(shape, dtype=torch.int8 if kind == wd.OUT_POINTS_I8 else torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.decode(desc, packed, scales, kind, out, err)
    return out, err


def _check_many(ts, kind, oracle_rows=4):
    devs = [dev(t) for t in ts]
    outs = []
    for t in ts:
        shape = (t.rows, t.kb * 24) if kind == wd.OUT_POINTS_I8 else (t.rows, t.cols)
        dt = torch.int8 if kind == wd.OUT_POINTS_I8 else torch.bfloat16
        outs.append(torch.full(shape, 0x55 if kind == wd.OUT_POINTS_I8 else 7.0, dtype=dt, device="cuda"))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.decode_many([d for d, _, _, _ in devs], [p for _, p, _, _ in devs], [s for _, _, s, _ in devs], kind,
                   outs, err)
    torch.cuda.synchronize()
    err_sum = 0
    for j, t in enumerate(ts):
        one, e1 = _decode_one(t, kind)
        torch.cuda.synchronize()
        err_sum += int(e1.item())
        a = outs[j].view(torch.int8 if kind == wd.OUT_POINTS_I8 else torch.int16).cpu().numpy()
        b = one.view(torch.int8 if kind == wd.OUT_POINTS_I8 else torch.int16).cpu().numpy()
        assert np.array_equal(a, b), (j, t.rows, t.cols)
        raw = t.packed.tobytes()
        rows = sample_rows(t.rows, oracle_rows, 100 + j) if t.rows > 2 else range(t.rows)
        for r in [r for r in rows if np.all(t.shape_idx[r] < np.uint64(leech.index_count(t.max_shell)))]:
            if kind == wd.OUT_POINTS_I8:
                ref = reference.decode_row_points(raw, t.rows, t.cols, t.max_shell, t.shape_bits, t.gain_bits, r)
                assert np.array_equal(a[r].astype(np.int64), ref), (j, r)
            else:
                sg = t.mode == synth.MODE_SHAPEGAIN
                ref = reference.decode_row_bf16(raw, t.rows, t.cols, t.max_shell, t.mode, t.shape_bits, t.gain_bits,
                                                t.scales_f16 if sg else None, None if sg else t.scales_f16, r)
                assert np.array_equal(a[r].view(np.uint16), ref), (j, r)
    assert int(err.item()) == err_sum
    say(f"decode_many: {len(ts)} tensors, {sum(t.rows * t.kb for t in ts)} blocks, kind {kind}, errors {err_sum}")


@pytest.mark.parametrize("kind", [0, 1])
def test_decode_many_mixed_shapes_equal_single_decodes(kind):
    # shapes of one transformer layer cut down, ragged rows and columns, a one-block tensor
    # and invalid blocks (counted once, over all tensors, and decoded to zero)
    ts = [synth.make_tensor("m0", 31, 0, 48, 4096, C10, batch=0),
          synth.make_tensor("m1", 31, 1, 37, 11008, C10, batch=0),
          synth.make_tensor("m2", 31, 2, 100, 100, C10, batch=0),
          synth.make_tensor("m3", 31, 3, 1, 24, C10, batch=0),
          synth.make_tensor("m4", 31, 4, 700, 4096, C10, batch=0)]
    ts[1] = _with_invalid_blocks(ts[1], [(0, 0), (36, 458), (20, 100)])
    _check_many(ts, kind)


def test_decode_many_sixteen_tensors_and_euclid():
    rng = np.random.default_rng(32)
    ts = [synth.make_tensor(f"s{j}", 32, j, int(rng.integers(1, 90)), int(rng.integers(1, 3000)), C10, batch=0)
          for j in range(16)]
    _check_many(ts, wd.OUT_BF16, oracle_rows=2)
    C3_ = leech.index_count(3)
    te = [synth.make_tensor(f"e{j}", 33, j, r, c, C3_, mode=synth.MODE_EUCLID, max_shell=3, shape_bits=25,
                            gain_bits=0, batch=0) for j, (r, c) in enumerate([(37, 100), (64, 4096), (1, 24)])]
    _check_many(te, wd.OUT_BF16)
    _check_many(te, wd.OUT_POINTS_I8)


def test_decode_many_falls_back_for_rows_longer_than_a_tile():
    # 96000 columns (4000 blocks per row) do not fit a tile buffer: tensor-by-tensor decode
    ts = [synth.make_tensor("w0", 34, 0, 3, 96000, C10, batch=0),
          synth.make_tensor("w1", 34, 1, 40, 4096, C10, batch=0)]
    _check_many(ts, wd.OUT_BF16, oracle_rows=3)


# ---------------------------------------------------------------------------
# fused GEMV

def test_gemv_tiny_workload_all_rows():
    t = synth.workload1(C3)
    check_gemv(t, list(range(t.rows)), t.name)


def test_gemv_q_proj_4096x4096_sampled_and_deterministic():
    t = synth.workload2(C10)
    check_gemv(t, sample_rows(t.rows, 40, 2), t.name)
    (y1, _), (y2, _) = gpu_gemv(t, repeat=2)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_gemv_batch1_two_buffer_pipeline_ragged():
    # 3001 x 28800 (Kb = 1200): a workgroup's rows do not fit one LDS tile, so the batch-1
    # kernel runs several 2-row tiles per workgroup with the next tile classified during the
    # decode of the current one; the last tile holds one row.
    t = synth.make_tensor("pipe", 17, 1, 3001, 28800, C10)
    rows = sorted(set(sample_rows(t.rows, 20, 17)) | {2996, 2997, 2998, 2999, 3000})
    check_gemv(t, rows, "3001x28800 batch 1")
    (y1, _), (y2, _) = gpu_gemv(t, repeat=2)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_gemv_batch1_large_single_tile():
    # 24577 x 2048 (Kb = 86): each workgroup's 97 rows (8342 blocks, 33 classification
    # units for 16 waves) form one LDS tile; the last workgroup's tile has 36 rows.
    t = synth.make_tensor("seg", 18, 1, 24577, 2048, C10)
    rows = set(sample_rows(t.rows, 16, 18)) | {32, 33, 65, 66, 97 + 32, 97 + 65, 24576, 24575, 24541}
    check_gemv(t, sorted(rows), "24577x2048 batch 1")
    (y1, _), (y2, _) = gpu_gemv(t, repeat=2)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("rows,cols,xd", [(40, 24 * 850, "f32"), (9, 24 * 1600 + 5, "bf16")])
def test_gemv_batch1_rows_too_long_for_the_seven_value_tail(rows, cols, xd):
    # rows whose activations leave no LDS for the 7-value tail table (fp32 Kb = 850, bf16
    # Kb = 1601) run the batch-1 kernel with the 6-value tail
    t = synth.make_tensor("tail6", 19, rows + cols, rows, cols, C10, x_dtype=xd)
    check_gemv(t, list(range(rows)), f"tail-6 {rows}x{cols} x={xd}")


def _fidelity(which):
    path = os.path.join(HERE, "golden", f"fidelity_c3_{which}.npz")
    if not os.path.exists(path):
        return None
    z = np.load(path)
    return z["shape_idx"], z["gain_idx"].astype(np.uint64)


@pytest.mark.parametrize("which", [0, 1])
def test_gemv_mlp_shapes_with_fidelity_rows(which):
    fid = _fidelity(which)
    t = synth.workload3(C10, which, fid)
    rows = sample_rows(t.rows, 24, 3 + which)
    if fid is not None:
        rows = sorted(set(rows) | set(range(0, fid[0].shape[0], 4)))
    check_gemv(t, rows, t.name)


@pytest.mark.parametrize("batch", [1, 4, 8, 16])
def test_gemm_28672x8192_small_batch(batch):
    t = synth.workload4(C10, batch)
    check_gemv(t, sample_rows(t.rows, 12, 5 + batch), f"{t.name} batch {batch}")


@pytest.mark.parametrize("rows,cols,batch", [(37, 24 * 50 + 16, 7), (20, 24 * 3 + 8, 2), (53, 24 * 400, 16),
                                             (16, 24 * 171, 3), (33, 24 * 700 + 8, 11)])
def test_gemm_aligned_column_layouts(rows, cols, batch):
    # bf16 activations with 16-byte aligned rows (cols % 8 == 0) take the matrix-core path's
    # buffer-load form: last blocks of 8 or 16 columns, chunks narrower than one batch of
    # four columns per wave, several column chunks, ragged row groups
    t = synth.make_tensor("mf", 17, rows * 7 + cols, rows, cols, C10, batch=batch)
    check_gemv(t, list(range(rows)), f"mfma {rows}x{cols} b{batch}")


def test_gemm_unaligned_activations_match_aligned():
    # the same activations 2 bytes off a 16-byte boundary take the per-element loads
    t = synth.make_tensor("mfu", 18, 1, 45, 24 * 90 + 16, C10, batch=6)
    desc, packed, scales, x = dev(t)
    y_ref, mag = oracle_gemv(t, list(range(t.rows)))
    outs = []
    for off in (0, 1):
        buf = torch.zeros(x.numel() + 8, dtype=torch.bfloat16, device="cuda")
        buf[off:off + x.numel()] = x.reshape(-1)
        xv = buf[off:off + x.numel()].view(x.shape)
        y = torch.full((x.shape[0], t.rows), float("nan"), dtype=torch.float32, device="cuda")
        wd.gemv(desc, packed, scales, xv, y)
        torch.cuda.synchronize()
        got = y.cpu().numpy().astype(np.float64)
        assert np.all(reference.gemv_within_tolerance(got, y_ref, mag)), off
        outs.append(got)
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("rows,cols,batch,xd", [(1, 1, 1, "f32"), (3, 23, 2, "bf16"), (5, 25, 3, "f32"),
                                                (70, 100, 1, "bf16"), (2, 24 * 65 + 7, 16, "bf16"),
                                                (37, 1001, 5, "bf16"), (17, 24 * 300 + 1, 9, "bf16")])
def test_gemv_ragged_edges(rows, cols, batch, xd):
    t = synth.make_tensor("edge", 14, rows * 1000 + cols, rows, cols, C10, batch=batch, x_dtype=xd)
    check_gemv(t, list(range(rows)), f"edge {rows}x{cols} b{batch}")


def test_gemv_euclid_fp32_and_bf16_x():
    for xd in ("f32", "bf16"):
        t = synth.make_tensor("eu", 15, 1 if xd == "f32" else 2, 64, 240, C3, mode=synth.MODE_EUCLID, max_shell=3,
                              shape_bits=25, gain_bits=0, batch=2, x_dtype=xd)
        check_gemv(t, list(range(t.rows)), f"euclid x={xd}")


def test_gemv_other_max_shells():
    for M in (2, 5, 8):
        C = leech.index_count(M)
        bits = max(1, (C - 1).bit_length())
        for batch in (1, 3):
            t = synth.make_tensor(f"M{M}", 16, M, 33, 24 * 70 + 5, C, max_shell=M, shape_bits=bits, gain_bits=3,
                                  batch=batch)
            check_gemv(t, list(range(t.rows)), f"max_shell {M} ({bits}+3 bit fields) batch {batch}")


# ---------------------------------------------------------------------------
# rank (encode_ref) and the index round trip

def membership_torch(pts):
    """Vectorised lattice membership (independent of both implementations):
    parity, sum rule and the residue mask looked up in a 2^24 codeword bitmap."""
    x = pts.to(torch.int32)
    p = x[:, :1] & 1
    same = ((x & 1) == p).all(dim=1)
    sums = x.sum(dim=1)
    sum_ok = ((sums - 4 * p[:, 0]) % 8) == 0
    want = torch.where(p == 1, 1, 2)
    bits = (((x % 4) == want).to(torch.int64) << torch.arange(24, device=x.device)).sum(dim=1)
    bitmap = torch.zeros(1 << 24, dtype=torch.bool, device=x.device)
    bitmap[torch.tensor(golay.table(), dtype=torch.int64, device=x.device)] = True
    return same & sum_ok & bitmap[bits]


def test_round_trip_one_million_points():
    n = 1 << 20
    idx = synth.workload5_roundtrip_indices(C10, n, chunk=0)
    t = point_list_tensor(idx)
    desc, packed, scales, _ = dev(t)
    pts = torch.empty((n, 24), dtype=torch.int8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.decode(desc, packed, scales, wd.OUT_POINTS_I8, pts, err)
    back = torch.empty(n, dtype=torch.int64, device="cuda")
    wd.encode_ref(pts, 10, back, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    expect = torch.from_numpy(idx.view(np.int64)).cuda()
    assert torch.equal(back, expect)
    assert bool(membership_torch(pts).all())
    n2 = (pts.to(torch.int32) ** 2).sum(dim=1)
    assert bool(((n2 % 16) == 0).all()) and int(n2.min()) >= 32 and int(n2.max()) <= 160
    sample = np.random.default_rng(8).choice(n, 300, replace=False)
    host = pts.cpu().numpy()
    for j in sample:
        assert list(host[j].astype(int)) == bijection.unrank(int(idx[j]), 10)


def test_rank_matches_oracle_and_flags_bad_points():
    rng = np.random.default_rng(9)
    good = [bijection.unrank(int(I), 10) for I in rng.integers(0, C10, size=200, dtype=np.uint64)]
    bad = [[1] * 24, [0] * 24, [2] + [0] * 23, [4, 4] + [0] * 22 + [0], [12] * 24]
    bad[3] = [4, 4] + [0] * 22
    pts = np.array(good + bad, dtype=np.int8)
    expect = [bijection.rank(x, 10) for x in good]
    p = torch.from_numpy(pts).cuda()
    out = torch.empty(len(pts), dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.encode_ref(p, 10, out, err)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint64)
    assert [int(v) for v in got[:200]] == expect
    # [4,4,0..] is a lattice point of shell 2 (valid); the others are not points of shells 2..10
    assert int(got[200 + 3]) == bijection.rank(bad[3], 10)
    assert all(int(v) == (1 << 64) - 1 for i, v in enumerate(got[200:]) if i != 3)
    assert int(err.item()) == 4
    # a shell-10 point is out of range when only shells 2..9 are allowed
    out9 = torch.empty(1, dtype=torch.int64, device="cuda")
    x10 = torch.from_numpy(np.array([bijection.unrank(C10 - 1, 10)], dtype=np.int8)).cuda()
    wd.encode_ref(x10, 9, out9)
    torch.cuda.synchronize()
    assert int(out9.cpu().numpy().view(np.uint64)[0]) == (1 << 64) - 1


def test_rank_perturbed_points_and_unaligned_input():
    # valid points of every shell and small perturbations of them: the GPU rank must give
    # the oracle's index exactly when the oracle says the point is in shells 2..10, and
    # UINT64_MAX (counted) otherwise
    rng = np.random.default_rng(21)
    pts = []
    for I in rng.integers(0, C10, size=600, dtype=np.uint64):
        x = bijection.unrank(int(I), 10)
        pts.append(list(x))
        y = list(x)
        i, j = rng.choice(24, size=2, replace=False)
        d = int(rng.choice([-4, -2, 2, 4]))
        y[i] += d
        y[j] -= d
        pts.append(y)
        z = list(x)
        z[int(rng.integers(24))] *= -1
        pts.append(z)
    pts = [[max(-128, min(127, v)) for v in x] for x in pts]
    expect = []
    for x in pts:
        n2 = leech.norm2(x)
        ok = leech.in_leech(x) and n2 % 16 == 0 and 2 <= n2 // 16 <= 10
        expect.append(bijection.rank(x, 10) if ok else (1 << 64) - 1)
    nbad = sum(1 for e in expect if e == (1 << 64) - 1)
    assert 0 < nbad < len(pts)
    arr = np.array(pts, dtype=np.int8)
    for offset in (0, 1):
        buf = torch.zeros(arr.size + 8, dtype=torch.int8, device="cuda")
        view = buf[offset:offset + arr.size]
        view.copy_(torch.from_numpy(arr.ravel()).cuda())
        say(f"rank: {len(pts)} points, byte offset {offset}")
        out = torch.empty(len(pts), dtype=torch.int64, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        wd.load_library().llvq_encode_ref(ctypes.c_void_p(view.data_ptr()), len(pts), 10,
                                           ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(err.data_ptr()),
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        got = [int(v) for v in out.cpu().numpy().view(np.uint64)]
        assert got == expect
        assert int(err.item()) == nbad


@pytest.mark.parametrize("wide", [False, True])
def test_decode_into_unaligned_outputs_equals_aligned(wide):
    # bf16 rows 2-byte aligned only, int8 points 4-byte aligned only: the element-wise store
    # paths of the streamed decode (2-bit) and of the general decoder's tile decode give the
    # same bytes as the vector stores; cols 4000 is not a multiple of 24 (ragged last block)
    if wide:
        t = synth.make_wide_tensor("wunal", 91, 0, 61, 4000, leech.index_count(42), batch=0)
    else:
        t = synth.make_tensor("unal", 91, 0, 61, 4000, C10, batch=0)
    desc, packed, scales, _ = dev(t)
    n16 = t.rows * t.cols
    ref = torch.empty((t.rows, t.cols), dtype=torch.bfloat16, device="cuda")
    wd.decode(desc, packed, scales, wd.OUT_BF16, ref)
    buf = torch.zeros(n16 + 8, dtype=torch.bfloat16, device="cuda")
    view = buf[1:1 + n16].view(t.rows, t.cols)                   # 2-byte aligned
    wd.decode(desc, packed, scales, wd.OUT_BF16, view)
    n8 = t.rows * t.kb * 24
    pref = torch.empty((t.rows, t.kb * 24), dtype=torch.int8, device="cuda")
    wd.decode(desc, packed, scales, wd.OUT_POINTS_I8, pref)
    pbuf = torch.zeros(n8 + 16, dtype=torch.int8, device="cuda")
    pview = pbuf[4:4 + n8].view(t.rows, t.kb * 24)               # 4-byte aligned
    wd.decode(desc, packed, scales, wd.OUT_POINTS_I8, pview)
    torch.cuda.synchronize()
    assert torch.equal(view.view(torch.int16), ref.view(torch.int16))
    assert not buf[:1].view(torch.int16).any() and not buf[1 + n16:].view(torch.int16).any()
    assert torch.equal(pview, pref)
    assert not pbuf[:4].any() and not pbuf[4 + n8:].any()
    raw = t.packed.tobytes()
    M = t.max_shell
    for r in (0, t.rows - 1):
        got = view[r].view(torch.int16).cpu().numpy().view(np.uint16)
        want = reference.decode_row_bf16(raw, t.rows, t.cols, M, t.mode, t.shape_bits, t.gain_bits, t.scales_f16,
                                         None, r)
        assert np.array_equal(got, want), r
    say(f"decode into unaligned outputs ({'general decoder' if wide else '2-bit'}): equal to aligned")
