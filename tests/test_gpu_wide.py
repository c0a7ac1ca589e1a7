"""GPU parity of the general decoder (other rates: shells 2..42, fields up to 128 bits)
against the CPU oracle, through the C ABI.

Bar: lattice points and bf16 weights bit-exact; GEMV within 1e-4 of the fp64 oracle,
normalised by sum_k |W_hat[r,k] x[k]|; out-of-range indices decode to zero and are
counted.  Configurations: 46 + 2 and 47 + 1 bits at shells 11 and 12 (2 bits per weight),
68 + 4 bits at shell 42 (3 bits per weight; global indices past 2^64), a Euclidean tensor
at shell 16 and a descriptor at shell 10 with 61-bit shapes (the 2-bit shell range, too
wide for the 2-bit kernels)."""

import random

import numpy as np
import pytest
import torch

import weight_decompression_amd as wd
from oracle import bijection, classes, leech, parallel, reference
from weight_decompression_amd import synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    wd.load_library()
    torch.cuda.init()
    yield


def dev(t):
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


def points_of(t):
    desc, packed, scales, _ = dev(t)
    out = torch.full((t.rows, t.kb * 24), 0x55, dtype=torch.int8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.decode(desc, packed, scales, wd.OUT_POINTS_I8, out, err)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(err.item())


def index_list_tensor(indices, M, shape_bits, gain_bits):
    """One block per row holding the given shape indices (gain 0)."""
    n = len(indices)
    lo = np.array([I & (2**64 - 1) for I in indices], dtype=np.uint64)
    hi = np.array([I >> 64 for I in indices], dtype=np.uint64)
    packed = synth.pack_fields_wide(lo, hi, shape_bits + gain_bits)
    idx = np.array(indices, dtype=object).reshape(n, 1)
    return synth.Tensor("points", synth.MODE_SHAPEGAIN, n, 24, M, shape_bits, gain_bits, idx,
                        np.zeros((n, 1), dtype=np.uint64), np.ones(1 << gain_bits, dtype=np.float16), packed)


def check_indices(indices, M, shape_bits, gain_bits):
    t = index_list_tensor(indices, M, shape_bits, gain_bits)
    pts, err = points_of(t)
    C = leech.index_count(M)
    bad = sum(1 for I in indices if I >= C)
    assert err == bad
    for j, I in enumerate(indices):
        want = bijection.unrank(I, M) if I < C else [0] * 24
        assert list(pts[j].astype(int)) == want, (M, I)


@pytest.mark.parametrize("M,sb,gb", [(11, 46, 2), (12, 47, 1), (10, 61, 3)])
def test_every_class_boundary(M, sb, gb):
    rnd = random.Random(M)
    idx = []
    for c in classes.class_table(M):
        idx += [c.start, c.end - 1, c.start + rnd.randrange(c.size)]
    idx += [leech.index_count(M), (1 << sb) - 1]                    # out of range: zero, counted
    say(f"general decoder M={M} {sb}+{gb}: {len(idx)} indices")
    check_indices(idx, M, sb, gb)


def test_shell_42_indices_past_2_64():
    M = 42
    T = classes.class_table(M)
    rnd = random.Random(42)
    C = leech.index_count(M)
    idx = []
    for k in rnd.sample(range(len(T)), 1500):
        idx += [T[k].start, T[k].end - 1]
    for k in range(len(T) - 40, len(T)):                           # the last classes of shell 42
        idx += [T[k].start, T[k].end - 1]
    idx += [rnd.randrange(C) for _ in range(1500)]
    idx += [2**64 - 1, 2**64, 2**64 + 1, 2**67, C - 1, C, C + 12345, 2**68 - 1]
    say(f"general decoder M=42 68+4: {len(idx)} indices")
    check_indices(idx, M, 68, 4)


@pytest.mark.parametrize("M,sb,gb,rows,cols,mode", [
    (42, 68, 4, 37, 100, synth.MODE_SHAPEGAIN),
    (11, 46, 2, 20, 4096, synth.MODE_SHAPEGAIN),
    (16, 52, 0, 9, 300, synth.MODE_EUCLID),
])
def test_decode_bf16_bit_exact(M, sb, gb, rows, cols, mode):
    t = synth.make_wide_tensor("wb", 50 + M, 0, rows, cols, leech.index_count(M), mode=mode, max_shell=M,
                               shape_bits=sb, gain_bits=gb, batch=0)
    desc, packed, scales, _ = dev(t)
    out = torch.full((rows, cols), 3.0, dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.decode(desc, packed, scales, wd.OUT_BF16, out, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    raw = t.packed.tobytes()
    sg = mode == synth.MODE_SHAPEGAIN
    for r in sorted(set([0, rows - 1] + random.Random(M).sample(range(rows), min(rows, 6)))):
        ref = reference.decode_row_bf16(raw, rows, cols, M, mode, sb, gb, t.scales_f16 if sg else None,
                                        None if sg else t.scales_f16, r)
        assert np.array_equal(got[r], ref), (M, r)
    pts, err2 = points_of(t)
    assert err2 == 0
    for r in (0, rows - 1):
        assert np.array_equal(pts[r].astype(np.int64),
                              reference.decode_row_points(raw, rows, cols, M, sb, gb, r)), r


@pytest.mark.parametrize("M,sb,gb,rows,cols,batch,xd,mode", [
    (42, 68, 4, 300, 1000, 1, "bf16", synth.MODE_SHAPEGAIN),
    (42, 68, 4, 333, 1000, 1, "f32", synth.MODE_SHAPEGAIN),
    (24, 59, 0, 66, 777, 1, "bf16", synth.MODE_EUCLID),
    (11, 46, 2, 50, 2400, 1, "f32", synth.MODE_SHAPEGAIN),
    (42, 68, 4, 70, 4096, 5, "f32", synth.MODE_SHAPEGAIN),
    (12, 47, 1, 129, 2000, 16, "bf16", synth.MODE_SHAPEGAIN),
    (24, 59, 0, 66, 777, 2, "bf16", synth.MODE_EUCLID),
])
def test_gemv_matches_oracle(M, sb, gb, rows, cols, batch, xd, mode):
    t = synth.make_wide_tensor("wg", 60 + M, batch, rows, cols, leech.index_count(M), mode=mode, max_shell=M,
                               shape_bits=sb, gain_bits=gb, batch=batch, x_dtype=xd)
    desc, packed, scales, x = dev(t)
    outs = []
    for _ in range(2):
        y = torch.full((batch, rows), float("nan"), dtype=torch.float32, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        wd.gemv(desc, packed, scales, x, y, err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        outs.append(y.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])                         # repeatable bit for bit
    rows_s = sorted(set([0, rows - 1] + random.Random(rows).sample(range(rows), 5)))
    sg = mode == synth.MODE_SHAPEGAIN
    y_ref, mag = reference.gemv(t.packed.tobytes(), rows, cols, M, mode, sb, gb, t.scales_f16 if sg else None,
                                None if sg else t.scales_f16, t.x_as_f64(), rows_s)
    got = outs[0][:, rows_s].astype(np.float64)
    e = reference.normalized_errors(got, y_ref, mag)
    say(f"general GEMV M={M} {sb}+{gb} batch {batch}: max normalised error {e.max():.3e}")
    assert np.all(reference.gemv_within_tolerance(got, y_ref, mag))


def test_gemv_3bit_4096x11008_sampled_rows():
    # the 3-bit configuration at the headline shape: 4096 x 11008, 72-bit fields
    C = leech.index_count(42)
    t = synth.make_wide_tensor("w3", 70, 0, 4096, 11008, C)
    desc, packed, scales, x = dev(t)
    y = torch.full((1, 4096), float("nan"), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.gemv(desc, packed, scales, x, y, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    rows_s = [0, 1777, 4095]
    y_ref, mag = reference.gemv(t.packed.tobytes(), 4096, 11008, 42, t.mode, 68, 4, t.scales_f16, None,
                                t.x_as_f64(), rows_s)
    got = y.cpu().numpy()[:, rows_s].astype(np.float64)
    assert np.all(reference.gemv_within_tolerance(got, y_ref, mag))


def test_gemv_batch1_tiles_and_invalid_blocks():
    # 20000 x 4096 at shell 42: a workgroup's rows (79 x 171 blocks) exceed one LDS tile, so
    # the batch-1 coset-queue kernel walks several tiles; blocks with indices past the shell
    # union are spread over the tensor (zero contribution, counted)
    import dataclasses
    M, rows, cols = 42, 20000, 4096
    C = leech.index_count(M)
    t = synth.make_wide_tensor("wtile", 74, 0, rows, cols, C)
    bad = [(0, 0), (0, 170), (9999, 55), (19999, 170), (12345, 1)]
    shape = t.shape_idx.copy()
    for j, (r, b) in enumerate(bad):
        shape[r, b] = C + 1000 * j
    lo = np.array([[int(v) & (2**64 - 1) for v in row] for row in shape], dtype=np.uint64)
    hi = np.array([[int(v) >> 64 for v in row] for row in shape], dtype=np.uint64)
    hi |= t.gain_idx << np.uint64(68 - 64)
    t = dataclasses.replace(t, shape_idx=shape, packed=synth.pack_fields_wide(lo, hi, 72))
    desc, packed, scales, x = dev(t)
    outs = []
    for _ in range(2):
        y = torch.full((1, rows), float("nan"), dtype=torch.float32, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        wd.gemv(desc, packed, scales, x, y, err)
        torch.cuda.synchronize()
        assert int(err.item()) == len(bad)
        outs.append(y.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    # oracle rows without invalid blocks; rows with them against the oracle's sum over the rest
    rows_s = [1, 5000, 19998]
    y_ref, mag = reference.gemv(t.packed.tobytes(), rows, cols, M, t.mode, 68, 4, t.scales_f16, None,
                                t.x_as_f64(), rows_s)
    got = outs[0][:, rows_s].astype(np.float64)
    assert np.all(reference.gemv_within_tolerance(got, y_ref, mag))
    xf = t.x_as_f64()[0]
    for r in sorted({r for r, _ in bad}):
        ref, m = 0.0, 0.0
        for b in range(t.kb):
            if (r, b) in bad:
                continue
            I = int(shape[r, b])
            vals = reference.block_f32(I, int(t.gain_idx[r, b]), M, t.mode, t.scales_f16, None).astype(np.float64)
            xs = np.zeros(24)
            seg = xf[24 * b:min(24 * b + 24, cols)]
            xs[:seg.size] = seg
            ref += float(vals @ xs)
            m += float(np.abs(vals) @ np.abs(xs))
        say(f"row {r}: gpu {outs[0][0, r]:.6e} oracle {ref:.6e}")
        assert abs(outs[0][0, r] - ref) <= 1e-4 * m


def test_decode_many_with_wide_tensors_equals_single_calls():
    M = 42
    ts = [synth.make_wide_tensor(f"wm{j}", 80, j, r, c, leech.index_count(M), batch=0)
          for j, (r, c) in enumerate([(5, 100), (17, 24), (3, 500)])]
    devs = [dev(t) for t in ts]
    outs = [torch.zeros((t.rows, t.cols), dtype=torch.bfloat16, device="cuda") for t in ts]
    wd.decode_many([d for d, _, _, _ in devs], [p for _, p, _, _ in devs], [s for _, _, s, _ in devs], wd.OUT_BF16,
                   outs)
    torch.cuda.synchronize()
    for t, (d, p, s, _), o in zip(ts, devs, outs):
        one = torch.zeros_like(o)
        wd.decode(d, p, s, wd.OUT_BF16, one)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), one.view(torch.int16))


@pytest.mark.parametrize("xd", ["bf16", "f32"])
def test_gemv_unaligned_activations_equal_aligned(xd):
    # 16-byte activation loads (aligned x, aligned rows) and element loads give the same sums
    t = synth.make_wide_tensor("wu", 90, 0, 40, 480, leech.index_count(42), batch=3, x_dtype=xd)
    desc, packed, scales, x = dev(t)
    y0 = torch.empty((3, 40), dtype=torch.float32, device="cuda")
    wd.gemv(desc, packed, scales, x, y0)
    buf = torch.zeros(x.numel() + 8, dtype=x.dtype, device="cuda")
    xu = buf[1:1 + x.numel()].view(3, 480)
    xu.copy_(x)
    y1 = torch.empty_like(y0)
    wd.gemv(desc, packed, scales, xu, y1)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_rank_full_grid_of_repeated_points():
    # 2,000 points tiled to 262,144 (1,024 workgroups, several per CU): every copy ranks to
    # its index
    M = 24
    rng = random.Random(77)
    C = leech.index_count(M)
    I = [rng.randrange(C) for _ in range(2000)]
    base = np.array([bijection.unrank(i, M) for i in I], dtype=np.int8)
    reps = 262144 // len(I) + 1
    P = np.tile(base, (reps, 1))[:262144]
    want = np.tile(np.array(I, dtype=np.uint64), reps)[:262144]
    out = torch.empty(len(P), dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.encode_ref(torch.from_numpy(P).cuda(), M, out, err)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint64)
    assert int(err.item()) == 0
    assert np.array_equal(got, want), int((got != want).sum())


def test_decode_rank_round_trip_every_block_4096x11008():
    # shell 33, 64 + 4-bit fields: decode every block of a 4096 x 11008 tensor to points on
    # the GPU and rank them back; every block's index must return
    M = 33
    t = synth.make_wide_tensor("rt33", 71, 0, 4096, 11008, leech.index_count(M), max_shell=M, shape_bits=64,
                               gain_bits=4, batch=0)
    desc, packed, scales, _ = dev(t)
    pts = torch.empty((4096, t.kb * 24), dtype=torch.int8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.decode(desc, packed, scales, wd.OUT_POINTS_I8, pts, err)
    idx = torch.empty(4096 * t.kb, dtype=torch.int64, device="cuda")
    wd.encode_ref(pts.view(-1, 24), M, idx, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = idx.cpu().numpy().view(np.uint64)
    want = np.array(t.shape_idx.ravel(), dtype=np.uint64)
    assert np.array_equal(got, want), int((got != want).sum())
    raw = t.packed.tobytes()
    p = pts.cpu().numpy()
    for r in (0, 2222, 4095):
        assert np.array_equal(p[r].astype(np.int64), reference.decode_row_points(raw, 4096, 11008, M, 64, 4, r)), r


def test_gemv_3bit_4096x11008_seeded_rows_against_oracle():
    # the 3-bit GEMV against the oracle on 512 seeded rows plus the first and last (the
    # oracle's general decode costs 0.4-1.3 s per row of 459 blocks in one process, so
    # every row would take minutes even on the host's pool)
    C = leech.index_count(42)
    t = synth.make_wide_tensor("w3all", 72, 0, 4096, 11008, C)
    desc, packed, scales, x = dev(t)
    y = torch.full((1, 4096), float("nan"), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.gemv(desc, packed, scales, x, y, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    rng = np.random.default_rng(72)
    rows_s = sorted(set([0, 4095] + [int(r) for r in rng.choice(4096, 512, replace=False)]))
    say(f"3-bit GEMV: the oracle on {len(rows_s)} rows ({parallel.cores()} processes)")
    y_ref, mag = parallel.gemv_rows(t.packed.tobytes(), 4096, 11008, 42, t.mode, 68, 4, t.scales_f16, None,
                                    t.x_as_f64(), rows_s)
    got = y.cpu().numpy()[:, rows_s].astype(np.float64)
    e = reference.normalized_errors(got, y_ref, mag)
    say(f"3-bit GEMV: {e.size} outputs, max normalised error {e.max():.3e}")
    assert np.all(reference.gemv_within_tolerance(got, y_ref, mag))


def test_gemv_every_row_consistent_with_the_library_decode_3bit():
    # Not an oracle comparison: the library's own 3-bit GEMV of all 4,096 rows against an
    # fp64 product of the library's decoded points, which ties every row of the fused
    # kernel to the decode kernel (the decode is checked against the oracle above: the
    # round trip of every block and the oracle rows)
    C = leech.index_count(42)
    t = synth.make_wide_tensor("w3all", 72, 0, 4096, 11008, C)
    desc, packed, scales, x = dev(t)
    y = torch.empty((1, 4096), dtype=torch.float32, device="cuda")
    wd.gemv(desc, packed, scales, x, y)
    pts = torch.empty((4096, t.kb * 24), dtype=torch.int8, device="cuda")
    wd.decode(desc, packed, scales, wd.OUT_POINTS_I8, pts)
    torch.cuda.synchronize()
    # per-block scale G[g] / (4 sqrt m) in fp64 from the decoded point's norm
    v = pts.view(4096, t.kb, 24).double()
    m = (v * v).sum(-1) / 16.0
    g = torch.from_numpy(t.gain_idx.astype(np.int64)).cuda()
    G = torch.from_numpy(t.scales_f16.astype(np.float64)).cuda()[g]
    w = (v * (G / (4.0 * torch.sqrt(m)))[..., None]).reshape(4096, -1)[:, :11008]
    xf = x.double().reshape(-1)
    ref = w @ xf
    mag = (w.abs() @ xf.abs())
    ok = (y[0].double() - ref).abs() <= 1e-4 * mag
    assert bool(ok.all()), int((~ok).sum())


def test_round_trip_3bit_every_block_128bit_indices():
    # 3 bits per weight (shell 42, indices past 2^64): decode every block of a 2048 x 4096
    # tensor to points and rank them back to 128-bit indices
    M = 42
    t = synth.make_wide_tensor("rt42", 73, 0, 2048, 4096, leech.index_count(M), batch=0)
    desc, packed, scales, _ = dev(t)
    pts = torch.empty((2048, t.kb * 24), dtype=torch.int8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.decode(desc, packed, scales, wd.OUT_POINTS_I8, pts, err)
    idx = torch.empty((2048 * t.kb, 2), dtype=torch.int64, device="cuda")
    wd.encode_wide(pts.view(-1, 24), M, idx, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = idx.cpu().numpy().view(np.uint64)
    flat = t.shape_idx.ravel()
    want_lo = np.array([int(i) & (2**64 - 1) for i in flat], dtype=np.uint64)
    want_hi = np.array([int(i) >> 64 for i in flat], dtype=np.uint64)
    assert np.array_equal(got[:, 0], want_lo) and np.array_equal(got[:, 1], want_hi)
    assert (want_hi > 0).any()                                      # indices past 2^64 present


def test_encode_wide_matches_oracle_and_rejects():
    M = 42
    rnd = random.Random(421)
    C = leech.index_count(M)
    T = classes.class_table(M)
    I = [rnd.randrange(C) for _ in range(300)] + [T[k].start for k in rnd.sample(range(len(T)), 300)]
    P = np.array([bijection.unrank(i, M) for i in I], dtype=np.int8)
    bad = P[:3].copy()
    bad[0, 0] += 2
    bad[1, :] = 0
    bad[2, 0] += 1
    allp = np.concatenate([P, bad])
    out = torch.empty((len(allp), 2), dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd.encode_wide(torch.from_numpy(allp).cuda(), M, out, err)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint64)
    vals = [int(a) | (int(b) << 64) for a, b in got]
    assert vals[:len(I)] == I
    assert vals[len(I):] == [2**128 - 1] * 3 and int(err.item()) == 3
