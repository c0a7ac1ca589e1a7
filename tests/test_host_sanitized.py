"""Sanitizer builds of the native code on the CPU (no GPU):

* the general decoder's device functions (llvq_wide.h, included unchanged by
  tests/host_build/wide_host.cpp) built for the host with AddressSanitizer and
  UndefinedBehaviorSanitizer: every table read is bounds-checked (including the odd-part
  inverse table indexed by n >> (ctz(n) + 1)) and every shift, conversion and overflow of
  the exact 64- and 128-bit arithmetic is checked, while the decoded points and the ranks
  are compared with the oracle (papernotes.org page, 关键设计 2: shell -> class ->
  codeword / signs / permutation rank and its div/mod inverse).  The indices include the
  two at which an LDS copy of the inverse table once gave wrong quotients on the GPU.
* the build-time table generator (128-bit class starts, bucket tables, generated code)
  under the same sanitizers: it must run clean and write exactly the files of the normal
  build.
* the whole library source (csrc/llvq.hip) with its host side under the same sanitizers,
  driven by tests/host_build/abi_host.cpp through the C ABI with arguments that every entry
  point must refuse before any launch (bad descriptors, null and misaligned pointers, sizes
  out of range, the no-allocation quantiser's size limit), plus the pure host queries.
  Device code is compiled at -O0 here: nothing of it runs.
"""

import os
import random
import shutil
import subprocess

import pytest

from oracle import classes, leech
from oracle.bijection import rank, unrank
from weight_decompression_amd import build_lib

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


@pytest.fixture(scope="module")
def tables():
    build_lib.build_tables(verbose=False)
    return build_lib.BUILD_DIR


@pytest.fixture(scope="module")
def wide_host(tables, tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("wide") / "wide_host")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", *SAN, "-I", build_lib.INCLUDE, "-I", build_lib.CSRC,
                    "-I", tables, "-o", exe, os.path.join(HERE, "host_build", "wide_host.cpp")], check=True)
    return exe


def _run(exe, lines):
    p = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, env=ENV)
    assert p.returncode == 0, p.stderr[-3000:]
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr, p.stderr[-3000:]
    out = p.stdout.splitlines()
    assert len(out) == len(lines)
    return out


def _decode(exe, M, idx):
    out = _run(exe, [f"D {M} {I & (2**64 - 1)} {I >> 64}" for I in idx])
    res = []
    for line in out:
        f = [int(t) for t in line.split()]
        res.append((f[0], f[1:]))
    return res


def _rank(exe, M, pts):
    out = _run(exe, [f"R {M} " + " ".join(str(a) for a in v) for v in pts])
    return [None if line == "none" else int(line.split()[0]) | (int(line.split()[1]) << 64) for line in out]


def _check(exe, M, idx):
    got = _decode(exe, M, idx)
    pts = []
    for I, (m, v) in zip(idx, got):
        assert v == unrank(I, M), (M, I)
        assert m == sum(a * a for a in v) // 16, (M, I)
        pts.append(v)
    if M <= 42:
        assert _rank(exe, M, pts) == list(idx)


def test_indices_of_the_lds_table_failure_decode_and_rank_exactly(wide_host):
    # the indices at which an LDS copy of the inverse table gave wrong quotients on the GPU
    _check(wide_host, 11, [21573226807194, 39000000000001])


@pytest.mark.parametrize("M", [11, 12])
def test_every_class_boundary(wide_host, M):
    idx = []
    for c in classes.class_table(M):
        if c.m > 10:
            idx += [c.start, c.end - 1]
    _check(wide_host, M, idx)


@pytest.mark.parametrize("M", [11, 16, 24, 33, 42])
def test_uniform_indices_and_sampled_boundaries(wide_host, M):
    rnd = random.Random(70 + M)
    C = leech.index_count(M)
    idx = [rnd.randrange(C) for _ in range(600)] + [0, C - 1]
    tab = classes.class_table(M)
    for c in rnd.sample(tab, min(300, len(tab))):
        idx += [c.start, c.end - 1]
    _check(wide_host, M, idx)


def test_rank_rejects_non_members(wide_host):
    rnd = random.Random(77)
    pts, want = [], []
    for _ in range(200):
        v = unrank(rnd.randrange(leech.index_count(16)), 16)
        i, j = rnd.sample(range(24), 2)
        u = list(v)
        u[i] += 2
        u[j] -= 2
        pts.append(u)
        n2 = sum(a * a for a in u)
        try:
            want.append(rank(u, 16) if n2 % 16 == 0 and 2 <= n2 // 16 <= 16 else None)
        except ValueError:
            want.append(None)
    got = _rank(wide_host, 16, pts)
    assert got == want
    assert sum(w is None for w in want) > 0


def test_c_abi_validation_is_clean_under_sanitizers(tables, tmp_path):
    try:
        hipcc = build_lib.hipcc_path()
    except RuntimeError:
        pytest.skip("needs hipcc")
    exe = str(tmp_path / "abi_host")
    host = [a for f in SAN for a in ("-Xarch_host", f)]
    subprocess.run([hipcc, f"--offload-arch={build_lib.OFFLOAD_ARCH}", "-O1", "-g", "-std=c++17",
                    "-Xarch_device", "-O0", *host,
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", build_lib.INCLUDE, "-I", build_lib.CSRC, "-I", tables, "-o", exe,
                    os.path.join(build_lib.CSRC, "llvq.hip"), os.path.join(HERE, "host_build", "abi_host.cpp")],
                   check=True, capture_output=True)
    p = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    assert p.returncode == 0, p.stdout[-1000:] + p.stderr[-3000:]
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr, p.stderr[-3000:]
    assert p.stdout.startswith("ok ") and int(p.stdout.split()[1]) >= 70


def test_table_generator_is_clean_under_sanitizers(tables, tmp_path):
    exe = str(tmp_path / "gen_san")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", *SAN, "-o", exe, os.path.join(build_lib.CSRC, "gen_tables.cpp")],
                   check=True)
    for flag, ref in (("--header", build_lib.TABLES_INC), ("--json", build_lib.TABLES_JSON),
                      ("--search", build_lib.SEARCH_INC), ("--wide", build_lib.WIDE_INC),
                      ("--wide-json", build_lib.WIDE_JSON)):
        out = str(tmp_path / os.path.basename(ref))
        p = subprocess.run([exe, flag, out], capture_output=True, text=True, env=ENV)
        assert p.returncode == 0, (flag, p.stderr[-3000:])
        assert "runtime error" not in p.stderr, (flag, p.stderr[-3000:])
        with open(out, "rb") as a, open(ref, "rb") as b:
            assert a.read() == b.read(), flag
