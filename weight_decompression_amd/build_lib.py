"""Build the LLVQ HIP library in-tree.

Steps:
  1. compile the host table generator (csrc/gen_tables.cpp) with g++;
  2. run it to write the table header (and a JSON dump of the same tables), the
     generated device code of the nearest-point search, and the class records of the
     general decoder (shells beyond 10, fields beyond 64 bits; also dumped as JSON);
  3. compile csrc/llvq.hip for gfx950 with hipcc into weight_decompression_amd/libllvq.so.

Generated files go to <repo>/_build/ (not committed).  Packed-fp32 VALU instructions
are switched off for all device code.
"""

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
BUILD_DIR = os.path.join(REPO_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libllvq.so")
TABLES_INC = os.path.join(BUILD_DIR, "llvq_tables.inc")
TABLES_JSON = os.path.join(BUILD_DIR, "llvq_tables.json")
SEARCH_INC = os.path.join(BUILD_DIR, "llvq_search.inc")
WIDE_INC = os.path.join(BUILD_DIR, "llvq_wide.inc")
WIDE_JSON = os.path.join(BUILD_DIR, "llvq_wide.json")
GEN_BIN = os.path.join(BUILD_DIR, "gen_tables")

OFFLOAD_ARCH = "gfx950"


def _run(cmd, verbose):
    if verbose:
        print("+ " + " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_tables(verbose=True):
    """Compile the generator and write its outputs.  Every file is written under a name
    private to this process and renamed into place, so concurrent builds (parallel test
    workers) never read a half-written table or run a generator that is being linked."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    tag = f".{os.getpid()}.tmp"
    gen = GEN_BIN + tag
    _run(["g++", "-O2", "-std=c++17", "-Wall", "-o", gen, os.path.join(CSRC, "gen_tables.cpp")], verbose)
    try:
        for flag, path in (("--header", TABLES_INC), ("--json", TABLES_JSON), ("--search", SEARCH_INC),
                           ("--wide", WIDE_INC), ("--wide-json", WIDE_JSON)):
            _run([gen, flag, path + tag], verbose)
            os.replace(path + tag, path)
        os.replace(gen, GEN_BIN)
    finally:
        for path in (gen,) + tuple(p + tag for p in (TABLES_INC, TABLES_JSON, SEARCH_INC, WIDE_INC, WIDE_JSON)):
            if os.path.exists(path):
                os.remove(path)


def hipcc_path():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the LLVQ library needs ROCm's hipcc to build")
    return p


CHECKS_LIB_PATH = os.path.join(PKG_DIR, "libllvq_checks.so")


def build(verbose=True, device_checks=False):
    """Build libllvq.so, or with device_checks the same library with the in-kernel invariant
    checks on (LLVQ_DEVICE_CHECKS) as libllvq_checks.so, for tests."""
    build_tables(verbose)
    out = CHECKS_LIB_PATH if device_checks else LIB_PATH
    tmp = out + ".tmp"
    cmd = [
        hipcc_path(),
        f"--offload-arch={OFFLOAD_ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-fvisibility=hidden",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-I", INCLUDE,
        "-I", CSRC,
        "-I", BUILD_DIR,
        "-o", tmp,
        os.path.join(CSRC, "llvq.hip"),
    ]
    if device_checks:
        cmd.insert(1, "-DLLVQ_DEVICE_CHECKS")
    _run(cmd, verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    build(verbose=True, device_checks=True)
    sys.exit(0)
