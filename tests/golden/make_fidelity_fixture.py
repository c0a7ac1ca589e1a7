"""Write the fidelity-row fixture for the MLP-shaped shape-gain workload.

For each of the two MLP tensors (11008x4096 and 4096x11008, rows x cols) the first 64
rows are dense N(0, 0.02^2) weights (seeded, from weight_decompression_amd/synth.py)
quantised by the oracle: every 24-block (zero-padded past the last column) gets the
exact angular search over shells 2..10 (oracle/search.py) and the gain index of the
nearest entry of the tensor's 16-entry gain table (0.02 * sorted |N(0,1)| * sqrt(24),
ties to the lower index).

Only oracle/ and the seeded input generator are used.  Output:
tests/golden/fidelity_c3_{0,1}.npz with arrays shape_idx (uint64 [64, Kb]) and
gain_idx (uint8 [64, Kb]).

Usage: python tests/golden/make_fidelity_fixture.py [--rows 64] [--procs 8]
"""

import argparse
import multiprocessing as mp
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import search  # noqa: E402
from weight_decompression_amd import synth  # noqa: E402

SHAPES = ((11008, 4096), (4096, 11008))


def _row(args):
    which, r, rows = args
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    _, cols = SHAPES[which]
    W = synth.fidelity_weights(3, which, rows, cols)
    gains = synth.draw_gain_table(3, which, 16, 0.02).astype(np.float64)
    kb = synth.blocks_per_row(cols)
    wpad = np.zeros(kb * 24)
    wpad[:cols] = W[r]
    s_idx = np.zeros(kb, dtype=np.uint64)
    g_idx = np.zeros(kb, dtype=np.uint8)
    for b in range(kb):
        blk = wpad[b * 24:(b + 1) * 24]
        I, _ = search.search(blk, 10, "angular")
        s_idx[b] = I
        g_idx[b] = search.nearest_gain(np.linalg.norm(blk), gains)
    return which, r, s_idx, g_idx


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--rows", type=int, default=64)
    ap.add_argument("--procs", type=int, default=8)
    a = ap.parse_args()
    jobs = [(which, r, a.rows) for which in (0, 1) for r in range(a.rows)]
    out = {0: {}, 1: {}}
    with mp.get_context("fork").Pool(a.procs) as pool:
        for n, (which, r, s_idx, g_idx) in enumerate(pool.imap_unordered(_row, jobs)):
            out[which][r] = (s_idx, g_idx)
            if n % 16 == 0:
                print(f"{n + 1}/{len(jobs)} rows", flush=True)
    for which in (0, 1):
        s = np.stack([out[which][r][0] for r in range(a.rows)])
        g = np.stack([out[which][r][1] for r in range(a.rows)])
        np.savez_compressed(os.path.join(HERE, f"fidelity_c3_{which}.npz"), shape_idx=s, gain_idx=g)
    print("done")


if __name__ == "__main__":
    main()
