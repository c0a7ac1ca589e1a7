"""Inputs of the Gaussian-source fidelity measurement (weight_decompression_amd/synth.py):
the chi-distribution gain table against Monte Carlo cell means of the norms of 24-dim
standard Gaussian vectors, and the source's moments."""

import numpy as np

from weight_decompression_amd import synth


def test_chi_gain_table_matches_sampled_cell_means():
    g = synth.chi_gain_table(16).astype(np.float64)
    assert g.shape == (16,) and np.all(np.diff(g) > 0)
    x = np.random.default_rng(11).standard_normal((400000, 24))
    r = np.sort(np.linalg.norm(x, axis=1))
    cells = np.array_split(r, 16)      # equal-probability cells of the sample
    want = np.array([c.mean() for c in cells])
    assert np.allclose(g, want, rtol=4e-3), (g, want)


def test_gaussian_source_moments():
    x = synth.gaussian_source(6, 50000).astype(np.float64)
    assert x.shape == (50000, 24)
    assert abs(x.mean()) < 0.01 and abs(x.var() - 1.0) < 0.01
