"""Pins for the oracle's counter-based generator (CPU only).

SplitMix64 is checked against its published test vectors
(tests/golden/splitmix64_published.txt) and against a second evaluation in
wrapping numpy uint64 arithmetic; the purpose streams against the same
vectors; Box-Muller at inputs whose outputs have closed forms and by a
Kolmogorov-Smirnov test against N(0,1); uniforms and signs by their range and
moments.
"""
import math
import os

import numpy as np
import scipy.stats

from oracle import rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_published.txt")


def _published():
    out = {}
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            seed, vals = line.split("|")
            out[int(seed)] = [int(v, 0) for v in vals.split()]
    return out


def test_splitmix64_reproduces_published_vectors():
    pub = _published()
    assert set(pub) == {0, 1234567}
    for seed, vals in pub.items():
        assert rng.splitmix64(seed, len(vals)) == vals


def test_purpose_streams_start_at_the_published_outputs():
    """Purpose p's stream starts at output p of the generator seeded with the
    codebook seed; with seeds 0 and 1234567 those outputs are published."""
    pub = _published()
    for seed, vals in pub.items():
        for p in (1, 2, 3):
            assert rng.stream_state(seed, p) == vals[p - 1]
    # the uniforms of a stream are the top 53 bits of its outputs
    first = rng.splitmix64(pub[0][2], 1)[0]
    assert rng.uniforms(0, 3, 1)[0] == (first >> 11) * 2.0 ** -53


def _splitmix_numpy(state, n):
    with np.errstate(over="ignore"):
        s = np.uint64(state) + np.arange(1, n + 1, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15)
        z = (s ^ (s >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def test_splitmix64_matches_wrapping_uint64_evaluation():
    for seed in (0, 1, 0xDEADBEEF, 2 ** 64 - 1):
        a = np.array(rng.splitmix64(seed, 1000), dtype=np.uint64)
        np.testing.assert_array_equal(a, _splitmix_numpy(seed, 1000))


def test_box_muller_closed_form_points():
    """Radius sqrt(-2 ln(1 - u1)) and angle 2 pi u2: 1 - u1 = e^-2 gives radius
    2, 1 - u1 = e^-1/2 gives radius 1; u2 = 0, 1/4, 1/2 point along +x, +y, -x."""
    z0, z1 = rng.box_muller(1.0 - math.exp(-2.0), 0.0)
    assert abs(z0 - 2.0) < 1e-15 and z1 == 0.0
    z0, z1 = rng.box_muller(1.0 - math.exp(-0.5), 0.25)
    assert abs(z0) < 1e-15 and abs(z1 - 1.0) < 1e-15
    z0, z1 = rng.box_muller(1.0 - math.exp(-4.5), 0.5)
    assert abs(z0 + 3.0) < 1e-14 and abs(z1) < 1e-14
    assert rng.box_muller(0.0, 0.3) == (0.0, 0.0)


def test_gaussians_are_standard_normal_by_kolmogorov_smirnov():
    for seed, purpose in ((3, 3), (0, 2), (1234567, 3)):
        z = rng.gaussians(seed, purpose, 100_000)
        assert scipy.stats.kstest(z, "norm").pvalue > 1e-3
    # the pairs are independent: the two halves of each pair are uncorrelated
    z = rng.gaussians(11, 3, 200_000).reshape(-1, 2)
    assert abs(np.corrcoef(z[:, 0], z[:, 1])[0, 1]) < 0.01


def test_streams_are_distinct_and_reproducible():
    s = {p: rng.stream_state(7, p) for p in (1, 2, 3)}
    assert len(set(s.values())) == 3
    np.testing.assert_array_equal(rng.gaussians(7, 3, 101), rng.gaussians(7, 3, 101))


def test_uniform_and_gaussian_moments():
    u = rng.uniforms(3, 2, 200_000)
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.003
    assert scipy.stats.kstest(u, "uniform").pvalue > 1e-3
    z = rng.gaussians(3, 3, 200_000)
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1) < 0.01
    assert abs(np.mean(z ** 4) - 3) < 0.06
    sg = rng.signs(3, 100_000)
    assert set(np.unique(sg)) == {-1, 1} and abs(sg.mean()) < 0.01
