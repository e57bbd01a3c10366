"""Pins for the oracle's Lloyd-Max table (CPU only).

Each test checks the oracle against something other than itself: an
independent quadrature, a closed form, a textbook table, Monte Carlo samples
of the sphere, or brute force.
"""
import math
import os

import numpy as np
import pytest
from scipy import integrate, special, stats

from oracle import lloyd_max as lm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _quad(f, a, b):
    return integrate.quad(f, a, b, limit=400, epsabs=0.0, epsrel=1e-13)[0]


@pytest.mark.parametrize("d", [4, 16, 128, 1536])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_centroid_and_midpoint_conditions(d, bits):
    """Both optimality conditions hold under an adaptive quadrature of the
    density written out directly (no incomplete beta function)."""
    t, tau = lm.lloyd_max(d, bits)
    logc = math.lgamma(d / 2) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2)
    pdf = lambda y: math.exp(logc + 0.5 * (d - 3) * math.log1p(-y * y)) if abs(y) < 1 else 0.0
    edges = np.concatenate([[-1.0], tau, [1.0]])
    scale = 1.0 / math.sqrt(d)
    # restrict the outer cells to where the density is not negligible
    lim = min(1.0, 40.0 * scale)
    for j in range(len(t)):
        a, b = max(edges[j], -lim), min(edges[j + 1], lim)
        mass = _quad(pdf, a, b)
        mom = _quad(lambda y: y * pdf(y), a, b)
        assert abs(mom / mass - t[j]) < 1e-10 * scale, (j, mom / mass, t[j])
    np.testing.assert_allclose(tau, 0.5 * (t[:-1] + t[1:]), rtol=0, atol=0)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_d3_is_uniform_quantiser(bits):
    """At d = 3 a sphere coordinate is uniform on [-1, 1] (Archimedes), so the
    Lloyd-Max table is the uniform quantiser with K cells."""
    t, tau = lm.lloyd_max(3, bits)
    K = 1 << bits
    np.testing.assert_allclose(t, (2 * np.arange(K) + 1) / K - 1, atol=1e-13)
    np.testing.assert_allclose(tau, 2 * np.arange(1, K) / K - 1, atol=1e-13)


@pytest.mark.parametrize("d", [3, 5, 8, 64, 128, 1536])
def test_one_bit_levels_closed_form(d):
    """b = 1: cells are the half lines, levels +-E|Y| with
    E|Y| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))."""
    t, tau = lm.lloyd_max(d, 1)
    e_abs = math.exp(math.lgamma(d / 2) - 0.5 * math.log(math.pi) - math.lgamma((d + 1) / 2))
    np.testing.assert_allclose(t, [-e_abs, e_abs], rtol=1e-11)
    assert tau[0] == 0.0


def _read_max_table():
    rows = {}
    with open(os.path.join(GOLDEN, "max1960_gaussian_lloyd_max.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = [p.strip() for p in line.split("|")]
            rows[int(parts[0])] = ([float(v) for v in parts[1].split()],
                                   [float(v) for v in parts[2].split()] if parts[2] else [])
    return rows


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_large_d_tends_to_gaussian_table(bits):
    """sqrt(d) * table at d = 2^20 reproduces Max (1960)'s Gaussian table to
    its printed precision."""
    levels, thr = _read_max_table()[bits]
    d = 1 << 20
    t, tau = lm.lloyd_max(d, bits)
    K = 1 << bits
    np.testing.assert_allclose(np.sqrt(d) * t[K // 2:], levels, atol=6e-4)
    np.testing.assert_allclose(np.sqrt(d) * tau[K // 2:], thr, atol=6e-4)


@pytest.mark.parametrize("d", [4, 5, 9])
def test_density_matches_sphere_samples(d):
    """Coordinates of normalised Gaussian vectors (uniform on the sphere)
    follow the oracle's marginal law (Kolmogorov-Smirnov), and the law has
    E[Y] = 0 and E[Y^2] = 1/d."""
    g = np.random.default_rng(1234 + d)
    x = g.standard_normal((200_000, d))
    y = (x / np.linalg.norm(x, axis=1, keepdims=True))[:, 0]
    res = stats.kstest(y, lambda v: lm.marginal_cdf(v, d))
    assert res.pvalue > 1e-3, res
    m0 = _quad(lambda v: lm.marginal_pdf(np.array([v]), d)[0], -1, 1)
    m2 = _quad(lambda v: v * v * lm.marginal_pdf(np.array([v]), d)[0], -1, 1)
    assert abs(m0 - 1) < 1e-10 and abs(m2 - 1 / d) < 1e-10


def test_density_is_the_beta_law():
    """(1 + Y)/2 ~ Beta((d-1)/2, (d-1)/2): compare the density with scipy's
    beta distribution at a few points."""
    for d in (4, 7, 128):
        a = (d - 1) / 2
        y = np.linspace(-0.9, 0.9, 13) / (1 if d < 10 else 5)
        np.testing.assert_allclose(lm.marginal_pdf(y, d), stats.beta.pdf((1 + y) / 2, a, a) / 2, rtol=1e-11)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_threshold_rule_is_nearest_level(bits):
    """The threshold code equals brute-force argmin |y - t_k| (midpoint
    thresholds make the two the same away from exact ties)."""
    d = 128
    t, tau = lm.table_f32(d, bits)
    y = np.random.default_rng(7).standard_normal(100_000) / np.sqrt(d)
    code = (y[:, None] >= tau[None, :]).sum(1)
    dist = np.abs(y[:, None] - t[None, :].astype(np.float64))
    near = np.argmin(dist, axis=1)
    srt = np.sort(dist, axis=1)
    clear = srt[:, 1] - srt[:, 0] > 1e-7
    assert np.array_equal(code[clear], near[clear])


@pytest.mark.parametrize("d,bits", [(16, 2), (128, 3)])
def test_table_is_a_local_minimum_of_distortion(d, bits):
    """Moving any one level (thresholds re-derived as midpoints) raises the
    mean squared error computed by quadrature."""
    t, tau = lm.lloyd_max(d, bits)
    base = lm.distortion(t, tau, d)
    h = 0.02 / np.sqrt(d)
    for j in range(len(t)):
        for sgn in (-1, 1):
            t2 = t.copy()
            t2[j] += sgn * h
            t2 = np.sort(t2)
            assert lm.distortion(t2, 0.5 * (t2[:-1] + t2[1:]), d) > base


@pytest.mark.parametrize("d", [3, 64, 128, 1536])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_table_is_symmetric(d, bits):
    t, tau = lm.table_f32(d, bits)
    assert np.array_equal(t, -t[::-1])
    assert np.array_equal(tau, -tau[::-1])
    assert tau[len(tau) // 2] == 0.0
    assert np.all(np.diff(t) > 0) and np.all(np.diff(tau) > 0)
