"""Pins for the oracle's counter-based generator (CPU only).

SplitMix64 is checked against a second evaluation in wrapping numpy uint64
arithmetic (a different integer path from the oracle's Python integers), and
the derived uniforms, Gaussians and signs against their defining properties.
"""
import numpy as np

from oracle import rng


def _splitmix_numpy(state, n):
    with np.errstate(over="ignore"):
        s = np.uint64(state) + np.arange(1, n + 1, dtype=np.uint64) * np.uint64(rng.GAMMA)
        z = (s ^ (s >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def test_splitmix64_matches_wrapping_uint64_evaluation():
    for seed in (0, 1, 0xDEADBEEF, 2 ** 64 - 1):
        a = np.array(rng.splitmix64(seed, 1000), dtype=np.uint64)
        np.testing.assert_array_equal(a, _splitmix_numpy(seed, 1000))


def test_streams_are_distinct_and_reproducible():
    s = {p: rng.stream_state(7, p) for p in (1, 2, 3)}
    assert len(set(s.values())) == 3
    np.testing.assert_array_equal(rng.gaussians(7, 3, 101), rng.gaussians(7, 3, 101))


def test_uniform_and_gaussian_moments():
    u = rng.uniforms(3, 2, 200_000)
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.003
    z = rng.gaussians(3, 3, 200_000)
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1) < 0.01
    assert abs(np.mean(z ** 4) - 3) < 0.06
    sg = rng.signs(3, 100_000)
    assert set(np.unique(sg)) == {-1, 1} and abs(sg.mean()) < 0.01
