"""Pins for the oracle's rotations and RoPE (CPU only)."""
import numpy as np
import pytest
import scipy.linalg

from oracle import rotation, rope


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 64, 128, 256])
def test_hadamard_matches_scipy_and_kronecker(d):
    h = rotation.sylvester_hadamard(d)
    np.testing.assert_array_equal(h, scipy.linalg.hadamard(d))
    if d > 1:
        np.testing.assert_array_equal(h, np.kron([[1, 1], [1, -1]], rotation.sylvester_hadamard(d // 2)))


@pytest.mark.parametrize("d", [16, 64, 128])
def test_rht_is_orthogonal_and_spreads_mass(d):
    """Pi Pi^T = I, norms and inner products are kept (TurboESM summary,
    technical section 2: Pi^T Pi = I), and a unit spike becomes a vector whose
    entries all have magnitude 1/sqrt(d) (TurboESM summary, plain-language
    point 2: the heavy outlier spread evenly)."""
    g = np.random.default_rng(d)
    sigma = np.where(g.integers(0, 2, d) == 1, 1, -1)
    pi = rotation.rht_matrix(sigma)
    np.testing.assert_allclose(pi @ pi.T, np.eye(d), atol=1e-13)
    x, y = g.standard_normal((2, d))
    np.testing.assert_allclose(np.linalg.norm(pi @ x), np.linalg.norm(x), rtol=1e-13)
    np.testing.assert_allclose((pi @ x) @ (pi @ y), x @ y, rtol=1e-12, atol=1e-12)
    for j in (0, d // 3, d - 1):
        np.testing.assert_allclose(np.abs(pi[:, j]), 1 / np.sqrt(d), rtol=1e-15)


@pytest.mark.parametrize("d", [3, 32, 200])
def test_haar_is_the_positive_diagonal_qr_factor(d):
    """Q is orthogonal and Q^T G is upper triangular with a positive diagonal,
    which fixes Q uniquely for a full-rank G."""
    g = np.random.default_rng(10 + d).standard_normal((d, d))
    q = rotation.haar_rotation(g)
    np.testing.assert_allclose(q.T @ q, np.eye(d), atol=1e-12)
    r = q.T @ g
    assert np.all(np.abs(np.tril(r, -1)) < 1e-10)
    assert np.all(np.diag(r) > 0)


def test_haar_first_column_is_uniform_on_sphere():
    """Columns of a Haar rotation are uniform on the sphere: at d = 3 a
    coordinate is uniform on [-1, 1], so its mean is 0 and its variance 1/3."""
    g = np.random.default_rng(5)
    v = np.array([rotation.haar_rotation(g.standard_normal((3, 3)))[0, 0] for _ in range(20000)])
    assert abs(v.mean()) < 0.02 and abs(v.var() - 1 / 3) < 0.01


def test_rope_position_zero_is_identity_and_norm_is_kept():
    d = 128
    c, s = rope.rope_table(500000.0, d, 64)
    x = np.random.default_rng(0).standard_normal((64, d))
    np.testing.assert_array_equal(rope.apply_rope(x[:1], np.array([0]), c, s), x[:1])
    xr = rope.apply_rope(x, np.arange(64), c, s)
    np.testing.assert_allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)


def test_rope_relative_position():
    """<R_a q, R_b k> = <q, R_{b-a} k>: the score depends on the offset only."""
    d = 64
    c, s = rope.rope_table(10000.0, d, 300)
    g = np.random.default_rng(1)
    q, k = g.standard_normal((2, 1, d))
    for a, b in [(5, 17), (100, 250), (0, 299)]:
        lhs = rope.apply_rope(q, np.array([a]), c, s) @ rope.apply_rope(k, np.array([b]), c, s).T
        rhs = q @ rope.apply_rope(k, np.array([b - a]), c, s).T
        np.testing.assert_allclose(lhs, rhs, rtol=1e-5, atol=1e-5)


def test_rope_before_rotation_keeps_scores_rotation_before_rope_does_not():
    """TurboESM summary, technical section 2 and contribution 1: RoPE first,
    then Pi, leaves every attention score exactly as without Pi; rotating
    before RoPE does not."""
    d = 64
    c, s = rope.rope_table(10000.0, d, 64)
    g = np.random.default_rng(2)
    pi = rotation.haar_rotation(g.standard_normal((d, d)))
    q, k = g.standard_normal((2, 1, d))
    pq, pk = 3, 40
    ref = rope.apply_rope(q, [pq], c, s) @ rope.apply_rope(k, [pk], c, s).T
    good = (rope.apply_rope(q, [pq], c, s) @ pi.T) @ (rope.apply_rope(k, [pk], c, s) @ pi.T).T
    bad = rope.apply_rope(q @ pi.T, [pq], c, s) @ rope.apply_rope(k @ pi.T, [pk], c, s).T
    np.testing.assert_allclose(good, ref, rtol=1e-12)
    assert abs(bad - ref).item() > 1e-3


def _angle_per_position(c, s):
    """Angle of each pair at position 1, from the table's cos and sin."""
    return np.arctan2(s[1].astype(np.float64), c[1].astype(np.float64))


def test_rope_frequencies_closed_form_cases():
    """RoFormer's frequencies are a geometric sequence starting at 1 rad per
    position with ratio base^(-2/d).  At d = 8 and base 1e4 the angles per
    position are exactly 1, 0.1, 0.01 and 0.001; at d = 4, base 1e4 they are
    1 and 0.01; for any d, pair d/4 turns by base^(-1/2) (1/100 at base 1e4,
    1/sqrt(5e5) = 1.41421356e-3 at base 5e5)."""
    c, s = rope.rope_table(10000.0, 8, 4)
    np.testing.assert_allclose(_angle_per_position(c, s), [1.0, 0.1, 0.01, 0.001], rtol=1e-6)
    c, s = rope.rope_table(10000.0, 4, 4)
    np.testing.assert_allclose(_angle_per_position(c, s), [1.0, 0.01], rtol=1e-6)
    for base, want in ((10000.0, 0.01), (500000.0, 1.41421356e-3)):
        c, s = rope.rope_table(base, 128, 2)
        np.testing.assert_allclose(_angle_per_position(c, s)[32], want, rtol=1e-6)
    # position p turns pair 0 by exactly p radians (cos(3) = -0.9899924966)
    c, s = rope.rope_table(500000.0, 128, 8)
    assert abs(float(c[3, 0]) - (-0.9899924966)) < 1e-7
    assert abs(float(s[3, 0]) - 0.1411200081) < 1e-7
