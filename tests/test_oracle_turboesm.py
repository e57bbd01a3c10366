"""Pins for the oracle's TurboESM variant (CPU only): the per-coordinate
residual signs with a calibrated mean residual magnitude, calibrated
symmetric tables, and values kept in their original coordinates.

Each test checks the oracle against something other than itself: brute
force over partitions, a closed form of the uniform law, Monte Carlo samples
of the sphere, a least-squares scan, an identity that holds only when the
packed sign bits line up with the residuals, or a record worked by hand
(tests/golden/turboesm_sign_record.json).
"""
import json
import os

import numpy as np
import pytest

from oracle import calibration, codec, estimator, lloyd_max, rotation

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sphere(n, d, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def _best_partition_levels(a, half):
    """Upper-half levels of the least-squares partition of sorted a into
    `half` contiguous groups, by trying every split."""
    import itertools
    a = np.sort(a)
    n = len(a)
    best, arg = np.inf, None
    for cuts in itertools.combinations(range(1, n), half - 1):
        groups = np.split(a, cuts)
        sse = sum(((g - g.mean()) ** 2).sum() for g in groups)
        if sse < best - 1e-15:
            best, arg = sse, [g.mean() for g in groups]
    return np.array(arg)


@pytest.mark.parametrize("seed", range(4))
def test_symmetric_lloyd_reaches_the_brute_force_partition(seed):
    """Four well-separated clusters of three values, signs scattered: the
    least-squares partition found by trying every split puts one level at
    each cluster's mean, and the calibrated table must be that partition's
    levels, mirrored."""
    g = np.random.default_rng(seed)
    centres = [0.1, 0.35, 0.6, 0.9]
    a = np.concatenate([c + 0.02 * g.standard_normal(3) for c in centres])
    y = a * np.where(g.integers(0, 2, a.size) == 1, 1.0, -1.0)   # signs do not matter
    t = calibration.symmetric_lloyd(y, 3)
    want = _best_partition_levels(a, 4)
    np.testing.assert_allclose(t[4:], want, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(t[:4], -t[4:][::-1])


@pytest.mark.parametrize("seed", range(6))
def test_symmetric_lloyd_ends_at_a_fixed_point(seed):
    """On clustered samples of unequal sizes (where Lloyd's method, a local
    one, may stop short of the best partition) the result still satisfies
    both Lloyd-Max conditions, checked by brute force: every level is the
    mean of the values nearest to it among all levels."""
    g = np.random.default_rng(seed)
    sizes = g.permutation([6, 2, 2, 3])
    centres = [0.1, 0.35, 0.6, 0.9]
    a = np.concatenate([c + 0.01 * g.standard_normal(s) for c, s in zip(centres, sizes)])
    t = calibration.symmetric_lloyd(a, 3)
    up = t[4:]
    nearest = np.argmin(np.abs(a[:, None] - up[None, :]), axis=1)
    for j in range(4):
        if np.any(nearest == j):
            assert abs(a[nearest == j].mean() - up[j]) < 1e-15


def test_uniform_law_gives_the_uniform_quantiser():
    """For the uniform law on [-1, 1] the Lloyd-Max table is the uniform
    quantiser, levels (2j+1)/K - 1 (within the sample's noise)."""
    y = np.random.default_rng(3).uniform(-1.0, 1.0, 2_000_000)
    for bits in (1, 2, 3):
        K = 1 << bits
        t = calibration.symmetric_lloyd(y, bits)
        want = (2 * np.arange(K) + 1) / K - 1
        np.testing.assert_allclose(t, want, atol=2e-3)


def test_sphere_sample_reproduces_the_beta_table_and_its_mean_error():
    """Rotated unit vectors are uniform on the sphere, so a calibration on
    many of them lands on the Beta-law Lloyd-Max table, and its mean
    residual magnitude on the Beta-law E|Y - Q(Y)|."""
    d, bits = 64, 3
    y = _sphere(40_000, d, 5)
    t = calibration.symmetric_lloyd(y, bits)
    t_ref, _ = lloyd_max.lloyd_max(d, bits)
    np.testing.assert_allclose(t, t_ref, atol=1.5e-3)
    t32, tau32 = lloyd_max.table_f32(d, bits)
    mu_mc = calibration.mean_residual_magnitude(t32, tau32, y)
    mu = lloyd_max.mean_abs_error(t32, tau32, d)
    assert abs(mu_mc - mu) < 2e-3 * mu, (mu_mc, mu)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mean_abs_error_closed_form_for_the_uniform_marginal(bits):
    """d = 3: one coordinate of a uniform point on S^2 is uniform on [-1, 1]
    and the table is the uniform quantiser with cells of width 2/K, so the
    error is uniform on [-1/K, 1/K] in every cell: E|e| = 1/(2K)."""
    t32, tau32 = lloyd_max.table_f32(3, bits)
    K = 1 << bits
    assert abs(lloyd_max.mean_abs_error(t32, tau32, 3) - 1.0 / (2 * K)) < 1e-9


def test_mu_is_the_least_squares_scale_of_the_signs():
    """Scanning a, the mean of (e - a sign(e))^2 is smallest at a = mean|e|,
    the value the calibration stores."""
    g = np.random.default_rng(8)
    y = _sphere(2000, 64, 9) @ rotation.rht_matrix(np.where(g.integers(0, 2, 64) == 1, 1, -1)).T
    t32, tau32 = lloyd_max.table_f32(64, 3)
    c = calibration.quantise_f32(t32, tau32, y)
    e = y - t32.astype(np.float64)[c]
    grid = np.linspace(0.0, 0.05, 20001)
    cost = [np.mean((e - a * np.sign(e)) ** 2) for a in grid]
    a_best = grid[int(np.argmin(cost))]
    mu = calibration.mean_residual_magnitude(t32, tau32, y)
    assert abs(a_best - mu) <= 2.5e-6, (a_best, mu)


@pytest.mark.parametrize("rot", ["hadamard", "none"])
def test_packed_signs_line_up_with_the_residuals(rot):
    """With z unpacked from the record, mean (e - mu z)^2 = mean e^2 - mu^2
    for mu = mean |e|: an identity that fails if any sign bit belongs to
    another coordinate or has the opposite convention."""
    d, bits = 128, 3
    cb = codec.make_sign_codebook(d, bits, rot, seed=4)
    x = np.random.default_rng(11).standard_normal((300, d)) * np.linspace(0.2, 3.0, d)
    enc = codec.encode(cb, x)
    _, z = codec.dequant(cb, enc)
    e = enc.e
    mu = np.abs(e).mean()
    lhs = np.mean((e - mu * z) ** 2)
    assert abs(lhs - (np.mean(e * e) - mu * mu)) < 1e-12
    assert enc.signs.shape == (300, d // 32)


def test_rotation_none_quantises_the_unit_vector_itself():
    d = 64
    cb = codec.make_sign_codebook(d, 3, "none", mu=[0.01])
    x = np.random.default_rng(2).standard_normal((50, d))
    enc = codec.encode(cb, x)
    np.testing.assert_array_equal(enc.y, x / np.linalg.norm(x, axis=1, keepdims=True))
    np.testing.assert_array_equal(enc.code_idx, calibration.quantise_f32(cb.t32, cb.tau32, enc.y))


def test_worked_sign_record():
    """A record worked by hand (tests/golden/turboesm_sign_record.json):
    codes, sign word, norm, the rebuilt vector and two logits."""
    with open(os.path.join(GOLDEN, "turboesm_sign_record.json")) as f:
        case = json.load(f)
    d = case["d"]
    cb = codec.make_sign_codebook(d, case["bits"], "none", levels=case["levels"], mu=case["mu"])
    x = np.zeros((1, d))
    x[0, :len(case["x_head"])] = case["x_head"]
    enc = codec.encode(cb, x)
    assert enc.norm[0] == case["norm"]
    assert [int(w) for w in enc.codes[0]] == [int(w, 16) for w in case["code_words"]]
    assert [int(w) for w in enc.signs[0]] == [int(w, 16) for w in case["sign_words"]]
    rec = codec.reconstruct(cb, enc)[0]
    want = np.full(d, case["rebuilt_tail"])
    want[:len(case["rebuilt_head"])] = case["rebuilt_head"]
    np.testing.assert_allclose(rec, want, rtol=0, atol=1e-12)
    for q_head, lg in case["logits"]:
        q = np.zeros((1, d))
        q[0, :len(q_head)] = q_head
        qp, s = estimator.prep_query(cb, q)
        assert abs(estimator.logits(cb, qp, s, enc)[0, 0] - lg) < 1e-12


def test_sign_logits_and_values_agree_with_the_rebuilt_vectors():
    """Logits equal <q, rebuilt key> (q' = Pi q against Pi^T in the
    rebuild) and each head uses its own mu; a value row is the rebuilt
    value."""
    d, bits = 64, 3
    g = np.random.default_rng(21)
    mu = np.array([0.011, 0.017], np.float32)
    ck = codec.make_sign_codebook(d, bits, "hadamard", seed=7, mu=mu)
    cv = codec.make_sign_codebook(d, bits, "none", mu=mu[::-1].copy())
    k = g.standard_normal((40, d))
    v = g.standard_normal((40, d))
    q = g.standard_normal((3, d))
    ek, ev = codec.encode(ck, k), codec.encode(cv, v)
    for head in (0, 1):
        qp, s = estimator.prep_query(ck, q)
        lg = estimator.logits(ck, qp, s, ek, head)
        np.testing.assert_allclose(lg, q @ codec.reconstruct(ck, ek, head).T, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(estimator.value_rows(cv, ev, head), codec.reconstruct(cv, ev, head),
                                   rtol=0, atol=1e-15)
    # the two heads' logits differ by (mu_1 - mu_0) nu <q', z>
    qp, s = estimator.prep_query(ck, q)
    _, z = codec.dequant(ck, ek)
    diff = estimator.logits(ck, qp, s, ek, 1) - estimator.logits(ck, qp, s, ek, 0)
    np.testing.assert_allclose(diff, (float(mu[1]) - float(mu[0])) * (ek.norm[:, None] * (z @ qp.T)).T,
                               rtol=1e-9, atol=1e-12)


def test_sign_correction_improves_on_codes_alone():
    """The calibrated sign correction lowers the rebuild error of held-out
    vectors below that of the codes alone (the MSE-only estimate)."""
    d, bits = 64, 3
    g = np.random.default_rng(30)
    sig = np.where(g.integers(0, 2, d) == 1, 1, -1)
    pi = rotation.rht_matrix(sig)
    cal = g.standard_normal((512, 2, d))
    lv, mu = calibration.calibrate(pi, bits, cal)
    cb = codec.make_sign_codebook(d, bits, "hadamard", sigma=sig, levels=lv, mu=mu)
    cb0 = codec.make_sign_codebook(d, bits, "hadamard", sigma=sig, levels=lv, mu=[0.0])
    x = g.standard_normal((400, d))
    err = np.mean((codec.reconstruct(cb, codec.encode(cb, x)) - x) ** 2)
    err0 = np.mean((codec.reconstruct(cb0, codec.encode(cb0, x)) - x) ** 2)
    assert err < 0.8 * err0, (err, err0)


def test_calibrate_per_head_mu_and_rope():
    """calibrate(): one table for all heads, mu per head (a head scaled by a
    constant has the same unit vectors, hence the same mu); RoPE is applied
    at tok_offset + t before the rotation."""
    from oracle.rope import rope_table, apply_rope
    d, bits = 64, 3
    g = np.random.default_rng(40)
    sig = np.where(g.integers(0, 2, d) == 1, 1, -1)
    pi = rotation.rht_matrix(sig)
    base = g.standard_normal((256, 1, d))
    x = np.concatenate([base, 7.0 * base, g.standard_normal((256, 1, d))], axis=1)
    cos, sin = rope_table(10000.0, d, 600)
    lv, mu = calibration.calibrate(pi, bits, x, tok_offset=100, rope=(cos, sin))
    assert abs(mu[0] - mu[1]) <= 1e-7 * mu[0] and mu[2] != mu[0]
    # same result when the RoPE is applied by hand first
    pos = 100 + np.arange(256)
    xr = np.stack([apply_rope(x[:, j], pos, cos, sin) for j in range(3)], axis=1)
    lv2, mu2 = calibration.calibrate(pi, bits, xr)
    np.testing.assert_array_equal(lv, lv2)
    np.testing.assert_array_equal(mu, mu2)
    np.testing.assert_array_equal(lv, -lv[::-1])
