"""Pins for the oracle's FibQuant codebooks (CPU only): the source sample
against Monte Carlo points on the sphere and its exact moments, the N = 2
closed form, Lloyd fixed points by brute force, the vector code's strict
advantage over the scalar Lloyd-Max table at equal rate (FibQuant summary,
sections 3.2 and 4.1), the rate arithmetic, and the decoder/logit pair."""
import math

import numpy as np
import pytest
from scipy import special, stats

from oracle import fibquant as F, lloyd_max, rotation


def _sphere_blocks(n, d, k, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, d))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    return x[:, :k]


@pytest.mark.parametrize("d,k", [(64, 2), (128, 2), (64, 3), (96, 3)])
def test_source_sample_matches_the_sphere(d, k):
    """The equal-mass sample's |x|^2 has nearly the exact mean k/d of a block of a
    uniform point on S^{d-1}, and its radii follow Monte Carlo points on the
    sphere (two-sample Kolmogorov-Smirnov)."""
    pts = F.source_sample(d, k)
    r2 = (pts * pts).sum(1)
    assert abs(r2.mean() - k / d) < 1e-2 * k / d  # 64 midpoint quantiles: within 1 %
    mc = _sphere_blocks(40000, d, k, seed=d + k)
    assert stats.ks_2samp(np.sqrt(r2), np.linalg.norm(mc, axis=1)).pvalue > 1e-3
    # directions are balanced: the sample's mean is (nearly) zero
    assert np.abs(pts.mean(0)).max() < 1e-15


@pytest.mark.parametrize("d,k", [(128, 2), (64, 2), (64, 3)])
def test_two_codewords_sit_at_plus_minus_e_abs_y(d, k):
    """For N = 2 the optimum of a rotationally symmetric source is a pair of
    antipodal points at the mean of one coordinate's absolute value,
    E|Y| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))."""
    c, _ = F.build_codebook(d, k, 2)
    e_abs = math.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    # (the sample's 256 directions resolve E|<x, n>| to a fraction of a percent)
    np.testing.assert_allclose(np.linalg.norm(c, axis=1), e_abs, rtol=3e-3 if k == 2 else 1e-2)
    np.testing.assert_allclose(c[0], -c[1], atol=1e-9)


@pytest.mark.parametrize("d,k,N", [(128, 2, 16), (64, 3, 8), (128, 2, 4)])
def test_refined_codebook_is_a_lloyd_fixed_point(d, k, N):
    """Every codeword is the mean of the sample points nearest to it, the
    nearest codeword found by brute force over all distances."""
    c, mse = F.build_codebook(d, k, N)
    pts = F.source_sample(d, k)
    dist = ((pts[:, None, :] - c[None, :, :]) ** 2).sum(-1)
    near = dist.argmin(1)
    for n in range(N):
        np.testing.assert_allclose(c[n], pts[near == n].mean(0), atol=1e-14)
    assert abs(dist.min(1).mean() - mse) < 1e-12


@pytest.mark.parametrize("d,k,N,bits", [(128, 2, 4, 1), (128, 2, 16, 2), (128, 2, 64, 3), (64, 2, 16, 2),
                                        (64, 3, 8, 1)])
def test_vector_code_beats_the_scalar_table_at_equal_rate(d, k, N, bits):
    """The page's claim of strict dominance over the scalar table at integer
    rates, measured on Monte Carlo points on the sphere (independent of the
    codebook's own sample) against the scalar table's exact distortion."""
    assert math.log2(N) / k == bits
    c, _ = F.build_codebook(d, k, N)
    mc = _sphere_blocks(60000, d, k, seed=7 * N + k)
    vq = ((mc[:, None, :] - c[None, :, :]) ** 2).sum(-1).min(1).mean() / k
    t32, tau32 = lloyd_max.table_f32(d, bits)
    scalar = lloyd_max.distortion(t32, tau32, d)
    assert vq < scalar, (vq, scalar)


def test_rate_arithmetic_and_sub_bit_rates():
    """b = log2(N)/k; a d = 128 record at k = 2, N = 16 is 4 + 64*4/8 = 36
    bytes; k = 3, N = 2 gives one third of a bit per coordinate."""
    sig = np.ones(128)
    cb = F.make_vq_codebook(128, 2, 16, sig, code=np.zeros((16, 2)))
    assert cb.rate == 2.0 and cb.words() == 8 and 4 + 4 * cb.words() == 36
    cb = F.make_vq_codebook(128, 2, 32, sig, code=np.zeros((32, 2)))
    assert cb.rate == 2.5 and cb.words() == 10
    assert F.VQCodebook(96, 3, 2, np.zeros((2, 3), np.float32), np.eye(96)).rate == pytest.approx(1 / 3)


def test_index_packing_by_hand():
    """Indices (3, 0, 2, 1) of 2 bits each: 0b01_10_00_11 = 0x63; with 5 bits
    index j starts at bit 5j and may straddle words."""
    w = F.pack_indices(np.array([[3, 0, 2, 1]]), 2)
    assert w.shape == (1, 1) and int(w[0, 0]) == 0x63
    idx = np.array([[31, 1, 0, 17, 5, 30, 2]])
    w5 = F.pack_indices(idx, 5)
    assert w5.shape == (1, 2)
    # index 6 (value 2) occupies bits 30..34: bit 31 of word 0 is its bit 1
    assert (int(w5[0, 0]) >> 30) & 3 == 2 and int(w5[0, 1]) & 7 == 0
    np.testing.assert_array_equal(F.unpack_indices(w5, 5, 7), idx)


def test_encoder_is_nearest_codeword_and_logits_match_the_decoder():
    """Each block's index is the brute-force nearest codeword of the rotated
    unit vector, and the logits equal <q, rebuilt vector>."""
    d, k, N = 64, 2, 16
    g = np.random.default_rng(3)
    sig = np.where(g.integers(0, 2, d) == 1, 1, -1)
    cb = F.make_vq_codebook(d, k, N, sig)
    x = g.standard_normal((200, d)) * np.linspace(0.5, 2, d)
    enc = F.encode(cb, x)
    y = x / np.linalg.norm(x, axis=1, keepdims=True) @ rotation.rht_matrix(sig).T
    blocks = y.reshape(-1, k)
    brute = ((blocks[:, None, :] - cb.code32[None].astype(np.float64)) ** 2).sum(-1).argmin(1)
    close = enc.margin.ravel() < 1e-9
    assert np.array_equal(brute[~close], enc.idx.ravel()[~close])
    q = g.standard_normal((3, d))
    lg = F.logits(cb, q @ cb.pi.T, enc.norm, enc.codes)
    np.testing.assert_allclose(lg, q @ F.reconstruct(cb, enc.norm, enc.codes).T, rtol=1e-12, atol=1e-12)
    # the decoder's error is the quantiser's: mean squared error per coordinate near the codebook's
    rec = F.reconstruct(cb, enc.norm, enc.codes) / enc.norm[:, None]
    err = ((rec - x / enc.norm[:, None]) ** 2).mean()
    _, mse = F.build_codebook(d, k, N)
    assert abs(err - mse / k) < 0.25 * mse / k


def test_attention_is_softmax_attention_over_decoded_keys_and_values():
    """The fused decode's oracle equals textbook attention (scipy's softmax)
    over the decoder's rebuilt keys and values, with RoPE applied to the
    query before the rotation; no keys give zeros."""
    from scipy.special import softmax
    from oracle import rope as orope
    d, n, G = 64, 300, 3
    g = np.random.default_rng(9)
    sk = np.where(g.integers(0, 2, d) == 1, 1, -1)
    sv = np.where(g.integers(0, 2, d) == 1, 1, -1)
    ck = F.make_vq_codebook(d, 2, 16, sk)
    cv = F.make_vq_codebook(d, 2, 8, sv)
    cs, sn = orope.rope_table(1e4, d, n + 1)
    K, V = g.standard_normal((n, d)) * 2.0, g.standard_normal((n, d))
    ek = F.encode(ck, K, pos=np.arange(n), rope=(cs, sn))
    ev = F.encode(cv, V)
    q = g.standard_normal((G, d))
    q_rot = orope.apply_rope(q, np.full(G, n), cs, sn)
    scale = 1.0 / math.sqrt(d)
    out = F.attention(ck, cv, q_rot @ ck.pi.T, ek.norm, ek.codes, ev.norm, ev.codes, scale)
    khat = F.reconstruct(ck, ek.norm, ek.codes)
    vhat = F.reconstruct(cv, ev.norm, ev.codes)
    ref = softmax(scale * (q_rot @ khat.T), axis=1) @ vhat
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    assert not np.any(F.attention(ck, cv, q_rot @ ck.pi.T, ek.norm[:0], ek.codes[:0], ev.norm[:0], ev.codes[:0],
                                  scale))
