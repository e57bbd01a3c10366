"""Pins for the oracle's logit and decode estimates (CPU only)."""
import numpy as np
import pytest
from scipy import special

from oracle import codec, estimator, lloyd_max, rope, rotation
from synth import codec_draws


def _cb(d, bits, m, dense=False, seed=0):
    sigma, rg, sk = codec_draws(d, m, dense, seed)
    return codec.make_codebook(d, bits, m, dense, sigma, rg, sk)


def test_qjl_logit_is_unbiased_with_closed_form_variance():
    """Over many independent Gaussian sketches the logit's mean converges to
    the exact <q, k> (within 4 standard errors) and its variance matches
    nu^2 (pi/(2m) gamma^2 ||q'||^2 - <q',e>^2/m) (iaemfoco post, "TurboQuant:
    Uma Nova Abordagem"; itstec post, "Por dentro do processo")."""
    d, bits, m = 128, 2, 64
    g = np.random.default_rng(21)
    sigma = np.where(g.integers(0, 2, d) == 1, 1, -1)
    k = g.standard_normal((1, d)) * 3.0
    q = g.standard_normal((1, d))
    true = float(q[0] @ k[0])
    n = 4000
    vals = np.empty(n)
    for i in range(n):
        cb = codec.make_codebook(d, bits, m, False, sigma, None, g.standard_normal((m, d)).astype(np.float32))
        enc = codec.encode(cb, k)
        qp, s = estimator.prep_query(cb, q)
        vals[i] = estimator.logits(cb, qp, s, enc)[0, 0]
    # the quantised part does not depend on S; e, q' are the same every time
    cb = codec.make_codebook(d, bits, m, False, sigma, None, np.zeros((m, d), np.float32))
    enc = codec.encode(cb, k)
    qp, _ = estimator.prep_query(cb, q)
    nu, e = enc.norm[0], enc.e[0]
    var = nu ** 2 * (np.pi / (2 * m) * (e @ e) * (qp[0] @ qp[0]) - (qp[0] @ e) ** 2 / m)
    se = np.sqrt(var / n)
    assert abs(vals.mean() - true) < 4 * se, (vals.mean(), true, se)
    assert abs(vals.var() / var - 1) < 0.1
    # the MSE-only part alone is off by nu <q', e>, many standard errors away
    mse_only = nu * float(qp[0] @ (enc.y[0] - e))
    assert abs(mse_only - true) > 10 * se


def test_mse_only_inner_product_bias_is_d_t1_squared():
    """itstec post, "Por dentro do processo" and tambur post: an MSE-optimal
    quantiser biases inner products.  At b = 1 with a Haar rotation, the
    expectation of nu <Pi q, yhat> is d t_1^2 <q, x> exactly (t_1 = E|Y|), which
    tends to 2/pi; the QJL-corrected estimate has expectation <q, x>."""
    d, bits = 32, 1
    g = np.random.default_rng(33)
    x = g.standard_normal((1, d))
    q = x[0] + 0.5 * g.standard_normal(d)
    true = float(q @ x[0])
    t1 = lloyd_max.lloyd_max(d, 1)[0][1]
    n = 6000
    mse = np.empty(n)
    qjl = np.empty(n)
    for i in range(n):
        cb = codec.make_codebook(d, bits, 32, True, None, g.standard_normal((d, d)),
                                 g.standard_normal((32, d)).astype(np.float32))
        enc = codec.encode(cb, x)
        qp, s = estimator.prep_query(cb, q[None])
        yhat, _ = codec.dequant(cb, enc)
        mse[i] = enc.norm[0] * float(qp[0] @ yhat[0])
        qjl[i] = estimator.logits(cb, qp, s, enc)[0, 0]
    ratio = d * t1 * t1
    assert abs(mse.mean() / true - ratio) < 4 * mse.std() / np.sqrt(n) / abs(true)
    assert abs(qjl.mean() - true) < 4 * qjl.std() / np.sqrt(n)
    assert abs(ratio - 2 / np.pi) < 0.02


@pytest.mark.parametrize("dense", [False, True])
def test_logit_equals_query_dot_decoded_key(dense):
    """The logit formula (codes dotted with q' = Pi q, sign bits dotted with
    s = S q') equals the plain inner product of RoPE(q) with the decoder's
    vector estimate nu Pi^T (yhat + sqrt(pi/2)/m gamma S^T z) of the key
    (FibQuant summary, section 2.3), computed along a different path."""
    d = 64
    cb = _cb(d, 3, 64, dense=dense, seed=4)
    c, s_ = rope.rope_table(10000.0, d, 200)
    g = np.random.default_rng(8)
    k = g.standard_normal((50, d))
    pos = np.arange(50) + 100
    q = g.standard_normal((3, d))
    enc = codec.encode(cb, k, pos, (c, s_))
    qp, s = estimator.prep_query(cb, q, 150, (c, s_))
    lg = estimator.logits(cb, qp, s, enc)
    qr = rope.apply_rope(q, np.full(3, 150), c, s_)
    ref = qr @ codec.reconstruct(cb, enc).T
    np.testing.assert_allclose(lg, ref, rtol=1e-10, atol=1e-10)


def test_attention_is_softmax_attention_over_decoded_rows():
    """With the quantiser's reconstructions as dense K and V matrices, the
    decode output is textbook softmax attention (scipy's softmax) restricted
    to the first seq_len keys; rows beyond seq_len are ignored."""
    d = 64
    ck, cv = _cb(d, 3, 64, seed=0), _cb(d, 3, 64, seed=1)
    g = np.random.default_rng(9)
    k, v = g.standard_normal((2, 40, d))
    q = g.standard_normal((4, d))
    ek, ev = codec.encode(ck, k), codec.encode(cv, v)
    qp, s = estimator.prep_query(ck, q)
    scale = 1 / np.sqrt(d)
    out = estimator.attention(ck, cv, qp, s, ek, ev, 31, scale)
    kh, vh = codec.reconstruct(ck, ek)[:31], codec.reconstruct(cv, ev)[:31]
    ref = special.softmax(scale * q @ kh.T, axis=1) @ vh
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    assert np.all(estimator.attention(ck, cv, qp, s, ek, ev, 0, scale) == 0)


def test_attention_with_identical_keys_averages_values():
    d = 64
    ck, cv = _cb(d, 2, 32, seed=0), _cb(d, 2, 32, seed=1)
    g = np.random.default_rng(10)
    k = np.repeat(g.standard_normal((1, d)), 12, axis=0)
    v = g.standard_normal((12, d))
    ek, ev = codec.encode(ck, k), codec.encode(cv, v)
    qp, s = estimator.prep_query(ck, g.standard_normal((2, d)))
    out = estimator.attention(ck, cv, qp, s, ek, ev, 12, 0.125)
    np.testing.assert_allclose(out, np.repeat(codec.reconstruct(cv, ev).mean(0)[None], 2, 0), rtol=1e-12)


def test_topk_order_and_ties():
    sc = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, -1.0]])
    idx, val = estimator.topk(sc, 4)
    assert idx.tolist() == [[1, 2, 4, 3]] and val.tolist() == [[3.0, 3.0, 3.0, 2.0]]
    g = np.random.default_rng(0).standard_normal((5, 1000))
    idx, val = estimator.topk(g, 10)
    np.testing.assert_array_equal(val, -np.sort(-g, axis=1)[:, :10])


def test_query_and_key_at_one_position_score_their_plain_product():
    """A query RoPE'd at position p against a key RoPE'd at the same p: the
    rotated query q' = Pi RoPE(q, p) and the rotated key Pi RoPE(k, p) have the
    inner product <q, k> of the un-rotated vectors (relative offset 0; TurboESM
    summary, technical section 2: RoPE, then Pi), at any p."""
    from oracle import rope as orope
    d = 128
    cb = codec.make_codebook(d, 3, 64, False, seed=0)
    rope = orope.rope_table(5e5, d, 4096)
    g = np.random.default_rng(12)
    q, k = g.standard_normal((2, d))
    for p in (0, 1, 777, 4095):
        qp, _ = estimator.prep_query(cb, q[None], p, rope)
        kr = orope.apply_rope(k[None], np.array([p]), rope[0], rope[1]) @ cb.pi.T
        # (the float32 RoPE table and rotation keep norms to about 1e-8)
        assert abs(float(qp[0] @ kr[0]) - float(q @ k)) < 1e-6 * (1 + abs(float(q @ k)))
    # a query one position after its key does not
    qp, _ = estimator.prep_query(cb, q[None], 778, rope)
    kr = orope.apply_rope(k[None], np.array([777]), rope[0], rope[1]) @ cb.pi.T
    assert abs(float(qp[0] @ kr[0]) - float(q @ k)) > 1e-3
