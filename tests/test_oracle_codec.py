"""Pins for the oracle's encoder and record layout (CPU only)."""
import itertools
import os

import numpy as np
import pytest

from oracle import codec, lloyd_max, rotation
from synth import codec_draws

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [64, 128, 1536])
def test_pack_unpack_round_trip(bits, d):
    g = np.random.default_rng(bits * 1000 + d)
    c = g.integers(0, 1 << bits, size=(37, d))
    w = codec.pack_codes(c, bits)
    assert w.shape == (37, bits * d // 32) and w.dtype == np.uint32
    np.testing.assert_array_equal(codec.unpack_codes(w, bits, d), c)
    s = g.integers(0, 2, size=(37, 128))
    np.testing.assert_array_equal(codec.unpack_signs(codec.pack_signs(s), 128), s)


def test_packing_matches_hand_derived_words():
    """The layouts, worked by hand:
    b=2 (LSB first), codes 0,1,2,3 repeated: each byte is 0b11100100 = 0xE4.
    b=3 (groups of 32), codes j % 8: byte k of W0 holds c_k = k (bits 0-2),
    c_{4+k} = 4+k (bits 3-5) and the low bits of c_{24+k} = k (bits 6-7):
    bytes 0x20, 0x69, 0xB2, 0xFB; W1 is the same (c_{8+k}, c_{12+k}, low bits
    of c_{28+k} = 4+k); byte k of W2 holds c_{16+k} = k, c_{20+k} = 4+k, bit
    2 of c_{24+k} (0) at bit 6 and bit 2 of c_{28+k} (1) at bit 7: bytes
    0xA0, 0xA9, 0xB2, 0xBB.
    b=3, single codes: c_26 = 7 puts 0b11 at W0 bits 22-23 and 1 at W2 bit 22;
    c_30 = 5 puts 0b01 at W1 bit 22 and 1 at W2 bit 23; c_13 = 6 (0b110) sits
    at W1 bits 11-13.
    Sketch bits 1,0,0,...,0,1 (bit 0 and bit 31 set) give 0x80000001."""
    c2 = np.tile(np.arange(4), 32)[None]
    assert list(codec.pack_codes(c2, 2)[0]) == [0xE4E4E4E4] * 8
    c3 = np.tile(np.arange(8), 16)[None]
    assert list(codec.pack_codes(c3, 3)[0]) == [0xFBB26920, 0xFBB26920, 0xBBB2A9A0] * 4
    c3 = np.zeros((1, 64), np.int64)
    c3[0, 26], c3[0, 30], c3[0, 13] = 7, 5, 6
    assert list(codec.pack_codes(c3, 3)[0]) == [0x00C00000, 0x00403000, 0x00C00000, 0, 0, 0]
    s = np.zeros((1, 64), np.int64)
    s[0, 0] = s[0, 31] = 1
    s[0, 32 + 4] = 1
    assert list(codec.pack_signs(s)[0]) == [0x80000001, 0x10]


def _cb(d, bits, m, dense=False, seed=0):
    sigma, rg, sk = codec_draws(d, m, dense, seed)
    return codec.make_codebook(d, bits, m, dense, sigma, rg, sk)


def test_zero_vector_record():
    """nu = 0 gives u = 0, so every coordinate sits on the middle threshold
    (exactly 0) and takes code K/2; gamma = sqrt(d) t_{K/2}; S e follows."""
    cb = _cb(64, 3, 64)
    enc = codec.encode(cb, np.zeros((2, 64)))
    assert np.all(enc.norm == 0)
    assert np.all(enc.code_idx == 4)
    np.testing.assert_allclose(enc.rnorm, np.sqrt(64) * abs(float(cb.t32[4])), rtol=1e-12)


def test_encode_is_scale_invariant_and_norm_is_exact():
    cb = _cb(128, 3, 64)
    x = np.random.default_rng(3).standard_normal((50, 128))
    a, b = codec.encode(cb, x), codec.encode(cb, 8.0 * x)
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_array_equal(a.signs, b.signs)
    np.testing.assert_allclose(b.norm, 8 * np.linalg.norm(x, axis=1), rtol=1e-14)


def test_brute_force_nearest_codeword_tiny_d():
    """At d = 4, b = 2 the per-coordinate codes are the nearest point of the
    whole product codebook {t}^4 to y, found by enumerating all 256 points."""
    cb = _cb(4, 2, 32)
    x = np.random.default_rng(4).standard_normal((40, 4))
    enc = codec.encode(cb, x)
    t = cb.t32.astype(np.float64)
    pts = np.array(list(itertools.product(range(4), repeat=4)))
    for n in range(len(x)):
        dist = ((t[pts] - enc.y[n][None, :]) ** 2).sum(1)
        best = np.argsort(dist)[:2]
        if dist[best[1]] - dist[best[0]] > 1e-9:
            np.testing.assert_array_equal(enc.code_idx[n], pts[best[0]])


def test_rotated_coordinates_follow_the_table_density():
    """After normalise-and-rotate with a Haar rotation, the share of
    coordinates in each cell matches the cell masses of the marginal law
    (FibQuant summary, section 2.1: the canonical source)."""
    d, bits = 64, 2
    cb = _cb(d, bits, 0, dense=True, seed=9)
    x = np.random.default_rng(11).standard_normal((4000, d)) * np.linspace(0.1, 30, d)
    enc = codec.encode(cb, x)
    frac = np.bincount(enc.code_idx.ravel(), minlength=4) / enc.code_idx.size
    tau = cb.tau32.astype(np.float64)
    cdf = lloyd_max.marginal_cdf(np.concatenate([[-1], tau, [1]]), d)
    # a single fixed rotation and one set of inputs: allow sampling noise
    np.testing.assert_allclose(frac, np.diff(cdf), atol=0.03)


def test_record_sizes_reproduce_the_pages_memory_figures():
    """Closed-form layout arithmetic against the figures the pages print
    (tests/golden/pages_memory_figures.txt)."""
    figs = {}
    with open(os.path.join(GOLDEN, "pages_memory_figures.txt")) as f:
        for line in f:
            if not line.startswith("#") and line.strip():
                name, val, unit, _ = [p.strip() for p in line.split("|")]
                figs[name] = float(val)
    # ESM-2 650M: 33 layers, 20 heads x 64 = 1280 wide, K and V, fp32
    fp32 = 33 * 2 * 1024 * 1280 * 4
    assert round(fp32 / 2 ** 20) == figs["esm2_650m_fp32_kv_1024_tokens"]
    # 3-bit codes + one sign bit per element + fp32 norm, per 64-wide head
    rec = codec.record_bytes(64, 3, 64, with_rnorm=False)
    assert rec == 36
    comp = 33 * 2 * 1024 * 20 * rec
    assert abs(comp / 2 ** 20 - figs["turboesm_compressed_kv"]) < 1.0
    assert round(fp32 / comp, 1) == figs["turboesm_reduction"]
    # Llama-70B: 80 layers, 8 KV heads of 128, K and V, bf16, 1e6 tokens
    llama = 80 * 2 * 8 * 128 * 2 * 10 ** 6
    assert round(llama / 1e9) == figs["llama70b_bf16_kv_1m_tokens"]


def test_reconstruct_is_unbiased_over_sketches():
    """Averaging the decoder's vector estimate over many independent sketch
    matrices recovers x (the QJL term removes the quantiser's error in
    expectation)."""
    d, bits, m = 32, 2, 64
    g = np.random.default_rng(12)
    sigma = np.where(g.integers(0, 2, d) == 1, 1, -1)
    x = g.standard_normal((1, d))
    acc = np.zeros(d)
    n = 3000
    for _ in range(n):
        cb = codec.make_codebook(d, bits, m, False, sigma, None, g.standard_normal((m, d)).astype(np.float32))
        acc += codec.reconstruct(cb, codec.encode(cb, x))[0]
    err = np.linalg.norm(acc / n - x[0]) / np.linalg.norm(x)
    assert err < 0.03, err
    cb0 = codec.make_codebook(d, bits, 0, False, sigma, None, None)
    bias = np.linalg.norm(codec.reconstruct(cb0, codec.encode(cb0, x))[0] - x[0]) / np.linalg.norm(x)
    assert bias > 0.1
