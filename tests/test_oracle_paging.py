"""Pins for the oracle's growing-cache layouts (CPU only): the contiguous
layout as a special case of the paged one, the paged map being one to one,
and token-by-token appends agreeing with a bulk encode."""
import numpy as np
import pytest

from oracle import codec, paging, rope as orope


def test_one_page_per_sequence_is_the_contiguous_layout():
    B, H, L = 3, 4, 96
    pages = np.arange(B)[:, None]
    b, h, t = np.meshgrid(np.arange(B), np.arange(H), np.arange(L), indexing="ij")
    np.testing.assert_array_equal(paging.paged_index(pages, L, H, b, h, t),
                                  paging.contiguous_index(b, h, t, H, L))
    # and by hand: record of (b=2, head=1, t=5) = (2*4 + 1)*96 + 5
    assert paging.contiguous_index(2, 1, 5, H, L) == 869


@pytest.mark.parametrize("seed", range(3))
def test_paged_map_is_one_to_one(seed):
    """Distinct physical pages give distinct records for every (b, head, t),
    all inside the pool, and a page's P slots of one head are consecutive."""
    g = np.random.default_rng(seed)
    B, H, P, J = 5, 3, 64, 7
    n_pages = B * J + 4
    pages = g.permutation(n_pages)[:B * J].reshape(B, J)
    b, h, t = np.meshgrid(np.arange(B), np.arange(H), np.arange(J * P), indexing="ij")
    idx = paging.paged_index(pages, P, H, b, h, t).ravel()
    assert len(np.unique(idx)) == idx.size
    assert idx.min() >= 0 and idx.max() < n_pages * H * P
    one = paging.paged_index(pages, P, H, 2, 1, np.arange(3 * P, 4 * P))
    np.testing.assert_array_equal(np.diff(one), 1)
    assert one[0] == (pages[2, 3] * H + 1) * P


@pytest.mark.parametrize("correction", ["qjl", "sign"])
def test_token_by_token_appends_equal_a_bulk_encode(correction):
    """Appending T tokens one per step (per-sequence lengths differ, RoPE at
    each token's own slot) leaves the records a single encode of the whole
    sequences writes."""
    g = np.random.default_rng(4)
    B, H, d, T, P = 2, 3, 64, 70, 64
    if correction == "sign":
        cb = codec.make_sign_codebook(d, 3, "hadamard", seed=2)
    else:
        cb = codec.make_codebook(d, 3, 32, False, seed=2)
    cos, sin = orope.rope_table(1e4, d, 256)
    x = g.standard_normal((B, T, H, d))
    start = np.array([0, 9])          # sequence 1 already holds 9 tokens
    pages = np.array([[3, 0], [1, 2]])
    index_of = lambda b, h, t: paging.paged_index(pages, P, H, b, h, t)
    pool = paging.empty_pool(cb, 4 * H * P)
    for step in range(T):
        paging.append(cb, pool, x[:, step], start + step, index_of, rope=(cos, sin))
    for b in range(B):
        for h in range(H):
            t = start[b] + np.arange(T)
            bulk = codec.encode(cb, x[b, :, h], pos=t, rope=(cos, sin))
            got = paging.gather(pool, index_of(b, h, t))
            np.testing.assert_array_equal(got.codes, bulk.codes)
            np.testing.assert_array_equal(got.signs, bulk.signs)
            np.testing.assert_allclose(got.norm, bulk.norm, rtol=1e-15)
    # slots before sequence 1's start were never written
    assert not pool["norm"][index_of(1, 0, np.arange(9))].any()
