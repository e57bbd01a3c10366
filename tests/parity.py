"""Helpers for GPU-vs-oracle parity tests (imported by the gpu tests).

Protocol:
* codes: bit-exact except coordinates whose oracle value y lies within 1e-5
  of a threshold; at most 1e-6 of the remaining coordinates may differ.
* sign bits: the oracle's residual is recomputed under the GPU's codes (on a
  boundary coordinate both codes are correct); bits must then match except
  where |(S e)_l| < 1e-5, again at a rate of at most 1e-6.
* nu and gamma: relative error <= 1e-5 (gamma under the GPU's codes); a sum of
  d = 128 float32 squares carries at most d * 2^-24 ~ 7.6e-6 relative error.
  Sign-corrected records (S = I) store no gamma; their sign bits follow the
  same rule with S e = e.
* logits and decode outputs: both sides read the same (oracle-encoded)
  packed cache; |gpu - ref| <= 1e-4 + 1e-3 |ref| per element.
"""
from __future__ import annotations

import numpy as np

from oracle import codec

BOUNDARY = 1e-5
RATE = 1e-6
RTOL, ATOL = 1e-3, 1e-4


def oracle_rows(x):
    """[n_seq, n_tok, h, d] -> rows in record order (seq, head, token)."""
    return np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)).reshape(-1, x.shape[-1]))


def compare_encoded(cb: codec.Codebook, enc: codec.Encoded, gpu, label=""):
    """gpu = (norm, rnorm, codes u32, signs u32) for the same rows as enc."""
    g_norm, g_rnorm, g_codes, g_signs = gpu
    n = len(enc.norm)
    y = enc.y
    g_ci = codec.unpack_codes(g_codes, cb.bits, cb.d)
    near = (np.abs(y[..., None] - cb.tau32.astype(np.float64)[None, None, :]) < BOUNDARY).any(-1)
    bad = (g_ci != enc.code_idx) & ~near
    allowed = int(RATE * (~near).sum())
    assert bad.sum() <= allowed, f"{label}: {bad.sum()} code mismatches off the boundary (allowed {allowed})"
    np.testing.assert_allclose(g_norm, enc.norm, rtol=1e-5, atol=1e-30, err_msg=f"{label}: norm")
    if cb.m:
        e_g, gam_g, se_g = codec.residual_and_sketch(cb, y, g_ci)
        bits_o = (se_g.astype(np.float32) >= 0)
        bits_g = codec.unpack_signs(g_signs, cb.m).astype(bool)
        near_s = np.abs(se_g) < BOUNDARY
        bad_s = (bits_g != bits_o) & ~near_s
        allowed_s = int(RATE * (~near_s).sum())
        assert bad_s.sum() <= allowed_s, f"{label}: {bad_s.sum()} sign mismatches (allowed {allowed_s})"
        if cb.correction == "qjl":
            np.testing.assert_allclose(g_rnorm, gam_g, rtol=1e-5, atol=1e-12, err_msg=f"{label}: rnorm")
        else:
            assert g_rnorm.size == 0, f"{label}: a sign-corrected record has no rnorm plane"
    return {"n": n, "boundary_coords": int(near.sum()), "code_mismatch": int(bad.sum())}


def assert_close(gpu, ref, label=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    lim = ATOL + RTOL * np.abs(ref)
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(f"{label}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu {gpu[i]!r} ref {ref[i]!r}")


def check_topk(vals, idx, ref_scores, k, label=""):
    """A GPU top-k against the oracle's scores of the same rows.

    vals, idx: [rows, k] from the GPU; ref_scores: [rows, n] oracle scores of
    every candidate.  Per row: the min(k, n) leading indices are distinct and
    in range, the values descend (equal values by ascending index), each value
    matches the oracle's score at its index, and each returned index scores no
    worse than the oracle's k-th best less the tolerance (near-ties at the
    cut may pick either key, and both answers are correct).  Slots past n
    hold index -1 and value -inf."""
    vals = np.asarray(vals)
    idx = np.asarray(idx)
    ref_scores = np.asarray(ref_scores, np.float64)
    n = ref_scores.shape[1]
    kk = min(k, n)
    for g in range(len(vals)):
        ii = idx[g, :kk]
        assert len(set(ii.tolist())) == kk, f"{label} row {g}: repeated indices {ii}"
        assert ii.min() >= 0 and ii.max() < n, f"{label} row {g}: index out of range {ii}"
        v = vals[g, :kk]
        assert np.all(np.diff(v) <= 0), f"{label} row {g}: values not descending {v}"
        tie = np.diff(v) == 0
        assert np.all(np.diff(ii)[tie] > 0), f"{label} row {g}: equal values not in index order"
        assert_close(v, ref_scores[g, ii], f"{label} top-k values row {g}")
        kth = np.partition(ref_scores[g], n - kk)[n - kk]
        assert np.all(ref_scores[g, ii] >= kth - (ATOL + RTOL * abs(kth))), f"{label} row {g}: below the k-th best"
        if kk < k:
            assert np.all(idx[g, kk:] == -1) and np.all(np.isneginf(vals[g, kk:])), f"{label} row {g}: padding"
