"""Calibration of the TurboESM variant's tables (oracle side).

Source: TurboESM summary, technical section 2.  Keys and values keep
separate 8-entry Lloyd-Max tables (keys in the rotated space, values in
their original space), and the one-bit residual correction adds a
calibrated mean residual magnitude along each stored sign.  The pages
calibrate on real protein activations; here every calibration sample is a
seeded synthetic one.

Readings where the pages are silent:

* The table is fitted to a calibration sample by Lloyd's algorithm with a
  mirror-symmetric constraint: its upper half is the Lloyd-Max quantiser of
  |y| with K/2 levels (cells [0, b_1), [b_1, b_2), ..., [b_{K/2-1}, inf)),
  and the lower half mirrors it.  The rotated coordinates' law is symmetric,
  and the encoder's code arithmetic relies on a symmetric table.
* Starting levels: the order statistics a_(floor((j + 1/2) N / (K/2))) of the
  sorted |y| (N values); iterations stop when no sample changes cell; a cell
  that empties keeps its level.
* mu of a KV head is the mean of |y_i - t[c_i]| over that head's calibration
  vectors and coordinates (codes decided in float32 against the float32
  table, as the encoder decides them).  It is the constant a that minimises
  the mean of (e - a sign(e))^2, so it is the least-squares scale of the
  sign correction.
* Vectors with nu = 0 carry no direction and are left out.

Pinned by tests: a brute-force optimal partition of a tiny sample; the
uniform law (levels at the cell midpoints); large sphere samples against the
Beta-law Lloyd-Max table and its mean absolute error; the least-squares
property of mu by a scan over a.
"""
from __future__ import annotations

import numpy as np

from .rope import apply_rope


def unit_rotated(pi: np.ndarray, x: np.ndarray, pos=None, rope=None) -> np.ndarray:
    """y = Pi (RoPE(x) / nu) for the rows of x [n, d] with nu > 0, float64."""
    x = np.asarray(x, np.float64)
    if rope is not None:
        x = apply_rope(x, pos, rope[0], rope[1])
    nu = np.sqrt((x * x).sum(1))
    keep = nu > 0
    return (x[keep] / nu[keep, None]) @ np.asarray(pi, np.float64).T


def symmetric_lloyd(y: np.ndarray, bits: int, max_iter: int = 100_000) -> np.ndarray:
    """float64 symmetric table [K] fitted to the sample y (any shape)."""
    a = np.sort(np.abs(np.asarray(y, np.float64)).ravel())
    n = a.size
    half = (1 << bits) // 2
    if n == 0:
        raise ValueError("empty calibration sample")
    lv = a[[int(np.floor((j + 0.5) * n / half)) for j in range(half)]].copy()
    counts = None
    for _ in range(max_iter):
        b = 0.5 * (lv[:-1] + lv[1:])                     # upper-cell boundaries
        cell = (a[:, None] >= b[None, :]).sum(1)          # cell index of each |y|
        new_counts = np.bincount(cell, minlength=half)
        for j in range(half):
            if new_counts[j]:
                lv[j] = a[cell == j].mean()
        if counts is not None and np.array_equal(new_counts, counts):
            break
        counts = new_counts
    else:
        raise RuntimeError("Lloyd iteration did not settle")
    return np.concatenate([-lv[::-1], lv])


def quantise_f32(t32: np.ndarray, tau32: np.ndarray, y: np.ndarray) -> np.ndarray:
    """c = #{j : y >= tau_j}, decided in float32."""
    y32 = np.asarray(y, np.float64).astype(np.float32)
    return (y32[..., None] >= np.asarray(tau32, np.float32)).sum(-1)


def mean_residual_magnitude(t32: np.ndarray, tau32: np.ndarray, y: np.ndarray) -> float:
    """mean |y - t[c(y)]| over all entries of y (float64), 0 for no entries."""
    y = np.asarray(y, np.float64)
    if y.size == 0:
        return 0.0
    c = quantise_f32(t32, tau32, y)
    return float(np.abs(y - np.asarray(t32, np.float32).astype(np.float64)[c]).mean())


def calibrate(pi: np.ndarray, bits: int, x: np.ndarray, tok_offset: int = 0, rope=None):
    """(levels float32 [K], mu float32 [h]) from a calibration batch
    x [n_tok, h, d] (token t sits at position tok_offset + t for RoPE).

    The table is fitted to every head's rotated unit vectors together (one
    table per tensor); mu is taken per head with that table."""
    x = np.asarray(x, np.float64)
    n_tok, h, d = x.shape
    pos = tok_offset + np.arange(n_tok)
    ys = []
    for j in range(h):
        xj = x[:, j, :]
        if rope is not None:
            xj = apply_rope(xj, pos, rope[0], rope[1])
        ys.append(unit_rotated(pi, xj))
    t64 = symmetric_lloyd(np.concatenate([y.ravel() for y in ys]), bits)
    t32 = t64.astype(np.float32)
    tau32 = (0.5 * (t32[:-1].astype(np.float64) + t32[1:].astype(np.float64))).astype(np.float32)
    mu = np.array([mean_residual_magnitude(t32, tau32, y) for y in ys], np.float32)
    return t32, mu
