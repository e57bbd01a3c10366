"""Rotary position embedding, applied before the codec's rotation (oracle side).

Source: TurboESM summary, technical section 2 (the RoPE-invariant orthogonal
pipeline: RoPE first, then the orthogonal rotation Pi; since Pi^T Pi = I the
attention score is preserved exactly) and its section 3, contribution 1.

The pages do not fix RoPE's pairing or frequencies; the reading used here is
the common half-split form: for i < d/2 the pair (x_i, x_{i+d/2}) is rotated
by the angle pos * base^(-2i/d).  Angles and their cosines and sines are
computed in float64 and stored as a float32 table [pos][d/2]; every consumer
rotates with the float32 table values.

Pinned by tests: the frequencies against closed-form cases of the RoFormer
definition (Su et al., 2021: a geometric sequence from 1 rad per position down
towards 1/base; at d = 8, base 1e4 the angles per position are exactly 1, 0.1,
0.01 and 0.001, and pair d/4 always turns by base^(-1/2)); rotation by
position 0 is the identity; norms are kept; <R_a q, R_b k> = <q, R_{b-a} k>;
RoPE then Pi keeps logits exactly while Pi then RoPE does not.
"""
from __future__ import annotations

import numpy as np


def rope_table(base: float, d: int, n_pos: int):
    """(cos, sin), each float32 [n_pos, d/2]."""
    half = d // 2
    theta = np.power(float(base), -2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def apply_rope(x: np.ndarray, pos: np.ndarray, cos32: np.ndarray, sin32: np.ndarray) -> np.ndarray:
    """Rotate rows of x [n, d] (float64) by their positions pos [n]."""
    x = np.asarray(x, np.float64)
    half = x.shape[1] // 2
    c = cos32[np.asarray(pos)].astype(np.float64)
    s = sin32[np.asarray(pos)].astype(np.float64)
    lo, hi = x[:, :half], x[:, half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=1)
