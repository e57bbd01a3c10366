"""Shared random rotations, as explicit d x d matrices (oracle side).

* Randomized Hadamard transform (iaemfoco post, "TurboQuant: Uma Nova
  Abordagem"): Pi = H diag(sigma) / sqrt(d), with H the Sylvester-ordered
  Hadamard matrix, H[i, j] = (-1)^popcount(i & j), and sigma a vector of
  random signs.  One round (the post names a single transform).
* Haar rotation (FibQuant summary, section 1 and 2.1: a shared random
  orthogonal Haar rotation): the Q factor of the QR factorisation of a
  matrix of i.i.d. N(0,1) draws, with its columns' signs chosen so that R has
  a positive diagonal (that choice makes Q Haar-distributed and unique).

Pinned by tests: orthogonality, norm and inner-product preservation, H
against scipy.linalg.hadamard and against its Kronecker construction, every
entry of Pi e_j being +-1/sqrt(d), and G = Q R with R upper triangular with a
positive diagonal.
"""
from __future__ import annotations

import numpy as np


def sylvester_hadamard(d: int) -> np.ndarray:
    if d < 1 or d & (d - 1):
        raise ValueError("Hadamard size must be a power of two")
    i = np.arange(d)
    parity = np.zeros((d, d), dtype=np.int64)
    a = i[:, None] & i[None, :]
    while np.any(a):
        parity ^= a & 1
        a = a >> 1
    return np.where(parity == 1, -1.0, 1.0)


def rht_matrix(sigma: np.ndarray) -> np.ndarray:
    """Pi = H diag(sigma) / sqrt(d), float64."""
    d = len(sigma)
    return sylvester_hadamard(d) * np.asarray(sigma, np.float64)[None, :] / np.sqrt(d)


def haar_rotation(gauss: np.ndarray) -> np.ndarray:
    """Q of G = Q R with diag(R) > 0, float64."""
    q, r = np.linalg.qr(np.asarray(gauss, np.float64))
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return q * s[None, :]
