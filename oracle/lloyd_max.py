"""Lloyd-Max scalar table for one coordinate of a normalised, rotated vector.

Source: FibQuant summary, section 2.1 (after the norm is removed and a Haar
rotation applied, the unit vector is uniform on the sphere S^{d-1}, so a
block of k coordinates follows the spherical-Beta law f_{d,k}; one offline
table serves every layer, head and input) and section 1 (each rotated
coordinate is quantised independently with a scalar Lloyd-Max table); itstec
post, "Por dentro do processo de compressao KV" (each coordinate follows a
concentrated Beta law).  For k = 1 the law is

    f_d(y) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1 - y^2)^((d-3)/2),  |y| < 1,

equivalently (1 + y)/2 ~ Beta((d-1)/2, (d-1)/2).

A K = 2^b level Lloyd-Max quantiser satisfies two conditions at its optimum:
every threshold is the midpoint of its neighbouring levels, and every level
is the conditional mean of the density over its cell.  The oracle iterates
the two conditions from quantile starting levels until the levels stop
moving.  The density is even, so each iterate is symmetrised (t_j = -t_{K-1-j});
this makes the middle threshold exactly 0 for every b.

Pinned by tests: residuals of both conditions under an independent
quadrature; d = 3 (uniform marginal, so the uniform quantiser); b = 1
(levels +-E|Y| in closed form); large d (sqrt(d) t tends to the Gaussian
Lloyd-Max table printed in Max, 1960); the density against Monte Carlo
samples on the sphere; nearest-level brute force.
"""
from __future__ import annotations

import numpy as np
from scipy import special


def _log_norm_const(d: int) -> float:
    return special.gammaln(d / 2.0) - 0.5 * np.log(np.pi) - special.gammaln((d - 1) / 2.0)


def marginal_pdf(y, d: int):
    """Density of one coordinate of a uniform point on S^{d-1} (d >= 3)."""
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros_like(y)
    inside = np.abs(y) < 1.0
    yy = y[inside]
    out[inside] = np.exp(_log_norm_const(d) + 0.5 * (d - 3) * np.log1p(-yy * yy))
    return out


def marginal_sf(y, d: int):
    """P(Y > y) through the regularised incomplete beta function."""
    a = 0.5 * (d - 1)
    x = np.clip((1.0 - np.asarray(y, dtype=np.float64)) / 2.0, 0.0, 1.0)
    return special.betainc(a, a, x)


def marginal_cdf(y, d: int):
    a = 0.5 * (d - 1)
    x = np.clip((1.0 + np.asarray(y, dtype=np.float64)) / 2.0, 0.0, 1.0)
    return special.betainc(a, a, x)


def _upper_tail_moment(y, d: int):
    """Integral of t f_d(t) over [y, 1] for y in [0, 1]:
    C (1 - y^2)^(alpha+1) / (2 (alpha+1)),  alpha = (d-3)/2."""
    y = np.asarray(y, dtype=np.float64)
    ap1 = 0.5 * (d - 1)
    out = np.zeros_like(y)
    inside = y < 1.0
    yy = y[inside]
    out[inside] = np.exp(_log_norm_const(d) + ap1 * np.log1p(-yy * yy) - np.log(2.0 * ap1))
    return out


def centroids_for_thresholds(tau: np.ndarray, d: int) -> np.ndarray:
    """Conditional means of f_d over the cells cut by ``tau`` (symmetric,
    ascending, K-1 entries).  Cells in the upper half are integrated directly
    with the survival function and the closed-form first moment; the lower
    half mirrors them, since f_d is even."""
    K = len(tau) + 1
    half = K // 2
    lo = np.concatenate([tau[half - 1:], []])            # tau_{K/2-1} = 0 ... tau_{K-2}
    hi = np.concatenate([tau[half:], [1.0]])
    mass = marginal_sf(lo, d) - marginal_sf(hi, d)
    mom = _upper_tail_moment(lo, d) - _upper_tail_moment(hi, d)
    upper = mom / mass
    return np.concatenate([-upper[::-1], upper])


def lloyd_max(d: int, bits: int, max_iter: int = 1_000_000):
    """Converged float64 (levels t [K], thresholds tau [K-1]) for f_d.

    Iterates until the levels stop moving: a relative step below 1e-14, or a
    step below 1e-12 that no longer shrinks (the floor set by the incomplete
    beta function's own rounding, a few units of 1e-15)."""
    if d < 3:
        raise ValueError("the sphere marginal needs d >= 3")
    K = 1 << bits
    a = 0.5 * (d - 1)
    # starting levels: the quantiles (j + 1/2)/K of the marginal
    t = 2.0 * special.betaincinv(a, a, (np.arange(K) + 0.5) / K) - 1.0
    t = 0.5 * (t - t[::-1])
    prev = np.inf
    for _ in range(max_iter):
        tau = 0.5 * (t[:-1] + t[1:])
        t_new = centroids_for_thresholds(tau, d)
        t_new = 0.5 * (t_new - t_new[::-1])
        step = np.max(np.abs(t_new - t)) / np.max(np.abs(t_new))
        t = t_new
        if step <= 1e-14 or (step <= 1e-12 and step >= prev):
            break
        prev = step
    else:
        raise RuntimeError("Lloyd-Max iteration did not converge")
    tau = 0.5 * (t[:-1] + t[1:])
    return t, tau


def table_f32(d: int, bits: int):
    """The table as the codec stores it: levels and thresholds rounded to
    float32.  Every later step uses these float32 values."""
    t, tau = lloyd_max(d, bits)
    return t.astype(np.float32), tau.astype(np.float32)


def distortion(t: np.ndarray, tau: np.ndarray, d: int) -> float:
    """E[(Y - Q(Y))^2] of a table under f_d, by adaptive quadrature."""
    from scipy import integrate
    edges = np.concatenate([[-1.0], np.asarray(tau, np.float64), [1.0]])
    s = 0.0
    for j in range(len(t)):
        f = lambda y, c=float(t[j]): (y - c) ** 2 * marginal_pdf(np.array([y]), d)[0]
        s += integrate.quad(f, edges[j], edges[j + 1], limit=200, epsabs=1e-15, epsrel=1e-12)[0]
    return s


def mean_abs_error(t: np.ndarray, tau: np.ndarray, d: int) -> float:
    """E|Y - Q(Y)| of a table under f_d (adaptive quadrature, each cell split
    at its level so the integrand is smooth on every piece).

    This is the data-oblivious value of the TurboESM correction's mean
    residual magnitude (TurboESM summary, technical section 2): for one
    coordinate, the constant a minimising E(e - a sign(e))^2 is E|e|."""
    from scipy import integrate
    t = np.asarray(t, np.float64)
    edges = np.concatenate([[-1.0], np.asarray(tau, np.float64), [1.0]])
    pdf = lambda y: marginal_pdf(np.array([y]), d)[0]
    s = 0.0
    for j in range(len(t)):
        lo, hi, c = edges[j], edges[j + 1], float(t[j])
        mid = min(max(c, lo), hi)
        if mid > lo:
            s += integrate.quad(lambda y: (c - y) * pdf(y), lo, mid, limit=200, epsabs=1e-15, epsrel=1e-12)[0]
        if hi > mid:
            s += integrate.quad(lambda y: (y - c) * pdf(y), mid, hi, limit=200, epsabs=1e-15, epsrel=1e-12)[0]
    return s
