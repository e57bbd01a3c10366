"""FibQuant k-dimensional codebooks (oracle side).

Source: FibQuant summary ("FibQuant: Quantizacao Vetorial Universal para
Compressao de KV-Cache de Acesso Aleatorio").
* Section 2.1: after the norm is removed and a Haar rotation applied, the
  unit vector is uniform on S^{d-1}, so a block of k consecutive coordinates
  follows one spherical-Beta law f_{d,k} on the unit ball B^k, whatever the
  input; one offline codebook serves every layer, head and input.
* Section 2.2: the shared codebook combines radii matched to the source's
  radial density by Bennett-Gersho companding (closed form with Beta
  quantiles for k = 2), near-uniform directions (k = 2: the planar Fibonacci
  spiral, the golden quantiser; k = 3: the Fibonacci sphere), and a Lloyd-Max
  refinement with several restarts that lowers the mean squared error for
  the finite size N.
* Section 2.3: the encoder stores nu = ||x||, rotates x / nu, cuts it into
  d/k blocks of k coordinates and stores the nearest codeword of each; the
  decoder looks the codewords up, concatenates them, rotates back and scales
  by nu.  The rate is b = log2(N) / k bits per coordinate, so fractional and
  below-one-bit rates exist.

Readings where the page is silent:
* f_{d,k}(x) is proportional to (1 - |x|^2)^((d-k-2)/2) on B^k, and |x|^2
  follows Beta(k/2, (d-k)/2).  Bennett-Gersho companding puts codewords with
  density proportional to f^(k/(k+2)); its radial law has |x|^2 ~
  Beta(k/2, a + 1) with a = k (d-k-2) / (2 (k+2)), and codeword n of N takes
  the squared radius at quantile (n + 1/2) / N of that law.
* Directions: k = 2, angle n * 2 pi / phi^2 (the golden angle) for the n-th
  radius (Vogel's spiral with companded radii); k = 3, the Fibonacci sphere
  z_n = 1 - 2 (n + 1/2) / N, longitude n times the golden angle, with the
  radius of quantile frac((n + 1/2) / phi) so that radius and height are
  not tied together.
* Lloyd-Max runs on a deterministic equal-mass sample of f_{d,k}: R radii at
  the quantiles (i + 1/2) / R of the radial law times the directions (k = 2:
  A angles 2 pi (j + 1/2) / A; k = 3: an A-point Fibonacci sphere and its
  A antipodes), all of equal weight.  Each iteration assigns every sample point to its nearest
  codeword (ties to the smaller index) and moves each codeword to the mean
  of its points (an empty cell keeps its codeword), until no assignment
  changes.  Restart r rotates the initial codebook by 2 pi r / (R_s N) in the
  plane of the first two axes (R_s restarts); the restart with the lowest
  mean squared error on the sample wins (within 1e-9 relative, the lower r).
* The stored codebook is float32; nearest-codeword decisions are taken in
  float32 like every other decision of the codec.
* Record: nu (float32) and d/k indices of log2(N) bits, index j at bits
  [j log2 N, (j+1) log2 N) of the LSB-first bit string of the record's
  words.

Pinned by tests: the sample's radial law against Monte Carlo points on the
sphere and its exact second moment; N = 2 against the closed form +-E|Y|;
Lloyd fixed points checked by brute-force nearest codewords; the vector
code's distortion below the scalar Lloyd-Max table's at equal rate (the
page's claim of strict dominance); the rate arithmetic; logits against the
decoder's rebuilt vectors; attention against textbook softmax attention over
the rebuilt keys and values.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
from scipy import special

PHI = (1.0 + math.sqrt(5.0)) / 2.0
GOLDEN_ANGLE = 2.0 * math.pi / (PHI * PHI)


def radial_quantiles(levels: np.ndarray, k: int, beta_b: float) -> np.ndarray:
    """Radii whose squares sit at the given quantile levels of Beta(k/2, beta_b)."""
    return np.sqrt(special.betaincinv(k / 2.0, beta_b, np.asarray(levels, np.float64)))


def fibonacci_sphere(n: int) -> np.ndarray:
    """n near-uniform unit vectors in R^3 [n, 3]."""
    i = np.arange(n, dtype=np.float64)
    z = 1.0 - 2.0 * (i + 0.5) / n
    rho = np.sqrt(np.maximum(0.0, 1.0 - z * z))
    th = i * GOLDEN_ANGLE
    return np.stack([rho * np.cos(th), rho * np.sin(th), z], axis=1)


def initial_codebook(d: int, k: int, N: int) -> np.ndarray:
    """Bennett-Gersho radii with Fibonacci directions, float64 [N, k]."""
    a = k * (d - k - 2) / (2.0 * (k + 2))
    n = np.arange(N, dtype=np.float64)
    if k == 2:
        r = radial_quantiles((n + 0.5) / N, 2, a + 1.0)
        th = n * GOLDEN_ANGLE
        return np.stack([r * np.cos(th), r * np.sin(th)], axis=1)
    if k == 3:
        lv = np.mod((n + 0.5) / PHI, 1.0)
        r = radial_quantiles(lv, 3, a + 1.0)
        return r[:, None] * fibonacci_sphere(N)
    raise ValueError("codebooks are built for k = 2 and 3")


def source_sample(d: int, k: int, n_radii: int = 64, n_dirs: int = 256) -> np.ndarray:
    """Equal-mass deterministic sample of f_{d,k}: [n_radii * n_dirs, k]."""
    r = radial_quantiles((np.arange(n_radii) + 0.5) / n_radii, k, (d - k) / 2.0)
    if k == 2:
        th = 2.0 * math.pi * (np.arange(n_dirs) + 0.5) / n_dirs
        u = np.stack([np.cos(th), np.sin(th)], axis=1)
    elif k == 3:
        # an n_dirs-point Fibonacci sphere and its antipodes (the law is symmetric)
        f = fibonacci_sphere(n_dirs)
        u = np.concatenate([f, -f])
    else:
        raise ValueError("codebooks are built for k = 2 and 3")
    return (r[:, None, None] * u[None, :, :]).reshape(-1, k)


def rotate_last_axis(c: np.ndarray, angle: float) -> np.ndarray:
    """Rotation by `angle` in the plane of the first two coordinates (k = 2:
    the plane; k = 3: about the z axis)."""
    ca, sa = math.cos(angle), math.sin(angle)
    out = c.copy()
    out[:, 0] = ca * c[:, 0] - sa * c[:, 1]
    out[:, 1] = sa * c[:, 0] + ca * c[:, 1]
    return out


def nearest(points: np.ndarray, code: np.ndarray) -> np.ndarray:
    """Index of the nearest codeword of each point (ties to the smaller
    index): squared distances summed coordinate by coordinate."""
    dist = np.zeros((len(points), len(code)))
    for i in range(points.shape[1]):
        diff = points[:, i:i + 1] - code[None, :, i]
        dist = dist + diff * diff
    return np.argmin(dist, axis=1)


def lloyd(points: np.ndarray, code: np.ndarray, max_iter: int = 5000):
    """Lloyd-Max on equal-weight points from `code`: (codebook, mse).  A
    cell's mean is its points' sum (in point order) over their count."""
    code = code.copy()
    N, k = code.shape
    assign = None
    for _ in range(max_iter):
        new = nearest(points, code)
        if assign is not None and np.array_equal(new, assign):
            break
        assign = new
        cnt = np.bincount(assign, minlength=N)
        for i in range(k):
            s = np.bincount(assign, weights=points[:, i], minlength=N)
            code[cnt > 0, i] = s[cnt > 0] / cnt[cnt > 0]
    else:
        raise RuntimeError("Lloyd iteration did not settle")
    diff = points - code[assign]
    return code, float((diff * diff).sum(axis=1).mean())


def build_codebook(d: int, k: int, N: int, restarts: int = 4, n_radii: int = 64, n_dirs: int = 256):
    """The refined codebook (float64 [N, k]) and its per-block MSE on the
    sample.  A later restart replaces the best so far only when its MSE is
    lower by more than 1e-9 relative (rotated copies of one optimum tie)."""
    pts = source_sample(d, k, n_radii, n_dirs)
    init = initial_codebook(d, k, N)
    best = None
    for r in range(restarts):
        c0 = rotate_last_axis(init, 2.0 * math.pi * r / (restarts * N))
        c, mse = lloyd(pts, c0)
        if best is None or mse < best[1] * (1.0 - 1e-9):
            best = (c, mse)
    return best


@dataclasses.dataclass
class VQCodebook:
    d: int
    k: int
    N: int
    code32: np.ndarray     # [N, k] float32 codewords
    pi: np.ndarray         # [d, d] float64 rotation

    @property
    def index_bits(self) -> int:
        return int(round(math.log2(self.N)))

    @property
    def rate(self) -> float:
        """Bits per coordinate, log2(N) / k."""
        return math.log2(self.N) / self.k

    def words(self) -> int:
        return (self.d // self.k * self.index_bits + 31) // 32


def make_vq_codebook(d: int, k: int, N: int, sigma, code=None, restarts: int = 4) -> VQCodebook:
    """A codebook with the RHT of signs sigma; `code` gives the codewords
    (else they are built here)."""
    from .rotation import rht_matrix
    if code is None:
        code, _ = build_codebook(d, k, N, restarts)
    return VQCodebook(d, k, N, np.asarray(code, np.float64).astype(np.float32), rht_matrix(np.asarray(sigma)))


@dataclasses.dataclass
class VQEncoded:
    norm: np.ndarray      # [n] float64
    codes: np.ndarray     # [n, words] uint32
    y: np.ndarray         # [n, d] rotated unit vectors
    idx: np.ndarray       # [n, d/k] codeword indices
    margin: np.ndarray    # [n, d/k] second-nearest minus nearest squared distance (float64)


def pack_indices(idx: np.ndarray, bits: int) -> np.ndarray:
    n, nb = idx.shape
    words = np.zeros((n, (nb * bits + 31) // 32), np.uint64)
    for j in range(nb):
        for b in range(bits):
            pos = j * bits + b
            words[:, pos // 32] |= ((idx[:, j].astype(np.uint64) >> np.uint64(b)) & np.uint64(1)) << np.uint64(pos % 32)
    return words.astype(np.uint32)


def unpack_indices(words: np.ndarray, bits: int, nb: int) -> np.ndarray:
    w = np.asarray(words).astype(np.uint64)
    out = np.zeros((w.shape[0], nb), np.int64)
    for j in range(nb):
        for b in range(bits):
            pos = j * bits + b
            out[:, j] |= ((w[:, pos // 32] >> np.uint64(pos % 32)) & np.uint64(1)).astype(np.int64) << b
    return out


def encode(cb: VQCodebook, x: np.ndarray, pos=None, rope=None) -> VQEncoded:
    """nu, rotate, cut into d/k blocks, nearest codeword of each block
    (decided in float32 against the float32 codewords)."""
    from .rope import apply_rope
    x = np.asarray(x, np.float64)
    if rope is not None:
        x = apply_rope(x, pos, rope[0], rope[1])
    nu = np.sqrt((x * x).sum(1))
    safe = np.where(nu > 0, nu, 1.0)
    u = np.where(nu[:, None] > 0, x / safe[:, None], 0.0)
    y = u @ cb.pi.T
    nb = cb.d // cb.k
    blocks = y.reshape(-1, cb.k).astype(np.float32).astype(np.float64)
    c = cb.code32.astype(np.float64)
    dist = np.zeros((len(blocks), cb.N))
    for i in range(cb.k):
        diff = blocks[:, i:i + 1] - c[None, :, i]
        dist = dist + diff * diff
    idx = np.argmin(dist, axis=1)
    srt = np.sort(dist, axis=1)
    margin = srt[:, 1] - srt[:, 0] if cb.N > 1 else np.full(len(blocks), np.inf)
    idx = idx.reshape(-1, nb)
    return VQEncoded(nu, pack_indices(idx, cb.index_bits), y, idx, margin.reshape(-1, nb))


def reconstruct(cb: VQCodebook, norm: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """The decoder: codewords looked up and concatenated, rotated back, scaled
    by nu (float64 [n, d])."""
    nb = cb.d // cb.k
    idx = unpack_indices(codes, cb.index_bits, nb)
    yhat = cb.code32.astype(np.float64)[idx].reshape(len(idx), cb.d)
    return np.asarray(norm, np.float64)[:, None] * (yhat @ cb.pi)


def logits(cb: VQCodebook, qp: np.ndarray, norm: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """[G, n] logits nu * sum_j <q'_j, c[idx_j]> of prepared queries q' = Pi q
    [G, d] against n records."""
    nb = cb.d // cb.k
    idx = unpack_indices(codes, cb.index_bits, nb)
    yhat = cb.code32.astype(np.float64)[idx].reshape(len(idx), cb.d)
    return (np.asarray(norm, np.float64)[:, None] * (yhat @ np.asarray(qp, np.float64).T)).T


def attention(ck: VQCodebook, cv: VQCodebook, qp: np.ndarray, knorm: np.ndarray, kcodes: np.ndarray,
              vnorm: np.ndarray, vcodes: np.ndarray, scale: float) -> np.ndarray:
    """Attention of prepared queries q' = Pi_k RoPE(q) [G, d] over n
    vector-coded keys and values (float64 [G, d]): softmax over scale times
    the logits, then the weighted sum of the decoded values (section 2.3's
    decoder; section 5 asks for decompression fused with attention).  No keys
    give zeros."""
    qp = np.asarray(qp, np.float64)
    if len(knorm) == 0:
        return np.zeros((qp.shape[0], cv.d))
    a = scale * logits(ck, qp, knorm, kcodes)
    a = a - a.max(axis=1, keepdims=True)
    w = np.exp(a)
    w /= w.sum(axis=1, keepdims=True)
    return w @ reconstruct(cv, vnorm, vcodes)
