"""Encoder and record layout (oracle side).

Steps, in the order the pages give them (FibQuant summary, sections 1 and
2.3; iaemfoco post, "TurboQuant: Uma Nova Abordagem"; itstec post, "Por
dentro do processo de compressao KV"; TurboESM summary, technical section 2):

  1. RoPE on keys at their token positions (TurboESM: RoPE before Pi).
  2. Store the norm nu = ||x||_2 and take the unit vector u = x / nu
     (u = 0 when nu = 0).
  3. Rotate: y = Pi u with the shared rotation.
  4. Quantise each coordinate with the scalar Lloyd-Max table:
     c_i = #{j : y_i >= tau_j}; code 0 is the most negative level.
  5. Residual e = y - t[c], with norm gamma = ||e||_2.
  6. One-bit QJL sketch of the residual: bit_l = [(S e)_l >= 0] for an
     m x d Gaussian S.

TurboESM variant (TurboESM summary, technical section 2, the dual lookup
tables and the one-bit residual correction): ``correction = "sign"`` keeps
one sign bit per residual coordinate instead of a Gaussian sketch (S is the
identity, m = d): bit_i = [e_i >= 0].  No gamma is stored; the decoder adds a
per-head calibrated mean residual magnitude mu along those signs.  The table
may be a calibrated one (``levels``), and ``rotation = "none"`` leaves the
vectors in their original coordinates (the value table of that section).

Readings where the pages are silent: the sketch acts on the residual in the
rotated domain; gamma
is stored per vector as float32 next to nu; ties go to the upper code and a
zero sketch value gives bit 1.  Integer decisions (codes, sign bits) are
taken in float32, the precision the GPU kernels decide in: the float64 value
is rounded to float32 and compared with the float32 thresholds.

Fixed-address record (FibQuant summary, section 1): per vector n, planes
norm[n] f32, rnorm[n] f32 (absent when m = 0), codes[n][b*d/32] u32 and
signs[n][m/32] u32.  Sketch bit l is bit l%32 of sign word l//32.  Code bit
positions (bit k is bit k%32 of word k//32 of the record's code words):

* b = 1, 2, 4: coordinate i's code is bits [b*i, b*i+b), LSB first.
* b = 3: coordinates go in groups of 32 (96 bits, words 3g..3g+2, called
  W0, W1, W2).  Coordinate j < 24 of a group takes bits [8(j%4) + 3((j%8)//4),
  +3) of word W_{j//8}: every byte holds two whole codes.  For j = 24 + r,
  the low two bits sit at bits 8(r%4) + 6, +7 of W_{r//4} and the high bit
  at bit 8(r%4) + 6 + r//4 of W2.  The pages fix only that records have
  fixed addresses; this order lets a byte-wise mask recover four codes at
  once.
"""
from __future__ import annotations

import dataclasses
import math
import numpy as np

from . import lloyd_max, rotation, rng as _rng
from . import rotation as rotation_mod
from .rope import apply_rope

QJL_CONST = math.sqrt(math.pi / 2.0)


@dataclasses.dataclass
class Codebook:
    d: int
    bits: int
    m: int
    dense: bool
    t32: np.ndarray          # [K] float32 levels
    tau32: np.ndarray        # [K-1] float32 thresholds
    pi: np.ndarray           # [d, d] float64 rotation as the codec applies it
    sketch: np.ndarray       # [m, d] float32 (empty when m == 0; the identity for "sign")
    sigma: np.ndarray | None = None
    correction: str = "qjl"  # "qjl": Gaussian sketch + gamma; "sign": per-coordinate signs + mu
    mu: np.ndarray | None = None  # float32 [n_mu] mean residual magnitude per KV head ("sign")
    rotation: str = "hadamard"    # "hadamard", "dense" or "none"

    def mu_of(self, head: int) -> float:
        """mu of a KV head (one shared value when n_mu = 1)."""
        return float(self.mu[head if len(self.mu) > 1 else 0])


def make_codebook(d: int, bits: int, m: int, dense: bool, sigma=None, rot_gauss=None,
                  sketch=None, seed: int | None = None) -> Codebook:
    """Build the codebook from explicit draws, or from ``seed`` through the
    counter-based generator when no draws are given.

    Hadamard form: Pi = H diag(sigma)/sqrt(d) in float64 (its entries are
    +-1/sqrt(d); the GPU applies H in float32 and scales by 1/sqrt(d)).
    Dense form: Pi = the Haar factor of rot_gauss, rounded to float32, since
    the codec stores and applies that float32 matrix."""
    if seed is not None and sigma is None and rot_gauss is None and sketch is None:
        sigma, rot_gauss, sketch = _rng.seeded_draws(d, m, dense, seed)
    t32, tau32 = lloyd_max.table_f32(d, bits)
    if dense:
        pi = rotation.haar_rotation(rot_gauss).astype(np.float32).astype(np.float64)
    else:
        pi = rotation.rht_matrix(np.asarray(sigma))
    s = np.zeros((0, d), np.float32) if m == 0 else np.asarray(sketch, np.float32)
    assert s.shape == (m, d)
    return Codebook(d, bits, m, dense, t32, tau32, pi, s,
                    None if sigma is None else np.asarray(sigma),
                    rotation="dense" if dense else "hadamard")


def thresholds_of(t32: np.ndarray) -> np.ndarray:
    """float32 thresholds of a float32 table: midpoints of neighbouring
    levels, formed in float64 and rounded once."""
    t = np.asarray(t32, np.float32).astype(np.float64)
    return (0.5 * (t[:-1] + t[1:])).astype(np.float32)


def make_sign_codebook(d: int, bits: int, rotation: str = "hadamard", sigma=None, seed: int | None = None,
                       levels=None, mu=None) -> Codebook:
    """TurboESM variant (TurboESM summary, technical section 2): sign of each
    residual coordinate, a per-head mean residual magnitude, its own table.

    rotation: "hadamard" (Pi = H diag(sigma)/sqrt(d); sigma from ``seed``
    when not given) or "none" (Pi = I: the vectors stay in their original
    coordinates).  levels: a float32 symmetric table (calibrated), or None for
    the Beta-law Lloyd-Max table.  mu: float32 [n_mu], or None for the
    Beta-law mean residual magnitude of the table (lloyd_max.mean_abs_error)."""
    if levels is None:
        t32, tau32 = lloyd_max.table_f32(d, bits)
    else:
        t32 = np.asarray(levels, np.float32)
        assert len(t32) == 1 << bits
        tau32 = thresholds_of(t32)
    if rotation == "hadamard":
        if sigma is None:
            sigma, _, _ = _rng.seeded_draws(d, 0, False, seed if seed is not None else 0)
        sigma = np.asarray(sigma)
        pi = rotation_mod.rht_matrix(sigma)
    elif rotation == "none":
        sigma = None
        pi = np.eye(d)
    else:
        raise ValueError("the sign correction takes the Hadamard rotation or none")
    if mu is None:
        mu = np.array([lloyd_max.mean_abs_error(t32, tau32, d)], np.float32)
    return Codebook(d, bits, d, False, t32, tau32, pi, np.eye(d, dtype=np.float32), sigma,
                    correction="sign", mu=np.asarray(mu, np.float32).reshape(-1), rotation=rotation)


# -------------------------------------------------------------- packing --
def code_bit_position(i: int, k: int, bits: int) -> int:
    """Position (in the record's code-word bit string) of bit k of
    coordinate i's code, per the layout in the module docstring."""
    if bits != 3:
        return bits * i + k
    g, j = divmod(i, 32)
    if j < 24:
        word, pos = j // 8, 8 * (j % 4) + 3 * ((j % 8) // 4) + k
    else:
        r = j - 24
        if k < 2:
            word, pos = r // 4, 8 * (r % 4) + 6 + k
        else:
            word, pos = 2, 8 * (r % 4) + 6 + r // 4
    return 96 * g + 32 * word + pos


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    n, d = codes.shape
    nw = (bits * d + 31) // 32
    words = np.zeros((n, nw), dtype=np.uint64)
    c = codes.astype(np.uint64)
    for i in range(d):
        for k in range(bits):
            pos = code_bit_position(i, k, bits)
            words[:, pos // 32] |= ((c[:, i] >> np.uint64(k)) & np.uint64(1)) << np.uint64(pos % 32)
    return words.astype(np.uint32)


def unpack_codes(words: np.ndarray, bits: int, d: int) -> np.ndarray:
    w = np.asarray(words).astype(np.uint64)
    n = w.shape[0]
    codes = np.zeros((n, d), dtype=np.int64)
    for i in range(d):
        for k in range(bits):
            pos = code_bit_position(i, k, bits)
            codes[:, i] |= (((w[:, pos // 32] >> np.uint64(pos % 32)) & np.uint64(1)).astype(np.int64)) << k
    return codes


def pack_signs(bitmat: np.ndarray) -> np.ndarray:
    n, m = bitmat.shape
    words = np.zeros((n, m // 32), dtype=np.uint64)
    b = bitmat.astype(np.uint64)
    for l in range(m):
        words[:, l // 32] |= b[:, l] << np.uint64(l % 32)
    return words.astype(np.uint32)


def unpack_signs(words: np.ndarray, m: int) -> np.ndarray:
    w = np.asarray(words).astype(np.uint64)
    out = np.zeros((w.shape[0], m), dtype=np.int64)
    for l in range(m):
        out[:, l] = ((w[:, l // 32] >> np.uint64(l % 32)) & np.uint64(1)).astype(np.int64)
    return out


# -------------------------------------------------------------- encoder --
@dataclasses.dataclass
class Encoded:
    norm: np.ndarray      # [n] float64 nu
    rnorm: np.ndarray     # [n] float64 gamma
    codes: np.ndarray     # [n, b*d/32] uint32
    signs: np.ndarray     # [n, m/32] uint32
    # intermediate values, for the parity protocol's boundary handling
    y: np.ndarray | None = None       # [n, d] rotated unit vectors
    code_idx: np.ndarray | None = None  # [n, d] codes as integers
    e: np.ndarray | None = None       # [n, d] residuals
    se: np.ndarray | None = None      # [n, m] sketch values S e


def quantise(cb: Codebook, y: np.ndarray) -> np.ndarray:
    """c_i = #{j : y_i >= tau_j}, decided in float32."""
    y32 = np.asarray(y, np.float64).astype(np.float32)
    return (y32[..., None] >= cb.tau32[None, None, :]).sum(-1).astype(np.int64)


def residual_and_sketch(cb: Codebook, y: np.ndarray, code_idx: np.ndarray):
    yhat = cb.t32.astype(np.float64)[code_idx]
    e = y - yhat
    gamma = np.sqrt((e * e).sum(1))
    se = e @ cb.sketch.astype(np.float64).T
    return e, gamma, se


def encode(cb: Codebook, x: np.ndarray, pos: np.ndarray | None = None, rope=None) -> Encoded:
    """Encode rows of x [n, d] (values as the input dtype holds them).

    ``rope`` is (cos32, sin32) to rotate rows by ``pos`` first (keys), or None."""
    x = np.asarray(x, np.float64)
    if rope is not None:
        x = apply_rope(x, pos, rope[0], rope[1])
    nu = np.sqrt((x * x).sum(1))
    safe = np.where(nu > 0, nu, 1.0)
    u = np.where(nu[:, None] > 0, x / safe[:, None], 0.0)
    y = u @ cb.pi.T
    code_idx = quantise(cb, y)
    if cb.correction == "sign":
        # one bit per residual coordinate: bit_i = [e_i >= 0]
        e = y - cb.t32.astype(np.float64)[code_idx]
        gamma = np.sqrt((e * e).sum(1))
        se = e
    else:
        e, gamma, se = residual_and_sketch(cb, y, code_idx)
    bits = (se.astype(np.float32) >= 0).astype(np.int64)
    signs = pack_signs(bits) if cb.m else np.zeros((len(x), 0), np.uint32)
    return Encoded(nu, gamma, pack_codes(code_idx, cb.bits), signs, y, code_idx, e, se)


def dequant(cb: Codebook, enc: Encoded):
    """(yhat [n, d], z [n, m]) from a record: levels looked up from the codes
    and the sketch bits mapped to +-1."""
    yhat = cb.t32.astype(np.float64)[unpack_codes(enc.codes, cb.bits, cb.d)]
    z = 2.0 * unpack_signs(enc.signs, cb.m) - 1.0 if cb.m else np.zeros((len(yhat), 0))
    return yhat, z


def reconstruct(cb: Codebook, enc: Encoded, head: int = 0) -> np.ndarray:
    """Unbiased vector estimate nu * Pi^T (yhat + sqrt(pi/2)/m gamma S^T z)
    (FibQuant summary, section 2.3: look up, inverse rotation, scale by the
    norm; the sketch term makes it unbiased over S).  Sign correction:
    nu * Pi^T (yhat + mu z), with mu of the records' KV head."""
    yhat, z = dequant(cb, enc)
    w = yhat.copy()
    if cb.correction == "sign":
        w += cb.mu_of(head) * z
    elif cb.m:
        w += (QJL_CONST / cb.m) * np.asarray(enc.rnorm, np.float64)[:, None] * (z @ cb.sketch.astype(np.float64))
    return np.asarray(enc.norm, np.float64)[:, None] * (w @ cb.pi)


def record_bytes(d: int, bits: int, m: int, with_rnorm: bool = True) -> int:
    """Bytes of one fixed-address record (with_rnorm False: the sign
    correction's record, which stores no gamma)."""
    return 4 + (4 if (m and with_rnorm) else 0) + bits * d // 8 + m // 8
