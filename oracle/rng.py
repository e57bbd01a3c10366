"""Counter-based generator for codebooks defined by a 64-bit seed (oracle side).

When a codebook is requested by seed alone (no draws supplied), the codec
derives its random signs, rotation Gaussians and sketch Gaussians from this
generator.  The oracle implements it here from the published definitions, in
plain Python integers and the C library's math functions (``math``); the HIP
library implements the same definitions independently in C++.

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): the state advances by the odd constant
  0x9E3779B97F4A7C15 and each output is the state passed through the
  variant-13 64-bit finaliser (xor-shift 30, multiply 0xBF58476D1CE4E5B9,
  xor-shift 27, multiply 0x94D049BB133111EB, xor-shift 31).
* Purpose streams: purpose p (1 = Hadamard signs, 2 = rotation Gaussians,
  3 = sketch Gaussians) runs a SplitMix64 whose initial state is output
  number p (1-based) of a SplitMix64 started at ``seed``.
* Uniforms: the top 53 bits of an output times 2**-53, in [0, 1).
* Gaussians: Box-Muller (1958) on consecutive uniforms (u1, u2):
  r = sqrt(-2 ln(1 - u1)), z0 = r cos(2 pi u2), z1 = r sin(2 pi u2).
* Signs: +1 when the top bit of an output is 0, else -1.

Pinned in tests: SplitMix64 against its published test vectors
(tests/golden/splitmix64_published.txt), Box-Muller at inputs with closed-form
outputs and by a Kolmogorov-Smirnov test of many draws against N(0,1), the
uniforms by their range and moments, and the signs by their balance.
"""
from __future__ import annotations

import math
import numpy as np

MASK = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15

PURPOSE_SIGNS = 1
PURPOSE_ROTATION = 2
PURPOSE_SKETCH = 3


def mix64(z: int) -> int:
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def splitmix64(state: int, n: int):
    """First n outputs of SplitMix64 started at ``state``."""
    out = []
    s = state & MASK
    for _ in range(n):
        s = (s + GAMMA) & MASK
        out.append(mix64(s))
    return out


def stream_state(seed: int, purpose: int) -> int:
    return splitmix64(seed, purpose)[purpose - 1]


def uniforms(seed: int, purpose: int, n: int) -> np.ndarray:
    outs = splitmix64(stream_state(seed, purpose), n)
    return np.array([(o >> 11) * 2.0 ** -53 for o in outs], dtype=np.float64)


def box_muller(u1: float, u2: float):
    """Two independent N(0,1) values from two uniforms in [0, 1) (Box and
    Muller, 1958): radius sqrt(-2 ln(1 - u1)), angle 2 pi u2."""
    r = math.sqrt(-2.0 * math.log(1.0 - u1))
    a = 2.0 * math.pi * u2
    return r * math.cos(a), r * math.sin(a)


def gaussians(seed: int, purpose: int, n: int) -> np.ndarray:
    """n standard normal values (float64) by Box-Muller."""
    npairs = (n + 1) // 2
    outs = splitmix64(stream_state(seed, purpose), 2 * npairs)
    z = []
    for k in range(npairs):
        u1 = (outs[2 * k] >> 11) * 2.0 ** -53
        u2 = (outs[2 * k + 1] >> 11) * 2.0 ** -53
        z.extend(box_muller(u1, u2))
    return np.array(z[:n], dtype=np.float64)


def signs(seed: int, n: int) -> np.ndarray:
    outs = splitmix64(stream_state(seed, PURPOSE_SIGNS), n)
    return np.array([1 if (o >> 63) == 0 else -1 for o in outs], dtype=np.int8)


def seeded_draws(d: int, m: int, dense: bool, seed: int):
    """(sigma, rot_gauss, sketch) as the codec derives them from ``seed``."""
    sigma = None if dense else signs(seed, d)
    rot_gauss = gaussians(seed, PURPOSE_ROTATION, d * d).reshape(d, d) if dense else None
    sketch = gaussians(seed, PURPOSE_SKETCH, m * d).reshape(m, d).astype(np.float32) if m else None
    return sigma, rot_gauss, sketch
