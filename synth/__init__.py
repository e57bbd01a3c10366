"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the benchmark.

This module holds input generation only: raw key/value/query tensors shaped
like the workloads the pages describe, and the random draws the codec makes
(random signs for the Hadamard rotation, the Gaussian matrix a Haar rotation is
taken from, and the Gaussian sketch matrix).  It contains none of the codec's
arithmetic: no rotation, quantisation, packing or estimation happens here, so
the oracle and the HIP path share nothing beyond the inputs they are fed.

Every array comes from ``numpy.random.Generator(PCG64(seed))`` and is drawn in
the order written below, so a (config, seed, size) triple always yields the
same bytes.

Workloads (each stands in for a model or corpus the pages measure on; no
dataset or trained weight is used or needed):

* ``tiny``   - 4096 fp32 keys of dimension 128 with two outlier channels x50,
               16 fp32 queries (a stress case for the scalar table).
* ``llama8b``- one Llama-3.1-8B-shaped layer: batch 8, 32 query heads, 8 KV
               heads, head dim 128, context 32768, bf16 K/V ~ N(0,1) with 10 of
               the 1024 (head, channel) pairs scaled x100, RoPE base 5e5.
* ``llama70b``- batch 1, 64 query heads, 8 KV heads, head dim 128, context
               131072, bf16 K/V with a Student-t(3) magnitude per
               (head, channel) times N(0,1), no RoPE.
* ``esm650m``- ESM-2-650M-shaped prefill: 33 layers x 20 heads of dim 64, 32
               sequences of 1024 residues drawn uniformly from a 20-letter
               alphabet, embedded (N(0,1), width 1280) and projected by random
               N(0, 1/1280) K and V matrices per layer; fp32; RoPE base 1e4.
* ``vsearch``- 1e6 database vectors and 1024 queries of dimension 1536, N(0,1)
               rows scaled to unit L2 norm, fp32.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "rng", "bf16_round_bits", "bf16_bits_to_f32", "codec_draws", "CONFIGS",
    "WorkloadSpec", "tiny_inputs", "llama_kv_inputs", "llama_q_inputs",
    "esm_tokens", "esm_layer_tables", "vsearch_rows",
]


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# ----------------------------------------------------------------- dtypes --
def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); returns the
    16-bit patterns as uint16.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------ the codec's draws --
def codec_draws(d: int, m: int, dense: bool, seed: int):
    """Random draws of one codebook: (sigma, rot_gauss, sketch).

    sigma     int8 [d]     entries +1 / -1 (Hadamard form; None if dense)
    rot_gauss float64[d,d] i.i.d. N(0,1); a Haar rotation is taken from its QR
                           factorisation (dense form; None otherwise)
    sketch    float32[m,d] i.i.d. N(0,1) rounded to fp32 (None if m == 0)
    """
    g = rng(seed)
    sigma = None
    rot_gauss = None
    if dense:
        rot_gauss = g.standard_normal((d, d))
    else:
        sigma = np.where(g.integers(0, 2, size=d) == 1, 1, -1).astype(np.int8)
    sketch = None
    if m > 0:
        sketch = g.standard_normal((m, d)).astype(np.float32)
    return sigma, rot_gauss, sketch


# -------------------------------------------------------------- workloads --
@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    d: int
    bits: int
    m: int
    dense: bool
    batch: int          # sequences
    hq: int             # query heads
    hkv: int            # KV heads
    ctx: int            # context length (tokens per sequence)
    dtype: str          # "f32" | "bf16"
    rope_base: float    # 0 = no RoPE
    layers: int = 1


CONFIGS = {
    "tiny": WorkloadSpec("tiny", 128, 2, 128, False, 1, 16, 1, 4096, "f32", 0.0),
    "llama8b": WorkloadSpec("llama8b", 128, 3, 64, False, 8, 32, 8, 32768, "bf16", 500000.0),
    "llama70b": WorkloadSpec("llama70b", 128, 3, 128, False, 1, 64, 8, 131072, "bf16", 0.0),
    "esm650m": WorkloadSpec("esm650m", 64, 3, 64, False, 32, 20, 20, 1024, "f32", 10000.0, 33),
    "vsearch": WorkloadSpec("vsearch", 1536, 2, 1536, True, 1, 1024, 1, 1000000, "f32", 0.0),
}

# codebook seeds: keys use 0, values use 1
K_SEED = 0
V_SEED = 1


def tiny_inputs(seed: int = 0, n: int = 4096, d: int = 128, nq: int = 16):
    """Keys [n, d] fp32 N(0,1) with two randomly chosen channels scaled x50,
    queries [nq, d] fp32 N(0,1)."""
    g = rng(seed)
    k = g.standard_normal((n, d)).astype(np.float32)
    ch = g.choice(d, size=2, replace=False)
    k[:, ch] *= np.float32(50.0)
    q = g.standard_normal((nq, d)).astype(np.float32)
    return k, q, ch


def llama_kv_inputs(kind: str, seed: int = 0, batch: int = 8, ctx: int = 32768,
                    hkv: int = 8, d: int = 128):
    """K and V as bf16 bit patterns (uint16) of shape [batch, ctx, hkv, d].

    kind "llama8b": N(0,1) with 10 of the hkv*d (head, channel) pairs per
    tensor multiplied by 100 (one percent of channels far above the median).
    kind "llama70b": each (head, channel) gets a scale |t_3|; entries are
    scale * N(0,1).
    """
    g = rng(seed)
    out = []
    for _tensor in range(2):
        if kind == "llama8b":
            pairs = g.choice(hkv * d, size=max(1, (hkv * d) // 100), replace=False)
            scale = np.ones(hkv * d, np.float32)
            scale[pairs] = 100.0
        elif kind == "llama70b":
            scale = np.abs(g.standard_t(3, size=hkv * d)).astype(np.float32)
        else:
            raise ValueError(kind)
        scale = scale.reshape(hkv, d)
        t = np.empty((batch, ctx, hkv, d), np.uint16)
        for b in range(batch):
            x = g.standard_normal((ctx, hkv, d), dtype=np.float32)
            x *= scale[None]
            t[b] = bf16_round_bits(x)
        out.append(t)
    return out[0], out[1]


def llama_q_inputs(seed: int = 100, batch: int = 8, hq: int = 32, d: int = 128):
    """Queries as bf16 bit patterns [batch, hq, d], N(0,1)."""
    g = rng(seed)
    return bf16_round_bits(g.standard_normal((batch, hq, d), dtype=np.float32))


def esm_tokens(seed: int = 0, batch: int = 32, length: int = 1024, alphabet: int = 20):
    return rng(seed).integers(0, alphabet, size=(batch, length))


def esm_layer_tables(layer: int, seed: int = 0, width: int = 1280, alphabet: int = 20):
    """Per-layer projected embeddings (P_k, P_v), each [alphabet, width] fp32.

    The embedding E ~ N(0,1) [alphabet, width] is shared by all layers; layer
    l draws W_k, W_v ~ N(0, 1/width).  Token t of the sequence then has key
    row P_k[t] (= E[t] W_k) and value row P_v[t]; reshaped to [heads, 64].
    """
    e = rng(seed + 7).standard_normal((alphabet, width))
    g = rng(seed + 1000 + layer)
    wk = g.standard_normal((width, width)) / np.sqrt(width)
    wv = g.standard_normal((width, width)) / np.sqrt(width)
    return (e @ wk).astype(np.float32), (e @ wv).astype(np.float32)


def vsearch_rows(seed: int, start: int, count: int, d: int = 1536, chunk: int = 65536):
    """Rows [start, start+count) of an N(0,1) matrix whose rows are scaled to
    unit L2 norm, fp32.  Rows are generated in fixed chunks of ``chunk`` rows
    (chunk c from seed (seed, c)), so any row range is reproducible alone."""
    out = np.empty((count, d), np.float32)
    r = start
    while r < start + count:
        c = r // chunk
        g = rng(seed * 1_000_003 + c)
        block = g.standard_normal((chunk, d))
        block /= np.linalg.norm(block, axis=1, keepdims=True)
        lo = r - c * chunk
        hi = min(chunk, start + count - c * chunk)
        out[r - start:r - start + (hi - lo)] = block[lo:hi].astype(np.float32)
        r += hi - lo
    return out
