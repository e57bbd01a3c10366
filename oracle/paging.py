"""Fixed-address record layouts for a growing cache (oracle side).

Source: FibQuant summary, section 1: a deployable cache codec keeps every
record at a fixed address, so that the key or value of any token decodes on
its own through simple address arithmetic; the cache grows with the context
and is read at every decode step.  TurboESM summary, technical section 5:
autoregressive generation, where keeping the context is the bottleneck.

Readings:

* Appending a token encodes it exactly as a bulk encode would (RoPE at its
  own position for keys) and writes its record at its slot, nothing else.
* Contiguous layout: record (b, head, t) is n = (b * h_kv + head) * L_cap + t.
* Paged layout: a sequence's slots are cut into pages of P tokens; a page
  table maps (sequence b, logical page j) to a physical page, and physical
  page p holds the P slots of every KV head:
      n = (pages[b, t // P] * h_kv + head) * P + t % P.
  The contiguous layout is the paged one with a single page of L_cap slots
  per sequence and pages[b, 0] = b.

Pinned by tests: the contiguous special case; the map is one to one over a
page table of distinct pages; appending tokens one by one leaves the same
records as encoding the sequence in one call.
"""
from __future__ import annotations

import numpy as np

from . import codec


def contiguous_index(b, head, t, h_kv: int, L_cap: int):
    return (np.asarray(b) * h_kv + np.asarray(head)) * L_cap + np.asarray(t)


def paged_index(pages: np.ndarray, page_size: int, h_kv: int, b, head, t):
    """Record index of (b, head, t) through the page table pages [B, max_pages]."""
    b, head, t = np.asarray(b), np.asarray(head), np.asarray(t)
    return (np.asarray(pages)[b, t // page_size].astype(np.int64) * h_kv + head) * page_size + t % page_size


def empty_pool(cb: codec.Codebook, n: int) -> dict:
    """Record planes for n records (norm 0, codes 0)."""
    return {"norm": np.zeros(n), "rnorm": np.zeros(n), "codes": np.zeros((n, cb.bits * cb.d // 32), np.uint32),
            "signs": np.zeros((n, cb.m // 32), np.uint32)}


def write(pool: dict, idx: np.ndarray, enc: codec.Encoded):
    """Store encoded rows at record indices idx."""
    pool["norm"][idx] = enc.norm
    pool["rnorm"][idx] = enc.rnorm
    pool["codes"][idx] = enc.codes
    pool["signs"][idx] = enc.signs


def gather(pool: dict, idx) -> codec.Encoded:
    """The records at indices idx, in that order."""
    idx = np.asarray(idx)
    return codec.Encoded(pool["norm"][idx], pool["rnorm"][idx], pool["codes"][idx], pool["signs"][idx])


def append(cb: codec.Codebook, pool: dict, x: np.ndarray, pos: np.ndarray, index_of, rope=None):
    """Append one token per (sequence, head): x [B, h_kv, d] goes to slot
    pos[b] of sequence b (also its RoPE position when rope is given);
    index_of(b, head, t) gives the record index.  Returns the encoded rows
    in (b, head) order."""
    x = np.asarray(x, np.float64)
    B, h_kv, d = x.shape
    b = np.repeat(np.arange(B), h_kv)
    head = np.tile(np.arange(h_kv), B)
    t = np.asarray(pos)[b]
    enc = codec.encode(cb, x.reshape(B * h_kv, d), pos=t if rope is not None else None, rope=rope)
    write(pool, index_of(b, head, t), enc)
    return enc
