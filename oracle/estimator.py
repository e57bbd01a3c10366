"""Decode-time estimates from packed records (oracle side).

* Attention logits straight from quantised keys (tambur post: 4-bit keys
  give up to 8x faster attention-logit computation than 32-bit keys).
* Unbiased inner products through the one-bit QJL sketch (iaemfoco post,
  "TurboQuant: Uma Nova Abordagem"; itstec post, "Por dentro do processo de
  compressao KV").  For a query q (RoPE'd at its position), q' = Pi q and
  s = S q'; a key record (nu, gamma, codes c, sketch bits z in {-1,+1}) gives

      logit = nu * ( sum_i q'_i t[c_i] + sqrt(pi/2)/m * gamma * sum_l s_l z_l ).

  For a Gaussian row S_l, E[(S_l q') sign(S_l e)] = sqrt(2/pi) <q', e>/||e||,
  so the second term's expectation over S is <q', e> and the logit's is
  nu <q', y> = <RoPE(q), RoPE(k)>.  With m = 0 the second term is absent.
* Fused decode (TurboESM summary, technical section 2, "Kernel Fused de
  Decodificacao"): softmax over the logits of the first seq_len keys, times
  the values rebuilt as nu_v Pi_v^T (yhat_v + sqrt(pi/2)/m_v gamma_v S_v^T z_v)
  (FibQuant summary, section 2.3).  The oracle takes the softmax in two
  passes (max, then exp and sum); the GPU's online form computes the same
  function.
* TurboESM variant (TurboESM summary, technical section 2): with one sign
  bit per residual coordinate (S = I) and a per-head calibrated mean residual
  magnitude mu, the key estimate is nu (yhat + mu z), so

      logit = nu * ( sum_i q'_i t[c_i] + mu * sum_i q'_i z_i ),

  and a value row is nu Pi_v^T (yhat_v + mu_v z_v) (Pi_v = I for a table in
  the original coordinates).  mu is that of the records' KV head.
* Vector search (tambur post; itstec post, introduction): a full scan of
  inner-product estimates and the k best per query; ties go to the smaller
  index.

Pinned by tests: Monte-Carlo unbiasedness over many sketches against the
closed-form variance; the MSE-only estimate's bias at b = 1 (the 2/pi factor
in high dimension); textbook softmax attention when quantisation is bypassed;
explicit dense attention over reconstructed keys and values.
"""
from __future__ import annotations

import numpy as np

from .codec import Codebook, Encoded, dequant, QJL_CONST
from .rope import apply_rope


def prep_query(cb: Codebook, q: np.ndarray, pos=None, rope=None):
    """(q' [G, d], s [G, m]) in float64 for queries q [G, d]."""
    q = np.asarray(q, np.float64)
    if rope is not None:
        q = apply_rope(q, np.full(len(q), pos) if np.isscalar(pos) else pos, rope[0], rope[1])
    qp = q @ cb.pi.T
    s = qp @ cb.sketch.astype(np.float64).T
    return qp, s


def logits(cb: Codebook, qp: np.ndarray, s: np.ndarray, enc: Encoded, head: int = 0) -> np.ndarray:
    """[G, n] logits of G prepared queries against n key records of KV head
    ``head`` (used by the sign correction's mu)."""
    yhat, z = dequant(cb, enc)
    out = yhat @ qp.T                                       # [n, G]
    if cb.correction == "sign":
        out = out + cb.mu_of(head) * (z @ qp.T)
    elif cb.m:
        out = out + (QJL_CONST / cb.m) * np.asarray(enc.rnorm, np.float64)[:, None] * (z @ s.T)
    return (np.asarray(enc.norm, np.float64)[:, None] * out).T


def value_rows(cbv: Codebook, enc: Encoded, head: int = 0) -> np.ndarray:
    """[n, d] value estimates nu Pi^T (yhat + sqrt(pi/2)/m gamma S^T z), or
    nu Pi^T (yhat + mu z) with the sign correction."""
    yhat, z = dequant(cbv, enc)
    w = yhat
    if cbv.correction == "sign":
        w = w + cbv.mu_of(head) * z
    elif cbv.m:
        w = w + (QJL_CONST / cbv.m) * np.asarray(enc.rnorm, np.float64)[:, None] * (z @ cbv.sketch.astype(np.float64))
    return np.asarray(enc.norm, np.float64)[:, None] * (w @ cbv.pi)


def softmax_rows(a: np.ndarray) -> np.ndarray:
    mx = a.max(axis=1, keepdims=True)
    p = np.exp(a - mx)
    return p / p.sum(axis=1, keepdims=True)


def attention(cbk: Codebook, cbv: Codebook, qp, s, enc_k: Encoded, enc_v: Encoded,
              seq_len: int, scale: float, head: int = 0) -> np.ndarray:
    """[G, d] decode output over the first seq_len records (zeros if 0) of
    KV head ``head``."""
    G = qp.shape[0]
    if seq_len == 0:
        return np.zeros((G, cbv.d))
    lg = logits(cbk, qp, s, enc_k, head)[:, :seq_len] * scale
    p = softmax_rows(lg)
    return p @ value_rows(cbv, enc_v, head)[:seq_len]


def topk(scores: np.ndarray, k: int):
    """(idx [G, k], vals [G, k]): the k largest per row, ties to the smaller
    index."""
    n = scores.shape[1]
    order = np.lexsort((np.broadcast_to(np.arange(n), scores.shape), -scores), axis=1)[:, :k]
    return order, np.take_along_axis(scores, order, axis=1)
