"""The parity helpers reject the mistakes they exist to catch (CPU only)."""
import numpy as np
import pytest

import parity
from oracle import estimator


def _case():
    g = np.random.default_rng(0)
    scores = g.standard_normal((3, 200))
    idx, vals = estimator.topk(scores, 10)
    return scores, idx.astype(np.int32), vals.astype(np.float32)


def test_check_topk_accepts_the_oracle_answer():
    scores, idx, vals = _case()
    parity.check_topk(vals, idx, scores, 10)


@pytest.mark.parametrize("mistake", ["repeat_best", "ascending", "wrong_value", "below_kth", "out_of_range"])
def test_check_topk_rejects(mistake):
    scores, idx, vals = _case()
    idx, vals = idx.copy(), vals.copy()
    if mistake == "repeat_best":
        idx[1, :] = idx[1, 0]
        vals[1, :] = vals[1, 0]
    elif mistake == "ascending":
        idx[0] = idx[0, ::-1]
        vals[0] = vals[0, ::-1]
    elif mistake == "wrong_value":
        vals[2, 3] += 0.5
        vals[2] = np.sort(vals[2])[::-1]
    elif mistake == "below_kth":
        worst = int(np.argmin(scores[0]))
        idx[0, 9] = worst
        vals[0, 9] = scores[0, worst]
    else:
        idx[1, 4] = 200
    with pytest.raises(AssertionError):
        parity.check_topk(vals, idx, scores, 10)


def test_check_topk_short_rows_need_padding():
    scores, idx, vals = _case()
    short = scores[:, :6]
    i6, v6 = estimator.topk(short, 6)
    idx = np.full((3, 10), -1, np.int32)
    vals = np.full((3, 10), -np.inf, np.float32)
    idx[:, :6], vals[:, :6] = i6, v6
    parity.check_topk(vals, idx, short, 10)
    idx[0, 7] = 3
    with pytest.raises(AssertionError):
        parity.check_topk(vals, idx, short, 10)
