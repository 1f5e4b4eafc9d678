"""Validity of a GPU expert selection against the oracle's router logits.

The oracle sums each router logit in one fixed fp32 order (64-wide chunk
partials, then one ascending chain over them).  The GPU kernels sum the same
exact products in an order of their own, so their logits differ from the
oracle's by rounding only.  Where two logits of a token lie that close, either
ranking of them is a correct top-k.  The band is relative to the token's
largest |logit|: two logits closer than BAND_REL * max|z| may swap; a rounding
difference of the sums is orders of magnitude smaller at the layer's shapes
(H <= 8192 fp32 terms of |z| ~ 1).

A selection `ids` of token t is accepted when it equals the oracle's, or when
  - its k ids are distinct and in [0, E), and every logit of the token is
    finite (non-finite logits are compared exactly: they come from products,
    which both sides form exactly);
  - every chosen expert's oracle logit is at least every unchosen one's
    minus delta, and consecutive chosen logits are ordered up to delta,
where delta = BAND_REL * max_e |z[t][e]|.  That is exactly the set of top-k
lists of some logits within delta/2 of the oracle's.
"""
from __future__ import annotations

import numpy as np

BAND_REL = 1e-5


def check_selection(ids: np.ndarray, z: np.ndarray, ids_ref: np.ndarray,
                    band_rel: float = BAND_REL):
    """Returns (valid [T] bool, substituted [T] bool): substituted marks the
    tokens whose ids differ from the oracle's ids_ref."""
    ids = np.asarray(ids)
    z = np.asarray(z, np.float64)
    T, k = ids.shape
    E = z.shape[1]
    valid = np.ones(T, bool)
    sub = np.zeros(T, bool)
    for t in range(T):
        if np.array_equal(ids[t], ids_ref[t]):
            continue
        sub[t] = True
        it = ids[t]
        zt = z[t]
        if (it < 0).any() or (it >= E).any() or len(set(it.tolist())) != k:
            valid[t] = False
            continue
        if not np.isfinite(zt).all():
            valid[t] = False
            continue
        delta = band_rel * np.abs(zt).max()
        chosen = zt[it]
        mask = np.ones(E, bool)
        mask[it] = False
        if mask.any() and chosen.min() < zt[mask].max() - delta:
            valid[t] = False
            continue
        if (chosen[1:] > chosen[:-1] + delta).any():
            valid[t] = False
    return valid, sub
