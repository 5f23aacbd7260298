"""Plain masked softmax attention in float64: the definition both methods reduce to.

For one head: ``S = scale * Q K^T`` restricted to a boolean mask, a row softmax, and
``O = P V``.  The backward is the textbook chain rule through the softmax
(``dS = P * (dP - rowsum(dO * O))``).  No blocking, no online softmax: the whole score
matrix is formed, which is why callers keep the shapes small or go unit by unit.
"""
from __future__ import annotations

import numpy as np


def masked_attention(q, k, v, mask, scale):
    """Forward for one head.

    q: [Lq, d], k/v: [Lk, d], mask: [Lq, Lk] bool (True = the key is visible), every row
    must have at least one visible key.  Returns (O [Lq, d], LSE [Lq]) where
    ``LSE = log(sum_u exp(S[t, u]))`` over the visible keys (natural log).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = scale * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no visible key")
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def softmax_probs(q, k, mask, scale, lse):
    """P[t, u] = exp(scale * q_t . k_u - LSE[t]) on the mask, 0 elsewhere."""
    s = scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    p = np.exp(np.where(mask, s, -np.inf) - lse[:, None])
    return p


def masked_attention_bwd(q, k, v, mask, scale, o, lse, do):
    """Backward for one head: returns (dQ [Lq,d], dK [Lk,d], dV [Lk,d]).

    With P the forward probabilities, ``dV = P^T dO``, ``dP = dO V^T``,
    ``D = rowsum(dO * O)``, ``dS = P * (dP - D)``, ``dQ = scale dS K``,
    ``dK = scale dS^T Q``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    p = softmax_probs(q, k, mask, scale, lse)
    dv = p.T @ do
    dp = do @ v.T
    dsum = (do * o).sum(axis=1, keepdims=True)
    ds = p * (dp - dsum)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv
