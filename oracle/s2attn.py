"""Shifted short attention (S2-Attn) oracle, float64.

What the pages fix (LongQLoRA post, section 03 方法介绍, Shift Short Attention paragraph;
LongLoRA abstract on the chatpaper.ai page): the sequence is split into groups, attention
runs only inside each group, and a shift lets information flow between groups; in
training it is a two-line change around an ordinary attention call.  The group size is a
quarter of the target length (LongQLoRA post, section 04).

Readings where the pages are silent:

* the shifted heads are ``[H/2, H)``; their shift is ``s = G/2``; with one group
  (``N == G``) nothing is shifted, so ``G == N`` is plain causal attention;
* a shifted head sees position ``p(t) = (t - s) mod N`` (the sequence rolled left by s),
  group ``floor(p / G)``;
* R1 (default): inside a group, key u is visible to query t iff ``p(u) <= p(t)``
  (roll, attend causally, roll back).  R2: iff ``u <= t`` in token order;
* kv head of q head h is ``floor(h * Hkv / H)``; dK/dV of a kv head sum over its q heads.

Layouts follow the library: Q/O/dO ``[B, N, H, d]``, K/V ``[B, N, Hkv, d]``, LSE
``[B, H, N]``.  Three independent forward formulations are provided (full mask, per
group, materialised roll); the tests require them to agree.
"""
from __future__ import annotations

import numpy as np

from .attention import masked_attention, masked_attention_bwd


def head_shift(h: int, H: int, N: int, G: int, shift: bool) -> int:
    """Shift amount of q head h: G/2 for the upper half of the heads when N/G >= 2."""
    if shift and N // G >= 2 and h >= H // 2:
        return G // 2
    return 0


def kv_head(h: int, H: int, Hkv: int) -> int:
    return (h * Hkv) // H


def s2attn_mask(N: int, G: int, s: int, reading: str = "R1") -> np.ndarray:
    """[N, N] visibility mask of one head whose sequence is rolled by s (brute force)."""
    t = np.arange(N)
    p = (t - s) % N
    g = p // G
    same = g[:, None] == g[None, :]
    if reading == "R1":
        order = p[None, :] <= p[:, None]
    elif reading == "R2":
        order = t[None, :] <= t[:, None]
    else:
        raise ValueError(reading)
    return same & order


def _check(N, G, H, Hkv):
    if N % G:
        raise ValueError("N must be a multiple of G")
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")


def s2attn_fwd_bruteforce(q, k, v, G, shift, scale, reading="R1"):
    """Formulation (i): the full N x N mask per head.  Small shapes only."""
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    _check(N, G, H, Hkv)
    o = np.zeros((B, N, H, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            m = s2attn_mask(N, G, head_shift(h, H, N, G, shift), reading)
            kv = kv_head(h, H, Hkv)
            o[b, :, h], lse[b, h] = masked_attention(q[b, :, h], k[b, :, kv], v[b, :, kv], m, scale)
    return o, lse


def s2attn_bwd_bruteforce(q, k, v, do, G, shift, scale, reading="R1"):
    """Backward of formulation (i).  Returns (O, LSE, dQ, dK, dV)."""
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    _check(N, G, H, Hkv)
    o, lse = s2attn_fwd_bruteforce(q, k, v, G, shift, scale, reading)
    dq = np.zeros_like(o)
    dk = np.zeros((B, N, Hkv, d))
    dv = np.zeros((B, N, Hkv, d))
    for b in range(B):
        for h in range(H):
            m = s2attn_mask(N, G, head_shift(h, H, N, G, shift), reading)
            kv = kv_head(h, H, Hkv)
            gq, gk, gv = masked_attention_bwd(q[b, :, h], k[b, :, kv], v[b, :, kv], m, scale,
                                              o[b, :, h], lse[b, h], do[b, :, h])
            dq[b, :, h] = gq
            dk[b, :, kv] += gk
            dv[b, :, kv] += gv
    return o, lse, dq, dk, dv


def group_tokens(N: int, G: int, s: int, g: int) -> np.ndarray:
    """Tokens of rolled group g, listed in rolled (attention) order."""
    return (g * G + np.arange(G) + s) % N


def s2attn_unit(q, k, v, do, b, h, g, G, shift, scale, reading="R1"):
    """Formulation (ii) for one independent unit (batch b, q head h, group g).

    Gathers the group's tokens, runs causal attention over them in the reading's order,
    and returns ``(tokens, O, LSE, dQ, dK_part, dV_part)``; rows are in ``tokens`` order.
    dK/dV are this q head's contribution to its kv head.  ``do`` may be None (forward).
    """
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    s = head_shift(h, H, N, G, shift)
    kv = kv_head(h, H, Hkv)
    tok = group_tokens(N, G, s, g)
    if reading == "R1":
        rank = np.arange(G)
    else:
        rank = tok
    mask = rank[None, :] <= rank[:, None]
    qg = q[b, tok, h]
    kg = k[b, tok, kv]
    vg = v[b, tok, kv]
    o, lse = masked_attention(qg, kg, vg, mask, scale)
    if do is None:
        return tok, o, lse, None, None, None
    gq, gk, gv = masked_attention_bwd(qg, kg, vg, mask, scale, o, lse, do[b, tok, h])
    return tok, o, lse, gq, gk, gv


def s2attn_groups(q, k, v, do, G, shift, scale, reading="R1"):
    """Formulation (ii) over every unit.  Returns (O, LSE, dQ, dK, dV); grads None if do is None."""
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    _check(N, G, H, Hkv)
    o = np.zeros((B, N, H, d))
    lse = np.zeros((B, H, N))
    dq = dk = dv = None
    if do is not None:
        dq = np.zeros((B, N, H, d))
        dk = np.zeros((B, N, Hkv, d))
        dv = np.zeros((B, N, Hkv, d))
    for b in range(B):
        for h in range(H):
            kv = kv_head(h, H, Hkv)
            for g in range(N // G):
                tok, go, gl, gq, gk, gv = s2attn_unit(q, k, v, do, b, h, g, G, shift, scale, reading)
                o[b, tok, h] = go
                lse[b, h, tok] = gl
                if do is not None:
                    dq[b, tok, h] = gq
                    dk[b, tok, kv] += gk
                    dv[b, tok, kv] += gv
    return o, lse, dq, dk, dv


def s2attn_fwd_roll(q, k, v, G, shift, scale):
    """Formulation (iii), reading R1 only: materialise the roll on the shifted heads.

    ``np.roll(x, -s)`` along tokens, split into N/G groups, causal attention inside each
    group (lower-triangular mask), then ``np.roll(O, +s)`` back to token order.
    """
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    _check(N, G, H, Hkv)
    ng = N // G
    tril = np.tril(np.ones((G, G), dtype=bool))
    o = np.zeros((B, N, H, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            s = head_shift(h, H, N, G, shift)
            kv = kv_head(h, H, Hkv)
            qr = np.roll(q[b, :, h], -s, axis=0).reshape(ng, G, d)
            kr = np.roll(k[b, :, kv], -s, axis=0).reshape(ng, G, d)
            vr = np.roll(v[b, :, kv], -s, axis=0).reshape(ng, G, d)
            sc = scale * np.einsum("gid,gjd->gij", qr, kr)
            sc = np.where(tril[None], sc, -np.inf)
            m = sc.max(axis=2, keepdims=True)
            p = np.exp(sc - m)
            l = p.sum(axis=2, keepdims=True)
            orr = np.einsum("gij,gjd->gid", p / l, vr).reshape(N, d)
            lr = (m + np.log(l)).reshape(N)
            o[b, :, h] = np.roll(orr, s, axis=0)
            lse[b, h] = np.roll(lr, s, axis=0)
    return o, lse


def s2attn_pair_count(N: int, G: int) -> int:
    """Visible (query, key) pairs of one head, counted from the mask (brute force)."""
    return int(s2attn_mask(N, G, G // 2 if N // G >= 2 else 0).sum())


def s2attn_rows(q, k, v, b, h, rows, G, shift, scale, reading="R1"):
    """Forward for selected query rows of one (batch, q head): (O [len(rows), d], LSE).

    Each row's visible keys are found from the rule directly (same rolled group, rolled
    position not after the query's), so sampled rows of very long sequences can be
    checked without forming the N x N mask.
    """
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    s = head_shift(h, H, N, G, shift)
    kv = kv_head(h, H, Hkv)
    t = np.arange(N)
    p = (t - s) % N
    out_o = np.zeros((len(rows), d))
    out_l = np.zeros(len(rows))
    for i, r in enumerate(rows):
        pr = (r - s) % N
        if reading == "R1":
            vis = (p // G == pr // G) & (p <= pr)
        else:
            vis = (p // G == pr // G) & (t <= r)
        keys = np.nonzero(vis)[0]
        o, l = masked_attention(np.asarray(q[b, r:r + 1, h], np.float64), np.asarray(k[b, keys, kv], np.float64),
                                np.asarray(v[b, keys, kv], np.float64), np.ones((1, keys.size), bool), scale)
        out_o[i], out_l[i] = o[0], l[0]
    return out_o, out_l
