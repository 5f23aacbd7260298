"""Bounded-history attention (HGA) oracle, float64.

What the page fixes ("Long-Context Fine-Tuning with Limited VRAM", BMW Group, English
abstract): gradients flow into the current segment alone, while earlier keys and values
are cut off from the graph; a summary per history chunk stays in memory; every query
block attends to a fixed-size selection of whole history chunks, token for token; the
summary table gets longer as the history does.

Readings (the page prints no formula for any of these):

* summary of chunk c, kv head j: mean of the chunk's ``chunk`` keys (``summarize``);
* block score of chunk c for q head h, query block b: ``mean(Q[block b, h]) . summary[c,
  kv(h)]``, without the 1/sqrt(d) factor (``block_scores``);
* top-k_eff with ``k_eff = min(k, C)``, ties broken toward the lower chunk index, the
  selected indices reported ascending and padded with ``-1`` (``select_topk``);
  selection is per (batch, q head, query block); the variant shared per kv head ranks
  chunks by the sum of the group's per-head scores (``group_block_scores``);
* a query at segment position t attends, under ONE softmax, to the active keys
  ``u <= t`` and to every token of its block's selected chunks (``block_key_set``);
* backward: dQ over that whole key set, dK/dV for the active segment from the local part
  only; the history receives nothing and the selection is held fixed.

Layouts: Q/O/dO ``[B, S, H, d]``; active K/V ``[B, S, Hkv, d]``; history K/V
``[B, T, Hkv, d]``; summaries ``[B, C, Hkv, d]``; indices ``[B, H, S/qblock, topk]``
int32; LSE ``[B, H, S]``.
"""
from __future__ import annotations

import numpy as np

from .attention import masked_attention, masked_attention_bwd


def kv_head(h: int, H: int, Hkv: int) -> int:
    return (h * Hkv) // H


def summarize(k_hist, chunk):
    """Per-chunk mean key: [B, T, Hkv, d] -> [B, T/chunk, Hkv, d]."""
    k_hist = np.asarray(k_hist, dtype=np.float64)
    B, T, Hkv, d = k_hist.shape
    if T % chunk:
        raise ValueError("T must be a multiple of chunk")
    C = T // chunk
    out = np.zeros((B, C, Hkv, d))
    for c in range(C):
        out[:, c] = k_hist[:, c * chunk:(c + 1) * chunk].sum(axis=1) / chunk
    return out


def block_means(q, qblock):
    """Mean query of each block: [B, S, H, d] -> [B, S/qblock, H, d]."""
    q = np.asarray(q, dtype=np.float64)
    B, S, H, d = q.shape
    if S % qblock:
        raise ValueError("S must be a multiple of qblock")
    nqb = S // qblock
    return q.reshape(B, nqb, qblock, H, d).mean(axis=2)


def block_scores(q, summ, qblock):
    """score[b, h, j, c] = qbar[b, j, h] . summ[b, c, kv(h)]  ->  [B, H, NQB, C]."""
    qbar = block_means(q, qblock)
    B, nqb, H, d = qbar.shape
    C, Hkv = summ.shape[1], summ.shape[2]
    sc = np.zeros((B, H, nqb, C))
    for b in range(B):
        for h in range(H):
            sc[b, h] = qbar[b, :, h] @ np.asarray(summ[b, :, kv_head(h, H, Hkv)], np.float64).T
    return sc


def select_topk(scores, topk):
    """Top-k chunk indices per row of ``scores`` [..., C].

    Returns ``(idx, gap)``: idx [..., topk] int32, ascending, ``-1`` padded; gap [...] is
    the k-th best score minus the (k+1)-th (``inf`` when every chunk is selected), the
    margin by which the selected set is decided.
    """
    scores = np.asarray(scores, dtype=np.float64)
    lead = scores.shape[:-1]
    C = scores.shape[-1]
    keff = min(topk, C)
    idx = np.full(lead + (topk,), -1, dtype=np.int32)
    gap = np.full(lead, np.inf)
    if C == 0:
        return idx, gap
    flat = scores.reshape(-1, C)
    fidx = idx.reshape(-1, topk)
    fgap = gap.reshape(-1)
    for r in range(flat.shape[0]):
        # descending by score, ascending by chunk index among equal scores
        order = sorted(range(C), key=lambda c: (-flat[r, c], c))
        chosen = sorted(order[:keff])
        fidx[r, :keff] = chosen
        if keff < C:
            fgap[r] = flat[r, order[keff - 1]] - flat[r, order[keff]]
    return idx, gap


def group_block_scores(q, summ, qblock):
    """Selection shared by the q heads of one kv head: [B, Hkv, NQB, C].

    Reading (the page fixes only that each query block gets a capped selection; whether the
    q heads of a GQA group choose together is open): one chunk list per (batch, kv head,
    query block), ranked by the SUM over the group's q heads of their block scores,
    ``score[b, g, j, c] = sum_{h : kv(h) = g} qbar[b, j, h] . summ[b, c, g]``.  Since every
    head of the group scores against the same summary, this is the dot product of the
    summed block means with it.
    """
    qbar = block_means(q, qblock)
    B, nqb, H, d = qbar.shape
    C, Hkv = summ.shape[1], summ.shape[2]
    sc = np.zeros((B, Hkv, nqb, C))
    for b in range(B):
        for g in range(Hkv):
            qsum = np.zeros((nqb, d))
            for h in range(H):
                if kv_head(h, H, Hkv) == g:
                    qsum += qbar[b, :, h]
            sc[b, g] = qsum @ np.asarray(summ[b, :, g], np.float64).T
    return sc


def expand_group_idx(idx_kv, H):
    """Per-kv-head chunk lists [B, Hkv, NQB, k] -> the per-q-head form [B, H, NQB, k]
    (every q head takes its kv head's list), which the attention functions consume."""
    idx_kv = np.asarray(idx_kv)
    B, Hkv = idx_kv.shape[:2]
    return np.stack([idx_kv[:, kv_head(h, H, Hkv)] for h in range(H)], axis=1)


def stage_plan(idx, Hkv, C, max_slots):
    """Staging of a host-tier history (reading: the page moves the older keys and values to
    host RAM and brings back a bounded set of chunks per query block; here the staging
    history of kv head j holds the union of the chunks named by the lists it serves, in
    ascending order, and every list entry is renamed to its chunk's slot).

    idx [B, lists, NQB, k] with lists = H (list h served by kv head h // (H/Hkv)) or
    lists = Hkv.  Entries outside [0, C) are absent.  -> (chunk_of [B, Hkv, max_slots] with
    -1 past the union, count [B, Hkv], idx_staged shaped like idx with -1 for absent)."""
    idx = np.asarray(idx)
    B, lists = idx.shape[:2]
    rep = lists // Hkv
    chunk_of = np.full((B, Hkv, max_slots), -1, dtype=np.int32)
    count = np.zeros((B, Hkv), dtype=np.int32)
    staged = np.full(idx.shape, -1, dtype=np.int32)
    for b in range(B):
        for j in range(Hkv):
            served = idx[b, j * rep:(j + 1) * rep]
            present = (served >= 0) & (served < C)
            union = sorted({int(c) for c in served[present]})
            if len(union) > max_slots:
                raise ValueError("the union does not fit in max_slots")
            count[b, j] = len(union)
            chunk_of[b, j, :len(union)] = union
            slot = {c: n for n, c in enumerate(union)}
            for pos in zip(*np.nonzero(present)):
                staged[(b, j * rep + pos[0]) + tuple(pos[1:])] = slot[int(served[pos])]
    return chunk_of, count, staged


def stage_update(prev_chunk_of, idx, Hkv, C, max_slots):
    """The staging history kept as a cache across calls (same reading as stage_plan, R20;
    consecutive segments name mostly the same chunks): for each kv head, the slots whose
    chunk its lists still name keep it; the other slots are freed; the named chunks not
    held take the free slots, ascending chunks into ascending slots.  ``prev_chunk_of``
    [B, Hkv, max_slots] is the previous table (-1 = free; distinct chunks).  -> (chunk_of,
    count [B, Hkv] = distinct named chunks, copied [B, Hkv] = chunks newly placed,
    idx_staged: every present entry renamed to its chunk's slot, -1 for absent)."""
    idx = np.asarray(idx)
    prev = np.asarray(prev_chunk_of)
    B, lists = idx.shape[:2]
    rep = lists // Hkv
    chunk_of = np.full((B, Hkv, max_slots), -1, dtype=np.int32)
    count = np.zeros((B, Hkv), dtype=np.int32)
    copied = np.zeros((B, Hkv), dtype=np.int32)
    staged = np.full(idx.shape, -1, dtype=np.int32)
    for b in range(B):
        for j in range(Hkv):
            served = idx[b, j * rep:(j + 1) * rep]
            present = (served >= 0) & (served < C)
            named = {int(c) for c in served[present]}
            slot = {}
            free = []
            for s in range(max_slots):
                c = int(prev[b, j, s])
                if c in named:
                    chunk_of[b, j, s] = c
                    slot[c] = s
                else:
                    free.append(s)
            missing = sorted(named - set(slot))
            if len(missing) > len(free):
                raise ValueError("the named chunks do not fit in max_slots")
            for c, s in zip(missing, free):
                chunk_of[b, j, s] = c
                slot[c] = s
            count[b, j], copied[b, j] = len(named), len(missing)
            for pos in zip(*np.nonzero(present)):
                staged[(b, j * rep + pos[0]) + tuple(pos[1:])] = slot[int(served[pos])]
    return chunk_of, count, copied, staged


def stage_history(hist, chunk_of, chunk):
    """Staging rows for history [B, T, Hkv, d]: rows [s*chunk, (s+1)*chunk) of kv head j
    are the rows of chunk chunk_of[b, j, s] of kv head j (zero for unused slots)."""
    hist = np.asarray(hist)
    B, _, Hkv, d = hist.shape
    slots = chunk_of.shape[2]
    out = np.zeros((B, slots * chunk, Hkv, d), dtype=hist.dtype)
    for b in range(B):
        for j in range(Hkv):
            for s in range(slots):
                c = int(chunk_of[b, j, s])
                if c >= 0:
                    out[b, s * chunk:(s + 1) * chunk, j] = hist[b, c * chunk:(c + 1) * chunk, j]
    return out


def block_key_set(j, qblock, chunk, idx_row):
    """Key set of query block j: (history token indices, number of active keys).

    History tokens: every token of each selected chunk (``idx_row`` entries >= 0), in
    index order.  Active keys: positions ``[0, (j+1)*qblock)``; query ``t`` of the block
    sees active key ``u`` iff ``u <= t``.
    """
    sel = [int(c) for c in idx_row if c >= 0]
    hist = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in sel]) if sel \
        else np.zeros(0, dtype=np.int64)
    return hist, (j + 1) * qblock


def _block(q, k_act, v_act, k_hist, v_hist, idx, b, h, j, chunk, qblock, scale, do=None):
    B, S, H, d = q.shape
    Hkv = k_act.shape[2]
    kv = kv_head(h, H, Hkv)
    hist, nloc = block_key_set(j, qblock, chunk, idx[b, h, j])
    rows = np.arange(j * qblock, (j + 1) * qblock)
    keys = np.concatenate([np.asarray(k_hist[b, hist, kv], np.float64).reshape(-1, d),
                           np.asarray(k_act[b, :nloc, kv], np.float64)])
    vals = np.concatenate([np.asarray(v_hist[b, hist, kv], np.float64).reshape(-1, d),
                           np.asarray(v_act[b, :nloc, kv], np.float64)])
    nh = hist.shape[0]
    mask = np.ones((qblock, nh + nloc), dtype=bool)
    mask[:, nh:] = np.arange(nloc)[None, :] <= rows[:, None]
    qb = np.asarray(q[b, rows, h], np.float64)
    o, lse = masked_attention(qb, keys, vals, mask, scale)
    if do is None:
        return rows, o, lse
    gq, gk, gv = masked_attention_bwd(qb, keys, vals, mask, scale, o, lse, do[b, rows, h])
    return rows, o, lse, gq, gk[nh:], gv[nh:], nloc


def hga_fwd(q, k_act, v_act, k_hist, v_hist, idx, chunk, qblock, scale, heads=None):
    """Forward over every (batch, head, block), or only the listed heads.  -> (O, LSE)."""
    B, S, H, d = q.shape
    o = np.zeros((B, S, H, d))
    lse = np.zeros((B, H, S))
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            for j in range(S // qblock):
                rows, go, gl = _block(q, k_act, v_act, k_hist, v_hist, idx, b, h, j, chunk, qblock, scale)
                o[b, rows, h] = go
                lse[b, h, rows] = gl
    return o, lse


def hga_bwd(q, k_act, v_act, k_hist, v_hist, idx, do, chunk, qblock, scale):
    """Forward plus active-only backward.  -> (O, LSE, dQ, dK_act, dV_act)."""
    B, S, H, d = q.shape
    Hkv = k_act.shape[2]
    o = np.zeros((B, S, H, d))
    lse = np.zeros((B, H, S))
    dq = np.zeros((B, S, H, d))
    dk = np.zeros((B, S, Hkv, d))
    dv = np.zeros((B, S, Hkv, d))
    for b in range(B):
        for h in range(H):
            kv = kv_head(h, H, Hkv)
            for j in range(S // qblock):
                rows, go, gl, gq, gk, gv, nloc = _block(q, k_act, v_act, k_hist, v_hist, idx, b, h, j,
                                                        chunk, qblock, scale, do=do)
                o[b, rows, h] = go
                lse[b, h, rows] = gl
                dq[b, rows, h] = gq
                dk[b, :nloc, kv] += gk
                dv[b, :nloc, kv] += gv
    return o, lse, dq, dk, dv


def decode(q, k_act, v_act, k_hist, v_hist, idx, chunk, scale):
    """Generation step: the last ``nq`` tokens of an active segment of ``Sa`` tokens.

    Reading (the page says only that the method also serves generation): query i of
    ``q [B, nq, H, d]`` sits at segment position ``t = Sa - nq + i`` and attends, under one
    softmax, to the active keys ``u <= t`` of ``k_act/v_act [B, Sa, Hkv, d]`` and to every
    token of the chunks listed in ``idx [B, H, topk]`` (the lists of its query block, as
    chosen by the caller; -1 = none).  With ``Sa`` a multiple of the query block and
    ``nq`` rows of the last block this is ``hga_fwd`` on those rows.  -> (O [B, nq, H, d],
    LSE [B, H, nq]).
    """
    q = np.asarray(q, np.float64)
    B, nq, H, d = q.shape
    Sa, Hkv = k_act.shape[1], k_act.shape[2]
    o = np.zeros((B, nq, H, d))
    lse = np.zeros((B, H, nq))
    t = Sa - nq + np.arange(nq)
    for b in range(B):
        for h in range(H):
            kv = kv_head(h, H, Hkv)
            sel = [int(c) for c in idx[b, h] if c >= 0]
            hist = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in sel]) if sel \
                else np.zeros(0, dtype=np.int64)
            keys = np.concatenate([np.asarray(k_hist[b, hist, kv], np.float64).reshape(-1, d),
                                   np.asarray(k_act[b, :, kv], np.float64)])
            vals = np.concatenate([np.asarray(v_hist[b, hist, kv], np.float64).reshape(-1, d),
                                   np.asarray(v_act[b, :, kv], np.float64)])
            nh = hist.shape[0]
            mask = np.ones((nq, nh + Sa), dtype=bool)
            mask[:, nh:] = np.arange(Sa)[None, :] <= t[:, None]
            o[b, :, h], lse[b, h] = masked_attention(q[b, :, h], keys, vals, mask, scale)
    return o, lse


def full_mask(S, T, chunk, qblock, idx_bh):
    """Brute-force [S, T + S] visibility mask of one (batch, head) over [history; active]."""
    m = np.zeros((S, T + S), dtype=bool)
    for t in range(S):
        j = t // qblock
        for c in idx_bh[j]:
            if c >= 0:
                m[t, c * chunk:(c + 1) * chunk] = True
        m[t, T:T + t + 1] = True
    return m


def hga_fwd_bruteforce(q, k_act, v_act, k_hist, v_hist, idx, chunk, qblock, scale):
    """Forward with the full mask over the concatenated keys.  Small shapes only."""
    B, S, H, d = q.shape
    T, Hkv = k_hist.shape[1], k_hist.shape[2]
    o = np.zeros((B, S, H, d))
    lse = np.zeros((B, H, S))
    for b in range(B):
        for h in range(H):
            kv = kv_head(h, H, Hkv)
            keys = np.concatenate([k_hist[b, :, kv], k_act[b, :, kv]]).astype(np.float64)
            vals = np.concatenate([v_hist[b, :, kv], v_act[b, :, kv]]).astype(np.float64)
            o[b, :, h], lse[b, h] = masked_attention(q[b, :, h], keys, vals,
                                                     full_mask(S, T, chunk, qblock, idx[b, h]), scale)
    return o, lse


def long_eval(q, k, v, seg, chunk, qblock, topk, scale, segments, heads, shared=False):
    """Segment-by-segment forward over one long sequence with running summaries.

    Segment s covers tokens ``[s*seg, (s+1)*seg)``; its history is every earlier token;
    the resident summaries are appended one segment at a time (16 chunks per 2048-token
    segment at chunk 128), so segment s selects among ``s * seg / chunk`` chunks.
    Returns ``{s: (idx, gap, O[heads], LSE[heads], scores)}`` for the requested segments
    and heads; ``scores`` are the block scores the selection ranked (``None`` while the
    history is empty).  With ``shared`` the lists are per kv head (summed scores of its q
    heads), as in ``train_segments``.
    """
    B, L, H, d = q.shape
    Hkv = k.shape[2]
    nseg = L // seg
    want = set(segments)
    summ = np.zeros((B, 0, Hkv, d))
    out = {}
    for s in range(nseg):
        if s in want:
            lo, hi = s * seg, (s + 1) * seg
            qs = q[:, lo:hi]
            nl = Hkv if shared else H
            sc = None
            if summ.shape[1]:
                sc = group_block_scores(qs, summ, qblock) if shared else block_scores(qs, summ, qblock)
                idx, gap = select_topk(sc, topk)
            else:
                idx = np.full((B, nl, seg // qblock, topk), -1, dtype=np.int32)
                gap = np.full((B, nl, seg // qblock), np.inf)
            use = expand_group_idx(idx, H) if shared else idx
            o, lse = hga_fwd(qs, k[:, lo:hi], v[:, lo:hi], k[:, :lo], v[:, :lo], use, chunk, qblock,
                             scale, heads=heads)
            out[s] = (idx, gap, o[:, :, list(heads)], lse[:, list(heads)], sc)
        if s + 1 < nseg and max(want) > s:
            summ = np.concatenate([summ, summarize(k[:, s * seg:(s + 1) * seg], chunk)], axis=1)
    return out


def train_segments(q, k, v, do, seg, chunk, qblock, topk, scale, idx_given=None, shared=False):
    """Segment-wise training pass over one long sequence (the page's training regime).

    Segment s (tokens ``[s*seg, (s+1)*seg)``) is the active, differentiable segment; every
    earlier token is detached history.  Its resident summaries hold the chunks of all
    earlier segments, appended one segment at a time after that segment's step.  Per
    segment: select on the resident summaries (``idx_given[s]`` replaces the selection
    when given, e.g. to follow another implementation's choice at a near tie), attend,
    and backpropagate into the active segment only (history keys get no gradient).

    With ``shared`` the selection is one list per (kv head, block) from the summed scores of
    the kv head's q heads (``group_block_scores``), and every q head attends to its kv
    head's list; idx (and ``idx_given``) are then per kv head.

    Returns (per-segment list of dicts with idx, gap, scores (the ranked block scores,
    ``None`` while the history is empty), o, lse, dq, dk, dv; the summaries after the last
    append, covering the whole sequence).
    """
    B, L, H, d = q.shape
    Hkv = k.shape[2]
    if L % seg or seg % qblock or seg % chunk:
        raise ValueError("L, seg, qblock and chunk must nest")
    summ = np.zeros((B, 0, Hkv, d))
    out = []
    for s in range(L // seg):
        lo, hi = s * seg, (s + 1) * seg
        qs = q[:, lo:hi]
        nl = Hkv if shared else H
        sc = None
        if summ.shape[1]:
            sc = group_block_scores(qs, summ, qblock) if shared else block_scores(qs, summ, qblock)
            idx, gap = select_topk(sc, topk)
        else:
            idx = np.full((B, nl, seg // qblock, topk), -1, dtype=np.int32)
            gap = np.full((B, nl, seg // qblock), np.inf)
        use = idx if idx_given is None else np.asarray(idx_given[s])
        if shared:
            use = expand_group_idx(use, H)
        o, lse, dq, dk, dv = hga_bwd(qs, k[:, lo:hi], v[:, lo:hi], k[:, :lo], v[:, :lo], use, do[:, lo:hi],
                                     chunk, qblock, scale)
        out.append(dict(idx=idx, gap=gap, scores=sc, o=o, lse=lse, dq=dq, dk=dk, dv=dv))
        # the finished segment is detached into the history: append its summaries
        summ = np.concatenate([summ, summarize(k[:, lo:hi], chunk)], axis=1)
    return out, summ
