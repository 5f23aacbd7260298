"""Host-side sequencing of the C-ABI calls into the two hot paths.

Only ordering and buffer slicing happen here; every arithmetic step runs in libs2a.so.

* ``s2attn_step``: shifted short attention forward + backward of one layer.
* ``hga_train_step``: one HGA training segment ("Long-Context Fine-Tuning with Limited
  VRAM", English abstract): summarise the detached history, select chunks per query
  block, attend, and backpropagate into the active segment only.
* ``hga_long_eval``: forward-only evaluation over a long sequence processed segment by
  segment; the resident summaries grow by one segment's chunks after every segment.
* ``hga_train_segments``: the segment-wise training pass: per segment select, attend,
  backpropagate into the active segment, then detach the segment into the resident
  history (keys, values and summaries) with one append.
"""
from __future__ import annotations

import torch

from . import ops


def s2attn_step(q, k, v, do, G, shift=True, scale=None, workspace=None):
    o, lse = ops.s2attn_fwd(q, k, v, G, shift, scale)
    dq, dk, dv = ops.s2attn_bwd(q, k, v, o, lse, do, G, shift, scale, workspace=workspace)
    return o, lse, dq, dk, dv


def _hga_ops(shared):
    """(select, forward, backward) for per-q-head chunk lists or, with ``shared``, one list
    per kv head used by all of its q heads."""
    if shared:
        return ops.hga_select_topk_shared, ops.hga_fwd_shared, ops.hga_bwd_active_shared
    return ops.hga_select_topk, ops.hga_fwd, ops.hga_bwd_active


def hga_train_step(q, k_act, v_act, k_hist, v_hist, do, chunk=128, qblock=64, topk=8, scale=None,
                   workspace=None, shared=False):
    select, fwd, bwd = _hga_ops(shared)
    summ = ops.hga_summarize(k_hist, chunk)
    idx = select(q, summ, qblock, topk)
    o, lse = fwd(q, k_act, v_act, k_hist, v_hist, idx, chunk, qblock, scale)
    dq, dk, dv = bwd(q, k_act, v_act, k_hist, v_hist, idx, o, lse, do, chunk, qblock, scale, workspace=workspace)
    return dict(summ=summ, idx=idx, o=o, lse=lse, dq=dq, dk=dk, dv=dv)


def hga_long_eval(q, k, v, seg=2048, chunk=128, qblock=64, topk=16, scale=None, o=None, lse=None,
                  summ=None, idx_all=None, shared=False, fused=False):
    """Segment-by-segment forward over ``q [1, L, H, d]``, ``k/v [1, L, Hkv, d]``.

    Segment s attends causally to itself plus the selected chunks of tokens
    ``[0, s*seg)``.  Returns ``(o, lse, idx_all)`` with ``o [1, L, H, d]``, ``lse [nseg, 1,
    H, seg]`` and ``idx_all [nseg, 1, H, seg/qblock, topk]``.  Every per-segment operand is
    a contiguous view of the full buffers (batch 1), so nothing is copied; buffers may be
    passed in to keep allocation out of timed loops.  With ``shared`` each kv head selects
    one chunk list for all of its q heads (idx_all then has Hkv rows per segment); with
    ``fused`` as well, each segment's selection runs inside its forward launch.
    """
    if fused and not shared:
        raise ValueError("the fused selection works on chunk lists shared per kv head")
    B, L, H, d = q.shape
    if B != 1:
        raise ValueError("hga_long_eval works on one sequence (batch 1)")
    Hkv = k.shape[2]
    nseg = L // seg
    cps = seg // chunk
    dev = q.device
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((nseg, B, H, seg), dtype=torch.float32, device=dev) if lse is None else lse
    summ = torch.empty((B, L // chunk, Hkv, d), dtype=torch.float32, device=dev) if summ is None else summ
    idx_all = (torch.empty((nseg, B, Hkv if shared else H, seg // qblock, topk), dtype=torch.int32, device=dev)
               if idx_all is None else idx_all)
    select, fwd, _ = _hga_ops(shared)
    for s in range(nseg):
        lo, hi = s * seg, (s + 1) * seg
        if s > 0:
            # append the previous segment's chunk summaries to the resident table
            ops.hga_summarize(k[:, lo - seg:lo], chunk, summ[:, (s - 1) * cps:s * cps])
        if fused:
            ops.hga_fwd_select_shared(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], k[:, :lo], v[:, :lo], summ[:, :s * cps],
                                      chunk, qblock, topk, scale, idx=idx_all[s], o=o[:, lo:hi], lse=lse[s])
            continue
        select(q[:, lo:hi], summ[:, :s * cps], qblock, topk, idx=idx_all[s])
        fwd(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], k[:, :lo], v[:, :lo], idx_all[s], chunk, qblock, scale,
            o=o[:, lo:hi], lse=lse[s])
    return o, lse, idx_all


def hga_train_segments(q, k, v, do, seg=2048, chunk=128, qblock=64, topk=8, scale=None, state=None,
                       shared=False, idx_given=None):
    """Segment-wise HGA training pass over ``q``/``do`` [1, L, H, d] and ``k``/``v`` [1, L, Hkv, d].

    Segment s (tokens ``[s*seg, (s+1)*seg)``) is active and differentiable; the tokens of
    earlier segments live, detached, in a history buffer owned by this driver, together
    with the summaries of their chunks.  Per segment: top-k chunks per query block from
    the summaries, the HGA forward over the local causal keys and the selected history,
    the backward into the active segment, and finally the append of the segment's keys,
    values and summaries to the history.

    ``state`` may carry preallocated buffers (as returned) to keep allocation out of
    timed loops.  With ``shared`` each kv head selects one chunk list for all of its q
    heads.  ``idx_given`` (int32 device tensor [nseg, 1, H or Hkv, seg/qblock, topk])
    replaces the selection step: its lists are copied into ``idx`` and attended instead,
    e.g. to run the pass on another implementation's choices at near ties.  Returns a dict with o [1, L, H, d], lse [nseg, 1, H, seg], idx [nseg, 1,
    H (Hkv when shared), seg/qblock, topk], dq [1, L, H, d], dk/dv [1, L, Hkv, d], and the history k_hist,
    v_hist [1, L, Hkv, d] and summ [1, L/chunk, Hkv, d].
    """
    B, L, H, d = q.shape
    if B != 1:
        raise ValueError("hga_train_segments works on one sequence (batch 1)")
    Hkv = k.shape[2]
    nseg = L // seg
    if nseg * seg != L:
        raise ValueError("L must be a multiple of seg")
    dev = q.device
    select, fwd, bwd = _hga_ops(shared)
    st = state if state is not None else {}
    if not st:
        st.update(o=torch.empty_like(q), lse=torch.empty((nseg, 1, H, seg), dtype=torch.float32, device=dev),
                  idx=torch.empty((nseg, 1, Hkv if shared else H, seg // qblock, topk), dtype=torch.int32,
                                  device=dev),
                  dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                  k_hist=torch.empty_like(k), v_hist=torch.empty_like(v),
                  summ=torch.empty((1, L // chunk, Hkv, d), dtype=torch.float32, device=dev),
                  ws=torch.empty(max(16, ops.hga_bwd_workspace_bytes(1, seg, H, Hkv, d)), dtype=torch.uint8,
                                 device=dev))
    kh, vh, summ = st["k_hist"], st["v_hist"], st["summ"]
    for s in range(nseg):
        lo, hi = s * seg, (s + 1) * seg
        C = lo // chunk
        qs, ks, vs, dos = q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], do[:, lo:hi]
        if idx_given is None:
            select(qs, summ[:, :C], qblock, topk, idx=st["idx"][s])
        else:
            st["idx"][s].copy_(idx_given[s])
        o, lse = fwd(qs, ks, vs, kh[:, :lo], vh[:, :lo], st["idx"][s], chunk, qblock, scale, o=st["o"][:, lo:hi],
                     lse=st["lse"][s])
        bwd(qs, ks, vs, kh[:, :lo], vh[:, :lo], st["idx"][s], o, lse, dos, chunk, qblock, scale, workspace=st["ws"],
            dq=st["dq"][:, lo:hi], dk_act=st["dk"][:, lo:hi], dv_act=st["dv"][:, lo:hi])
        ops.hga_append_history(ks, vs, kh, vh, summ, lo, chunk)
    return st
