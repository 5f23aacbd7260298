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
* ``hga_host_step`` / ``hga_host_segments``: the same with the detached history in pinned
  host memory (same page: older keys and values move to host RAM): per segment the
  selected chunks are gathered into an HBM staging history that the attention reads;
  with ``overlap`` the detach, selection and gathering of the next segment run on a
  second stream while the current segment attends.
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
                  ws=torch.empty(max(16, ops.hga_bwd_workspace_bytes_dsq(1, seg, H, Hkv, d)), dtype=torch.uint8,
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


_PIPE_STREAMS = {}


def _pipeline_streams(dev):
    """Three streams of the host-history pipeline (attention, gathering, detaching), made
    once per device in one go.  Streams made in a row get distinct hardware queues (the
    runtime hands queues out in turn), so work on them can run side by side; two streams
    that share a queue run one after the other whatever their events say."""
    key = torch.device(dev).index or 0
    if key not in _PIPE_STREAMS:
        _PIPE_STREAMS[key] = tuple(torch.cuda.Stream(device=dev) for _ in range(3))
    return _PIPE_STREAMS[key]


def hga_host_step(q, k_act, v_act, k_host, v_host, summ, do, T, chunk=128, qblock=64, topk=8, scale=None,
                  shared=False, workspace=None, idx=None, staging=None):
    """One HGA training segment over a history of ``T`` tokens held in pinned host memory.

    ``k_host``/``v_host`` [B, >= T, Hkv, d] pinned; ``summ`` [B, >= T/chunk, Hkv, d] on the
    GPU (as hga_detach_segment keeps it).  Selects from the summaries (unless ``idx`` is
    given), gathers the selected chunks into an HBM staging history (``staging`` may carry
    the buffers, as keyword arguments of ops.hga_stage_selected), then runs the forward
    and the backward on it.  Returns a dict with idx, the staging outputs and o, lse, dq,
    dk, dv."""
    select, fwd, bwd = _hga_ops(shared)
    if idx is None:
        idx = select(q, summ[:, :T // chunk], qblock, topk)
    ks, vs, ist, cof, cnt = ops.hga_stage_selected(idx, k_host, v_host, T, chunk, **(staging or {}))
    o, lse = fwd(q, k_act, v_act, ks, vs, ist, chunk, qblock, scale)
    dq, dk, dv = bwd(q, k_act, v_act, ks, vs, ist, o, lse, do, chunk, qblock, scale, workspace=workspace)
    return dict(idx=idx, idx_staged=ist, chunk_of=cof, count=cnt, k_stage=ks, v_stage=vs, o=o, lse=lse, dq=dq,
                dk=dk, dv=dv)


def hga_host_segments(q, k, v, do=None, seg=2048, chunk=128, qblock=64, topk=8, scale=None, shared=False,
                      overlap=True, cached=True, state=None):
    """Segment-wise HGA pass over ``q`` [1, L, H, d], ``k``/``v`` [1, L, Hkv, d] with the
    detached history in pinned host memory: training (forward and backward per segment)
    when ``do`` is given, evaluation (forward only) otherwise.

    Segment s: its lists are selected from the HBM summaries of tokens [0, s*seg), the
    chunks they name are gathered from host memory into one of two HBM staging histories,
    and the segment attends (and backpropagates) on that staging history.  Its own keys
    and values are detached into host memory (hga_detach_segment: rows and summaries) as
    soon as they exist, since nothing of the segment's attention feeds them; at the end
    the host history holds all L tokens.  With ``overlap`` three streams run side by side:
    the detaches (host writes), the selection and gathering (host reads) of segment s + 1,
    and the attention of segment s; the gathering for s + 2 waits until segment s is done
    with its staging buffer.  With ``cached`` each staging buffer keeps the chunks it
    holds (hga_stage_update): a segment copies only the chunks its lists name that the
    buffer does not hold from two segments before.  Results equal hga_train_segments (or
    hga_long_eval) bit for bit.

    Returns the state dict: o, lse [nseg, 1, H, seg], idx [nseg, 1, H or Hkv, seg/qblock,
    topk], k_host/v_host (pinned), summ, the staging buffers, and dq/dk/dv when training.
    """
    B, L, H, d = q.shape
    if B != 1:
        raise ValueError("hga_host_segments works on one sequence (batch 1)")
    Hkv = k.shape[2]
    nseg = L // seg
    if nseg * seg != L or seg % chunk or seg % qblock:
        raise ValueError("L must be a multiple of seg, and seg of chunk and qblock")
    cps, nqb = seg // chunk, seg // qblock
    lists = Hkv if shared else H
    slots = ops.hga_stage_slots(lists, Hkv, nqb, topk, (nseg - 1) * cps)
    select, fwd, bwd = _hga_ops(shared)
    dev = q.device
    st = state if state is not None else {}
    if not st:
        st.update(o=torch.empty_like(q), lse=torch.empty((nseg, 1, H, seg), dtype=torch.float32, device=dev),
                  idx=torch.empty((nseg, 1, lists, nqb, topk), dtype=torch.int32, device=dev),
                  k_host=ops.pinned_empty(tuple(k.shape)), v_host=ops.pinned_empty(tuple(v.shape)),
                  summ=torch.empty((1, L // chunk, Hkv, d), dtype=torch.float32, device=dev),
                  # two staging sets, each buffer its own allocation (16-byte aligned)
                  k_stage=[torch.empty((1, slots * chunk, Hkv, d), dtype=torch.bfloat16, device=dev)
                           for _ in range(2)],
                  v_stage=[torch.empty((1, slots * chunk, Hkv, d), dtype=torch.bfloat16, device=dev)
                           for _ in range(2)],
                  idx_staged=[torch.empty((1, lists, nqb, topk), dtype=torch.int32, device=dev) for _ in range(2)],
                  chunk_of=[torch.full((1, Hkv, slots), -1, dtype=torch.int32, device=dev) for _ in range(2)],
                  count=[torch.empty((1, Hkv), dtype=torch.int32, device=dev) for _ in range(2)],
                  copied=[torch.zeros((1, Hkv), dtype=torch.int32, device=dev) for _ in range(2)],
                  copy_list=[torch.empty((1, Hkv, slots), dtype=torch.int32, device=dev) for _ in range(2)])
        if do is not None:
            st.update(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                      ws=torch.empty(max(16, ops.hga_bwd_workspace_bytes_dsq(1, seg, H, Hkv, d)), dtype=torch.uint8,
                                     device=dev))
    caller = torch.cuda.current_stream(dev)
    for t in st["chunk_of"]:
        t.fill_(-1)   # a new pass brings its own history: the staging buffers start empty
    if overlap:
        main, side, det = _pipeline_streams(dev)
    else:
        main = side = det = caller
    staged = [torch.cuda.Event(), torch.cuda.Event()]
    done = [torch.cuda.Event(), torch.cuda.Event()]
    detached = [torch.cuda.Event() for _ in range(nseg)]
    for x in {main, side, det}:
        x.wait_stream(caller)
    for s in range(nseg):
        lo, hi = s * seg, (s + 1) * seg
        buf = s % 2
        with torch.cuda.stream(det):
            # rows [lo, hi) and their summaries; read by the selection and gathering of later
            # segments only
            ops.hga_detach_segment(k[:, lo:hi], v[:, lo:hi], st["k_host"], st["v_host"], st["summ"], lo, chunk)
            detached[s].record(det)
        with torch.cuda.stream(side):
            if s > 0:
                side.wait_event(detached[s - 1])
            select(q[:, lo:hi], st["summ"][:, :s * cps], qblock, topk, idx=st["idx"][s])
            if s >= 2:
                side.wait_event(done[buf])
            if cached:
                ops.hga_stage_update(st["idx"][s], st["k_host"], st["v_host"], lo, chunk, st["chunk_of"][buf],
                                     st["k_stage"][buf], st["v_stage"][buf], idx_staged=st["idx_staged"][buf],
                                     count=st["count"][buf], copied=st["copied"][buf],
                                     copy_list=st["copy_list"][buf])
            else:
                ops.hga_stage_selected(st["idx"][s], st["k_host"], st["v_host"], lo, chunk, slots,
                                       k_stage=st["k_stage"][buf], v_stage=st["v_stage"][buf],
                                       idx_staged=st["idx_staged"][buf], chunk_of=st["chunk_of"][buf],
                                       count=st["count"][buf])
            staged[buf].record(side)
        with torch.cuda.stream(main):
            main.wait_event(staged[buf])
            ks, vs, ist = st["k_stage"][buf], st["v_stage"][buf], st["idx_staged"][buf]
            o, lse = fwd(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], ks, vs, ist, chunk, qblock, scale,
                         o=st["o"][:, lo:hi], lse=st["lse"][s])
            if do is not None:
                bwd(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], ks, vs, ist, o, lse, do[:, lo:hi], chunk, qblock, scale,
                    workspace=st["ws"], dq=st["dq"][:, lo:hi], dk_act=st["dk"][:, lo:hi], dv_act=st["dv"][:, lo:hi])
            done[buf].record(main)
    for x in {main, side, det}:
        caller.wait_stream(x)
    return st
