"""GPU parity of the host-tier history (older K/V rows in pinned host memory): the staging
plan and gather against the oracle's staging (bit-exact), attention on the staging
history against attention on the resident history (same bits), the detach against the
resident append, the 16K step with its history in host memory against the oracle, and the
segment pipelines against the resident ones."""
import numpy as np
import pytest
import torch

from block_sparse_attention_41_amd import synth
from block_sparse_attention_41_amd.workload import CONFIGS
from oracle import hga as OH

from gpu_util import GRAD_RTOL, LSE_ATOL, O_ATOL, max_abs, rel_fro, to_dev, to_f64
from test_gpu_hga import _ids, _setup
from test_gpu_hga_shared import SHARED_CASES

pytestmark = pytest.mark.gpu

i16 = lambda t: t.view(torch.int16)  # noqa: E731


def _pinned(t):
    from block_sparse_attention_41_amd import ops
    h = ops.pinned_empty(tuple(t.shape))
    h.copy_(t)
    torch.cuda.synchronize()
    return h


def _lists(B, lists, nqb, C, topk, seed):
    idx = synth.random_topk_indices(B, lists, nqb, max(C, 1), topk, seed=seed, fill=0.6)
    if C == 0:
        idx[:] = -1
    else:
        idx[0, 0, 0, -1] = C + 5          # out of range: counts as absent
    return idx


@pytest.mark.parametrize("case", SHARED_CASES, ids=_ids)
@pytest.mark.parametrize("shared", [False, True], ids=["per_head", "shared"])
def test_staging_matches_oracle_and_attention_keeps_its_bits(case, shared):
    from block_sparse_attention_41_amd import ops
    B, S, T, H, Hkv, d, chunk, topk = case
    dev, _ = _setup(case, seed=21)
    C, nqb = T // chunk, S // 64
    lists = Hkv if shared else H
    kh, vh = _pinned(dev["k_hist"]), _pinned(dev["v_hist"])
    ridx = _lists(B, lists, nqb, C, topk, seed=22)
    idx = torch.from_numpy(ridx).to("cuda:0")
    ks, vs, ist, cof, cnt = ops.hga_stage_selected(idx, kh, vh, T, chunk)
    torch.cuda.synchronize()
    slots = cof.shape[-1]
    rco, rcnt, rst = OH.stage_plan(ridx, Hkv, C, slots)
    assert np.array_equal(cof.cpu().numpy(), rco) and np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(ist.cpu().numpy(), rst)
    # the staged rows of every used slot, bit for bit
    hk, hv = i16(kh).numpy(), i16(vh).numpy()
    gk, gv = i16(ks).cpu().numpy(), i16(vs).cpu().numpy()
    for b in range(B):
        for j in range(Hkv):
            for s in range(int(rcnt[b, j])):
                c = int(rco[b, j, s])
                rows, src = slice(s * chunk, (s + 1) * chunk), slice(c * chunk, (c + 1) * chunk)
                assert np.array_equal(gk[b, rows, j], hk[b, src, j]) and np.array_equal(gv[b, rows, j], hv[b, src, j])
    # forward and backward on the staging history = on the resident history
    scale = d ** -0.5
    fwd = ops.hga_fwd_shared if shared else ops.hga_fwd
    bwd = ops.hga_bwd_active_shared if shared else ops.hga_bwd_active
    res = (dev["k_hist"], dev["v_hist"], idx)
    stg = (ks, vs, ist)
    outs = []
    for kk, vv, ii in (res, stg):
        o, lse = fwd(dev["q"], dev["k_act"], dev["v_act"], kk, vv, ii, chunk, 64, scale)
        g = bwd(dev["q"], dev["k_act"], dev["v_act"], kk, vv, ii, o, lse, dev["do"], chunk, 64, scale)
        outs.append((o, lse) + tuple(g))
    for a, b_ in zip(*outs):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else i16(a),
                           b_.view(torch.int32) if b_.dtype == torch.float32 else i16(b_))


@pytest.mark.parametrize("d", [64, 128])
def test_detach_writes_the_host_history_and_the_summaries_of_the_append(d):
    from block_sparse_attention_41_amd import ops
    B, S, T, Hkv, chunk = 2, 256, 512, 2, 128
    inp = synth.hga_inputs(B, S, T, 2 * Hkv, Hkv, d, seed=31)
    kf, vf = to_dev(inp["k_full"]), to_dev(inp["v_full"])
    ks, vs = kf[:, T:], vf[:, T:]
    k_host = ops.pinned_empty((B, T + S + 128, Hkv, d))
    v_host = ops.pinned_empty((B, T + S + 128, Hkv, d))
    k_host.fill_(7.0)
    v_host.fill_(-3.0)
    summ = torch.full((B, (T + S) // chunk, Hkv, d), 5.0, device="cuda:0")
    ops.hga_detach_segment(ks, vs, k_host, v_host, summ, T, chunk)
    kd, vd = torch.zeros_like(kf), torch.zeros_like(vf)
    summ2 = torch.full_like(summ, 5.0)
    ops.hga_append_history(ks, vs, kd, vd, summ2, T, chunk)
    torch.cuda.synchronize()
    assert torch.equal(i16(k_host[:, T:T + S]), i16(ks.cpu())) and torch.equal(i16(v_host[:, T:T + S]), i16(vs.cpu()))
    assert bool((k_host[:, :T] == 7.0).all()) and bool((k_host[:, T + S:] == 7.0).all())
    assert bool((v_host[:, :T] == -3.0).all()) and bool((v_host[:, T + S:] == -3.0).all())
    assert torch.equal(summ, summ2)


def test_host_history_rejects_device_and_pageable_memory():
    from block_sparse_attention_41_amd import ops
    idx = torch.zeros((1, 2, 2, 4), dtype=torch.int32, device="cuda:0")
    kd = torch.zeros((1, 512, 2, 64), dtype=torch.bfloat16, device="cuda:0")
    kp = torch.zeros((1, 512, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        ops.hga_stage_selected(idx, kd, kd, 512, 128)
    with pytest.raises(TypeError):
        ops.hga_stage_selected(idx, kp, kp, 512, 128)
    # through the C ABI directly: device memory and pageable memory are rejected
    lib = ops.lib()
    out = torch.zeros((1, 2, 8), dtype=torch.int32, device="cuda:0")
    stage = torch.zeros((1, 8 * 128, 2, 64), dtype=torch.bfloat16, device="cuda:0")
    for p in (kd.data_ptr(), kp.data_ptr()):
        st = lib.hga_stage_selected(idx.data_ptr(), 2, 2, 4, p, p, 512 * 128, 512, out.data_ptr(), out.data_ptr(),
                                    out.data_ptr(), stage.data_ptr(), stage.data_ptr(), 0, 4, 1, 2, 64, 128, None)
        assert st == 1
    torch.cuda.synchronize()


@pytest.mark.parametrize("shared", [False, True], ids=["per_head", "shared"])
def test_host_step_full_size_matches_oracle(shared):
    """The 16K step (history of 14336 tokens in host memory) on the oracle's chunk lists:
    O/LSE/dQ/dK/dV against the oracle on two sampled kv groups; the pipeline's own step
    (its own selection) equals the resident step bit for bit."""
    from block_sparse_attention_41_amd import ops, pipeline
    cfg = CONFIGS["c4"]
    B, S, T, H, Hkv, d = cfg.B, cfg.S, cfg.T, cfg.H, cfg.Hkv, cfg.d
    inp = synth.hga_inputs(B, S, T, H, Hkv, d, seed=5)
    kf, vf = to_dev(inp["k_full"]), to_dev(inp["v_full"])
    q, do = to_dev(inp["q"]), to_dev(inp["do"])
    kh, vh = _pinned(kf[:, :T]), _pinned(vf[:, :T])
    summ = ops.hga_summarize(kf[:, :T], cfg.chunk)
    q32 = synth.bf16_to_f32(inp["q"])
    k32, v32 = synth.bf16_to_f32(inp["k_full"]), synth.bf16_to_f32(inp["v_full"])
    do32 = synth.bf16_to_f32(inp["do"])
    score = OH.group_block_scores if shared else OH.block_scores
    ridx, _ = OH.select_topk(score(q32, OH.summarize(k32[:, :T], cfg.chunk), cfg.qblock), cfg.topk)
    tidx = torch.from_numpy(ridx).to("cuda:0")
    r = pipeline.hga_host_step(q, kf[:, T:], vf[:, T:], kh, vh, summ, do, T, cfg.chunk, cfg.qblock, cfg.topk,
                               cfg.scale, shared=shared, idx=tidx)
    go, gl, gdq, gdk, gdv = (to_f64(r[n]) for n in ("o", "lse", "dq", "dk", "dv"))
    print(f"c4 host ({'shared' if shared else 'per head'}): {int(r['count'].max())} of {T // cfg.chunk} chunks "
          "staged per kv head at most")
    rep = H // Hkv
    for kv in (1, 6):
        heads = list(range(kv * rep, (kv + 1) * rep))
        sub = lambda x: x[:, :, heads]  # noqa: E731
        lists = OH.expand_group_idx(ridx[:, kv:kv + 1], rep) if shared else ridx[:, heads]
        ro, rl, rdq, rdk, rdv = OH.hga_bwd(sub(q32), k32[:, T:, kv:kv + 1], v32[:, T:, kv:kv + 1],
                                           k32[:, :T, kv:kv + 1], v32[:, :T, kv:kv + 1], lists, sub(do32),
                                           cfg.chunk, cfg.qblock, cfg.scale)
        e = dict(o=max_abs(go[:, :, heads], ro), lse=max_abs(gl[:, heads], rl), dq=rel_fro(gdq[:, :, heads], rdq),
                 dk=rel_fro(gdk[:, :, kv:kv + 1], rdk), dv=rel_fro(gdv[:, :, kv:kv + 1], rdv))
        print(f"c4 host kv {kv}: " + " ".join(f"{n} {x:.3e}" for n, x in e.items()))
        assert e["o"] <= O_ATOL and e["lse"] <= LSE_ATOL
        assert e["dq"] <= GRAD_RTOL and e["dk"] <= GRAD_RTOL and e["dv"] <= GRAD_RTOL
    # its own selection: the same bits as the step on the resident history
    own = pipeline.hga_host_step(q, kf[:, T:], vf[:, T:], kh, vh, summ, do, T, cfg.chunk, cfg.qblock, cfg.topk,
                                 cfg.scale, shared=shared)
    ref = pipeline.hga_train_step(q, kf[:, T:], vf[:, T:], kf[:, :T], vf[:, :T], do, cfg.chunk, cfg.qblock,
                                  cfg.topk, cfg.scale, shared=shared)
    assert torch.equal(own["idx"], ref["idx"])
    for n in ("o", "dq", "dk", "dv"):
        assert torch.equal(i16(own[n]), i16(ref[n])), n
    assert torch.equal(own["lse"], ref["lse"])


@pytest.mark.parametrize("overlap", [True, False], ids=["overlap", "serial"])
@pytest.mark.parametrize("shared", [False, True], ids=["per_head", "shared"])
def test_host_training_pass_equals_the_resident_pass(shared, overlap):
    from block_sparse_attention_41_amd import pipeline
    L, seg, H, Hkv, d, chunk, topk = 8192, 2048, 8, 2, 128, 128, 8
    inp = synth.s2attn_inputs(1, L, H, Hkv, d, seed=41)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    a = pipeline.hga_train_segments(q, k, v, do, seg, chunk, 64, topk, d ** -0.5, shared=shared)
    b = pipeline.hga_host_segments(q, k, v, do, seg, chunk, 64, topk, d ** -0.5, shared=shared, overlap=overlap)
    torch.cuda.synchronize()
    assert torch.equal(a["idx"], b["idx"]) and torch.equal(a["lse"], b["lse"]) and torch.equal(a["summ"], b["summ"])
    for n in ("o", "dq", "dk", "dv"):
        assert torch.equal(i16(a[n]), i16(b[n])), n
    assert torch.equal(i16(b["k_host"]), i16(k.cpu())) and torch.equal(i16(b["v_host"]), i16(v.cpu()))


def test_host_evaluation_equals_the_resident_evaluation():
    from block_sparse_attention_41_amd import pipeline
    L, seg, H, Hkv, d, chunk, topk = 16384, 2048, 32, 8, 128, 128, 16
    inp = synth.hga_long_inputs(1, L, H, Hkv, d, chunk=chunk, seed=4)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o, lse, idx = pipeline.hga_long_eval(q, k, v, seg, chunk, 64, topk, d ** -0.5, shared=True)
    st = pipeline.hga_host_segments(q, k, v, None, seg, chunk, 64, topk, d ** -0.5, shared=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, st["idx"]) and torch.equal(lse, st["lse"]) and torch.equal(i16(o), i16(st["o"]))


@pytest.mark.parametrize("shared", [False, True], ids=["per_head", "shared"])
def test_cached_staging_sequence_matches_oracle(shared):
    """Three calls on the same staging buffers with different lists: the tables, counts,
    copied counts and renamed lists equal the oracle's stage_update, every named chunk's
    rows are in its slot, and the attention on the staging equals the resident one."""
    from block_sparse_attention_41_amd import ops
    case = (1, 512, 2048, 32, 8, 128, 128, 8)
    B, S, T, H, Hkv, d, chunk, topk = case
    dev, _ = _setup(case, seed=51)
    C, nqb = T // chunk, S // 64
    lists = Hkv if shared else H
    kh, vh = _pinned(dev["k_hist"]), _pinned(dev["v_hist"])
    slots = ops.hga_stage_slots(lists, Hkv, nqb, topk, C)
    chunk_of = torch.full((B, Hkv, slots), -1, dtype=torch.int32, device="cuda:0")
    ks = torch.empty((B, slots * chunk, Hkv, d), dtype=torch.bfloat16, device="cuda:0")
    vs = torch.empty_like(ks)
    prev = np.full((B, Hkv, slots), -1, dtype=np.int32)
    hk, hv = i16(kh).numpy(), i16(vh).numpy()
    fwd = ops.hga_fwd_shared if shared else ops.hga_fwd
    for step, fill in enumerate((0.5, 1.0, 0.7)):
        ridx = synth.random_topk_indices(B, lists, nqb, C, topk, seed=60 + step, fill=fill)
        idx = torch.from_numpy(ridx).to("cuda:0")
        ist, cnt, cp = ops.hga_stage_update(idx, kh, vh, T, chunk, chunk_of, ks, vs)
        torch.cuda.synchronize()
        rco, rcnt, rcp, rst = OH.stage_update(prev, ridx, Hkv, C, slots)
        assert np.array_equal(chunk_of.cpu().numpy(), rco) and np.array_equal(ist.cpu().numpy(), rst)
        assert np.array_equal(cnt.cpu().numpy(), rcnt) and np.array_equal(cp.cpu().numpy(), rcp)
        print(f"step {step}: {int(rcp.sum())} of {int(rcnt.sum())} named chunks copied")
        gk, gv = i16(ks).cpu().numpy(), i16(vs).cpu().numpy()
        for j in range(Hkv):
            for s_ in range(slots):
                c = int(rco[0, j, s_])
                if c >= 0:
                    rows, src = slice(s_ * chunk, (s_ + 1) * chunk), slice(c * chunk, (c + 1) * chunk)
                    assert np.array_equal(gk[0, rows, j], hk[0, src, j]) and np.array_equal(gv[0, rows, j], hv[0, src, j])
        o1, l1 = fwd(dev["q"], dev["k_act"], dev["v_act"], dev["k_hist"], dev["v_hist"], idx, chunk, 64, d ** -0.5)
        o2, l2 = fwd(dev["q"], dev["k_act"], dev["v_act"], ks, vs, ist, chunk, 64, d ** -0.5)
        assert torch.equal(i16(o1), i16(o2)) and torch.equal(l1, l2)
        prev = rco


@pytest.mark.parametrize("cached", [True, False], ids=["cached", "fresh"])
def test_host_training_pass_with_cached_staging_equals_the_resident_pass(cached):
    from block_sparse_attention_41_amd import pipeline
    L, seg, H, Hkv, d, chunk, topk = 8192, 2048, 8, 2, 128, 128, 8
    inp = synth.s2attn_inputs(1, L, H, Hkv, d, seed=42)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    a = pipeline.hga_train_segments(q, k, v, do, seg, chunk, 64, topk, d ** -0.5, shared=True)
    st = pipeline.hga_host_segments(q, k, v, do, seg, chunk, 64, topk, d ** -0.5, shared=True, cached=cached)
    # a second pass on the same state with other keys: the caches must not carry over
    inp2 = synth.s2attn_inputs(1, L, H, Hkv, d, seed=43)
    q2, k2, v2, do2 = (to_dev(inp2[n]) for n in ("q", "k", "v", "do"))
    a2 = pipeline.hga_train_segments(q2, k2, v2, do2, seg, chunk, 64, topk, d ** -0.5, shared=True)
    b2 = pipeline.hga_host_segments(q2, k2, v2, do2, seg, chunk, 64, topk, d ** -0.5, shared=True, cached=cached,
                                    state=st)
    torch.cuda.synchronize()
    for n in ("o", "dq", "dk", "dv"):
        assert torch.equal(i16(a2[n]), i16(b2[n])), n
    assert torch.equal(a2["idx"], b2["idx"]) and torch.equal(a2["lse"], b2["lse"])
