"""The training steps captured once in a HIP graph (torch.cuda.CUDAGraph over the C-ABI
launches) and replayed: every replay, with eager work and synchronisations between
replays, gives the bits of the eager step.  The kernels use no atomics and no memset
nodes, and take their workspace from the caller, so a captured step is reusable."""
import pytest
import torch

from block_sparse_attention_41_amd import synth

from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _capture_and_replay(step, outs, replays=3):
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(replays):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, r in zip(outs, ref):
            assert torch.equal(_bits(a), _bits(r))


@pytest.mark.parametrize("stored_ds", [False, True], ids=["recompute", "stored_ds"])
def test_s2attn_step_replays_from_a_graph(stored_ds):
    from block_sparse_attention_41_amd import ops
    B, N, H, Hkv, d, G = 1, 2048, 8, 4, 128, 512
    inp = synth.s2attn_inputs(B, N, H, Hkv, d, seed=31)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    o, dq = torch.empty_like(q), torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    size = ops.s2attn_bwd_workspace_bytes_dsq(B, N, H, Hkv, d, G) if stored_ds else \
        ops.s2attn_bwd_workspace_bytes(B, N, H, Hkv, d)
    ws = torch.empty(size, dtype=torch.uint8, device="cuda:0")

    def step():
        ops.s2attn_fwd(q, k, v, G, True, o=o, lse=lse)
        ops.s2attn_bwd(q, k, v, o, lse, do, G, True, workspace=ws, dq=dq, dk=dk, dv=dv)

    _capture_and_replay(step, [o, lse, dq, dk, dv])


@pytest.mark.parametrize("stored_ds", [False, True], ids=["recompute", "stored_ds"])
def test_hga_step_replays_from_a_graph(stored_ds):
    from block_sparse_attention_41_amd import ops
    B, S, T, H, Hkv, d, chunk, topk = 1, 512, 2048, 8, 2, 128, 128, 4
    inp = synth.hga_inputs(B, S, T, H, Hkv, d, seed=32)
    kf, vf = to_dev(inp["k_full"]), to_dev(inp["v_full"])
    q, do = to_dev(inp["q"]), to_dev(inp["do"])
    ka, va, kh, vh = kf[:, T:], vf[:, T:], kf[:, :T], vf[:, :T]
    summ = torch.empty((B, T // chunk, Hkv, d), dtype=torch.float32, device="cuda:0")
    idx = torch.empty((B, Hkv, S // 64, topk), dtype=torch.int32, device="cuda:0")
    o, dq = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda:0")
    dk = torch.empty((B, S, Hkv, d), dtype=torch.bfloat16, device="cuda:0")
    dv = torch.empty_like(dk)
    size = ops.hga_bwd_workspace_bytes_dsq(B, S, H, Hkv, d) if stored_ds else \
        ops.hga_bwd_workspace_bytes(B, S, H, Hkv, d)
    ws = torch.empty(size, dtype=torch.uint8, device="cuda:0")

    def step():   # the shared-list step: four q heads per kv head use the grouped forward
        ops.hga_summarize(kh, chunk, summ=summ)
        ops.hga_select_topk_shared(q, summ, 64, topk, idx=idx)
        ops.hga_fwd_shared(q, ka, va, kh, vh, idx, chunk, 64, o=o, lse=lse)
        ops.hga_bwd_active_shared(q, ka, va, kh, vh, idx, o, lse, do, chunk, 64, workspace=ws, dq=dq, dk_act=dk,
                                  dv_act=dv)

    _capture_and_replay(step, [summ, idx, o, lse, dq, dk, dv])
