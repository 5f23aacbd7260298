"""GPU parity: HGA with one chunk selection per kv head (shared by its q heads), through
the C ABI, against the oracle's summed-score selection and its per-q-head attention run
on the expanded chunk lists."""
import numpy as np
import pytest
import torch

from block_sparse_attention_41_amd import synth
from oracle import hga as OH

from gpu_util import GRAD_RTOL, LSE_ATOL, O_ATOL, check_selection, max_abs, rel_fro, to_f64
from test_gpu_hga import CASES, _ids, _setup

pytestmark = pytest.mark.gpu

# the c4 step's head layout (32 q heads on 8 kv heads) at a length the oracle finishes
# in seconds, plus the cases of the per-head tests
SHARED_CASES = [(1, 512, 2048, 32, 8, 128, 128, 8),
                # two batches, history as a prefix view, 3 query blocks, d = 64
                (2, 192, 768, 8, 2, 64, 128, 4)] + CASES


def _oracle_select_shared(ref, chunk, topk, qblock=64, with_scores=False):
    C = ref["k_hist"].shape[1] // chunk
    B, S = ref["q"].shape[:2]
    Hkv = ref["k_act"].shape[2]
    if C == 0:
        idx, gap = np.full((B, Hkv, S // qblock, topk), -1, dtype=np.int32), np.full((B, Hkv, S // qblock), np.inf)
        return (idx, gap, np.zeros((B, Hkv, S // qblock, 0))) if with_scores else (idx, gap)
    sc = OH.group_block_scores(ref["q"], OH.summarize(ref["k_hist"], chunk), qblock)
    idx, gap = OH.select_topk(sc, topk)
    return (idx, gap, sc) if with_scores else (idx, gap)


@pytest.mark.parametrize("case", SHARED_CASES, ids=_ids)
def test_shared_selection_matches_oracle(case):
    from block_sparse_attention_41_amd import ops
    B, S, T, H, Hkv, d, chunk, topk = case
    dev, ref = _setup(case)
    summ = ops.hga_summarize(dev["k_hist"], chunk)
    idx = ops.hga_select_topk_shared(dev["q"], summ, 64, topk).cpu().numpy()
    ridx, gap, sc = _oracle_select_shared(ref, chunk, topk, with_scores=True)
    assert idx.shape == (B, Hkv, S // 64, topk)
    nbad, nnear = check_selection(idx, ridx, sc, gap, topk)
    print(f"{_ids(case)}: {nbad} differing rows of {ridx[..., 0].size}, {nnear} near-ties")


@pytest.mark.parametrize("case", SHARED_CASES, ids=_ids)
@pytest.mark.parametrize("which", ["selected", "random"])
def test_shared_fwd_bwd_match_oracle(case, which):
    from block_sparse_attention_41_amd import ops
    B, S, T, H, Hkv, d, chunk, topk = case
    dev, ref = _setup(case, seed=3)
    if which == "selected":
        ridx, _ = _oracle_select_shared(ref, chunk, topk)
    else:
        ridx = synth.random_topk_indices(B, Hkv, S // 64, T // chunk, topk, seed=5, fill=0.6)
    scale = d ** -0.5
    idx = torch.from_numpy(ridx).to("cuda:0")
    o, lse = ops.hga_fwd_shared(dev["q"], dev["k_act"], dev["v_act"], dev["k_hist"], dev["v_hist"], idx, chunk, 64,
                                scale)
    dq, dk, dv = ops.hga_bwd_active_shared(dev["q"], dev["k_act"], dev["v_act"], dev["k_hist"], dev["v_hist"], idx,
                                           o, lse, dev["do"], chunk, 64, scale)
    ro, rl, rdq, rdk, rdv = OH.hga_bwd(ref["q"], ref["k_act"], ref["v_act"], ref["k_hist"], ref["v_hist"],
                                       OH.expand_group_idx(ridx, H), ref["do"], chunk, 64, scale)
    e_o, e_l = max_abs(to_f64(o), ro), max_abs(to_f64(lse), rl)
    e_g = {n: rel_fro(to_f64(a), r) for n, a, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv))}
    print(f"{_ids(case)} {which}: O {e_o:.3e} LSE {e_l:.3e} " + " ".join(f"{n} {e:.3e}" for n, e in e_g.items()))
    assert e_o <= O_ATOL and e_l <= LSE_ATOL
    for n, e in e_g.items():
        assert e <= GRAD_RTOL, n


@pytest.mark.parametrize("case", SHARED_CASES[:4] + SHARED_CASES[-2:], ids=_ids)
def test_shared_entry_points_equal_per_head_ones_on_expanded_lists(case):
    """The shared forms give the same bits as the per-q-head forms fed the expanded lists
    (with four q heads per kv head the shared forward is a kernel of its own that deals
    each block's tiles to its key streams in the same order)."""
    from block_sparse_attention_41_amd import ops
    B, S, T, H, Hkv, d, chunk, topk = case
    dev, _ = _setup(case, seed=6)
    ridx = synth.random_topk_indices(B, Hkv, S // 64, T // chunk, topk, seed=7, fill=0.8)
    scale = d ** -0.5
    idx_kv = torch.from_numpy(ridx).to("cuda:0")
    idx_q = torch.from_numpy(OH.expand_group_idx(ridx, H).copy()).to("cuda:0")
    args = (dev["q"], dev["k_act"], dev["v_act"], dev["k_hist"], dev["v_hist"])
    o1, l1 = ops.hga_fwd_shared(*args, idx_kv, chunk, 64, scale)
    o2, l2 = ops.hga_fwd(*args, idx_q, chunk, 64, scale)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    g1 = ops.hga_bwd_active_shared(*args, idx_kv, o1, l1, dev["do"], chunk, 64, scale)
    g2 = ops.hga_bwd_active(*args, idx_q, o2, l2, dev["do"], chunk, 64, scale)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
