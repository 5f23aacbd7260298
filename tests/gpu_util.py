"""Helpers for the GPU parity tests: move seeded bf16 bit patterns to the device and
compare against the oracle with the tolerances the parity contract fixes."""
import numpy as np
import torch

from block_sparse_attention_41_amd import synth

# Parity bars: O max-abs <= 1e-2; dQ/dK/dV relative Frobenius <= 2e-2.
O_ATOL = 1e-2
GRAD_RTOL = 2e-2
# LSE is float32 from float32 row sums; 1e-3 absolute leaves room for exp2/log2 rounding.
LSE_ATOL = 1e-3


def to_dev(u16: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 on cuda:0 (bit-exact)."""
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def f64(u16):
    return synth.bf16_to_f64(u16)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def rel_fro(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a))


# Chunk lists may differ from the oracle's only where the oracle's k-th and (k+1)-th
# scores are closer than this (the parity contract's near-tie bar).  The GPU computes the
# scores in float32 from the same bf16 inputs; their rounding error is below 1e-6 at the
# workload sizes, so a flip needs a gap well under the bar.
NEAR_TIE = 1e-5


def check_selection(gidx, ridx, scores, gap, topk, tie=NEAR_TIE):
    """Compare a GPU chunk selection with the oracle's, row by row.

    Rows (the last axis is the list) must match exactly unless the oracle's gap is below
    ``tie``.  A differing near-tie row must still be a valid top-k list under the oracle's
    scores: k_eff = min(topk, C) distinct in-range chunks in ascending order, -1 after
    them, and every chosen chunk scoring at least the oracle's k-th best minus ``tie``.
    Returns (differing rows, near-tie rows)."""
    gidx, ridx = np.asarray(gidx), np.asarray(ridx)
    assert gidx.shape == ridx.shape, (gidx.shape, ridx.shape)
    bad = np.any(gidx != ridx, axis=-1)
    near = np.asarray(gap) < tie
    assert not np.any(bad & ~near), f"{int((bad & ~near).sum())} rows differ away from a near tie"
    if bad.any():
        sc = np.asarray(scores)
        C = sc.shape[-1]
        keff = min(topk, C)
        for r in map(tuple, np.argwhere(bad)):
            row, s = gidx[r], sc[r]
            chosen = row[:keff]
            assert np.all(row[keff:] == -1), (r, row)
            assert np.all((chosen >= 0) & (chosen < C)), (r, row)
            assert np.all(np.diff(chosen) > 0), (r, row)
            kth = np.sort(s)[::-1][keff - 1]
            assert np.all(s[chosen] >= kth - tie), (r, row, kth)
    return int(bad.sum()), int(near.sum())
