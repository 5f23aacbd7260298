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
