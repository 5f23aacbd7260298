"""Seeded synthetic inputs shared by the CPU oracle tests, the GPU parity tests and the bench.

This module only draws random numbers and rounds them to bfloat16.  It holds none of
the attention arithmetic, so both the oracle (fp64 NumPy) and the HIP library can be fed
the exact same bit patterns without sharing any method code.

Draw order is part of the contract (changing it changes every stored fixture):

* S2-Attn workloads: Q, K, V, dO, each ``standard_normal`` in float32 with shape
  ``[B, L, heads, d]``, then round-to-nearest-even to bfloat16.
* HGA workloads: Q (active segment), K_full, V_full (history followed by the active
  segment, ``T + S`` tokens), dO.
* HGA long evaluation: Q, K_full, V_full over all tokens, then the offset direction u
  (``standard_normal(d)`` normalised to unit length) and a Bernoulli(1/2) query subset.
  Every chunk whose global index is a multiple of 4 gets ``+0.5 u`` on its keys (all kv
  heads); every query token in the subset gets ``+0.5 u`` (all heads).  Offsets are added
  in float32 before the bfloat16 rounding.  The pages ask only that selection be
  non-trivial; the subset fraction and the direction are this module's choice.
"""
from __future__ import annotations

import numpy as np


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = (bits + 0x7FFF + lsb) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(u: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float64 exactly."""
    return bf16_to_f32(u).astype(np.float64)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_round(rng.standard_normal(shape, dtype=np.float32))


def s2attn_inputs(B: int, N: int, H: int, Hkv: int, d: int, seed: int = 0) -> dict:
    """Q, K, V, dO for one shifted-short-attention call, as bfloat16 bit patterns."""
    rng = np.random.default_rng(seed)
    return {
        "q": _normal_bf16(rng, (B, N, H, d)),
        "k": _normal_bf16(rng, (B, N, Hkv, d)),
        "v": _normal_bf16(rng, (B, N, Hkv, d)),
        "do": _normal_bf16(rng, (B, N, H, d)),
    }


def hga_inputs(B: int, S: int, T: int, H: int, Hkv: int, d: int, seed: int = 0) -> dict:
    """One HGA training segment: active queries plus one K/V sequence of ``T + S`` tokens.

    ``k_full[:, :T]`` is the detached history and ``k_full[:, T:]`` the active segment.
    """
    rng = np.random.default_rng(seed)
    return {
        "q": _normal_bf16(rng, (B, S, H, d)),
        "k_full": _normal_bf16(rng, (B, T + S, Hkv, d)),
        "v_full": _normal_bf16(rng, (B, T + S, Hkv, d)),
        "do": _normal_bf16(rng, (B, S, H, d)),
    }


def hga_long_inputs(B: int, L: int, H: int, Hkv: int, d: int, chunk: int = 128,
                    offset: float = 0.5, every: int = 4, seed: int = 0) -> dict:
    """Structured long-evaluation inputs (Q, K, V over all ``L`` tokens) with planted offsets."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, L, H, d), dtype=np.float32)
    k = rng.standard_normal((B, L, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((B, L, Hkv, d), dtype=np.float32)
    u = rng.standard_normal(d, dtype=np.float32)
    u = (u / np.float32(np.linalg.norm(u.astype(np.float64)))).astype(np.float32)
    subset = rng.random((B, L)) < 0.5
    off = (np.float32(offset) * u).astype(np.float32)
    n_chunks = L // chunk
    planted = np.zeros(n_chunks, dtype=bool)
    planted[::every] = True
    token_planted = np.repeat(planted, chunk)
    k[:, token_planted] += off
    q[subset] += off
    return {
        "q": bf16_round(q),
        "k": bf16_round(k),
        "v": bf16_round(v),
        "u": u,
        "subset": subset,
        "planted_chunks": planted,
    }


def random_topk_indices(B: int, H: int, nqb: int, C: int, topk: int, seed: int = 0,
                        fill: float = 1.0) -> np.ndarray:
    """Seeded valid chunk-index sets: ascending, distinct, ``-1`` padding at the end.

    Each row keeps ``round(fill * min(topk, C))`` chunks (at least one when C > 0).
    Used to drive the gathered-history attention independently of the selection step.
    """
    rng = np.random.default_rng(seed)
    out = np.full((B, H, nqb, topk), -1, dtype=np.int32)
    keff = min(topk, C)
    n = max(1, int(round(fill * keff))) if C > 0 else 0
    for b in range(B):
        for h in range(H):
            for j in range(nqb):
                if n:
                    sel = np.sort(rng.choice(C, size=n, replace=False))
                    out[b, h, j, :n] = sel
    return out
