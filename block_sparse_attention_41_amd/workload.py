"""The five workloads and their algorithmic work (pairs, FLOPs, bytes).

A "pair" is a (query, key) pair inside the attention mask.  Useful FLOPs count two
matrix products per pair in the forward (``QK^T`` and ``PV``: ``4 d`` per pair) and four
in the backward (``dV``, ``dP``, ``dQ``, ``dK``: ``8 d`` per pair); the backward's
recomputation of ``QK^T`` is not counted as useful.  For the bounded-history backward
the history side only has ``dP`` and ``dQ`` (``4 d`` per history pair), since the
history is detached.

Closed forms (checked against brute-force mask counts in the tests):

* shifted short attention, one head: ``(N/G) * G (G+1) / 2`` pairs for any shift, because
  a shift only permutes which tokens share a group;
* dense causal, one head: ``N (N+1) / 2``;
* bounded-history attention, one head: local ``S (S+1) / 2`` plus ``S * chunk * k_eff``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, vendor figure
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, vendor figure


@dataclass(frozen=True)
class S2Config:
    name: str
    B: int
    N: int
    H: int
    Hkv: int
    d: int
    G: int
    shift: bool = True

    @property
    def scale(self) -> float:
        return self.d ** -0.5

    def pairs(self) -> int:
        return s2_pairs(self.B, self.N, self.H, self.G)

    def fwd_flops(self) -> float:
        return 4.0 * self.d * self.pairs()

    def bwd_flops(self) -> float:
        return 8.0 * self.d * self.pairs()

    def tokens(self) -> int:
        return self.B * self.N


@dataclass(frozen=True)
class HGAConfig:
    name: str
    B: int
    S: int           # active segment length
    T: int           # history length (for one-segment configs)
    H: int
    Hkv: int
    d: int
    chunk: int = 128
    qblock: int = 64
    topk: int = 8
    segments: int = 1  # >1: long evaluation over segments*S tokens, forward only
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def scale(self) -> float:
        return self.d ** -0.5

    @property
    def C(self) -> int:
        return self.T // self.chunk


def s2_pairs(B: int, N: int, H: int, G: int) -> int:
    return B * H * (N // G) * (G * (G + 1) // 2)


def dense_causal_pairs(B: int, N: int, H: int) -> int:
    return B * H * (N * (N + 1) // 2)


def hga_pairs(B: int, S: int, H: int, chunk: int, topk: int, C: int) -> tuple[int, int]:
    """(local pairs, history pairs) of one segment."""
    keff = min(topk, C)
    return B * H * (S * (S + 1) // 2), B * H * S * chunk * keff


def hga_fwd_flops(B, S, H, d, chunk, topk, C) -> float:
    loc, hist = hga_pairs(B, S, H, chunk, topk, C)
    return 4.0 * d * (loc + hist)


def hga_bwd_flops(B, S, H, d, chunk, topk, C) -> float:
    loc, hist = hga_pairs(B, S, H, chunk, topk, C)
    return 8.0 * d * loc + 4.0 * d * hist


CONFIGS = {
    "c1": S2Config("c1_s2attn_n1024_g256_h4_d64", B=1, N=1024, H=4, Hkv=4, d=64, G=256),
    "c2": S2Config("c2_s2attn_n8192_g2048_h32_d128", B=1, N=8192, H=32, Hkv=32, d=128, G=2048),
    "c3": S2Config("c3_s2attn_n32768_g8192_h32_d128", B=1, N=32768, H=32, Hkv=32, d=128, G=8192),
    "c3_dense": S2Config("c3_dense_causal_n32768_h32_d128", B=1, N=32768, H=32, Hkv=32, d=128, G=32768,
                         shift=False),
    "c4": HGAConfig("c4_hga_train_s2048_t14336_hq32_hkv8_d128_k8", B=1, S=2048, T=14336, H=32, Hkv=8, d=128,
                    chunk=128, qblock=64, topk=8),
    "c5": HGAConfig("c5_hga_eval_l131072_seg2048_hq32_hkv8_d128_k16", B=1, S=2048, T=0, H=32, Hkv=8, d=128,
                    chunk=128, qblock=64, topk=16, segments=64),
}


def c5_totals(cfg: HGAConfig = CONFIGS["c5"]) -> dict:
    """Pairs and FLOPs of the whole long evaluation (segment s sees s*S/chunk chunks)."""
    loc = hist = 0
    for s in range(cfg.segments):
        C = s * cfg.S // cfg.chunk
        l_, h_ = hga_pairs(cfg.B, cfg.S, cfg.H, cfg.chunk, cfg.topk, C)
        loc += l_
        hist += h_
    return {"local_pairs": loc, "history_pairs": hist, "fwd_flops": 4.0 * cfg.d * (loc + hist)}
