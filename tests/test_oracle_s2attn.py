"""Pins for the S2-Attn oracle: hand-worked masks, closed forms, library special cases,
three independent formulations, torch autograd and fp64 finite differences."""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import s2attn as O
from oracle.attention import masked_attention, masked_attention_bwd, softmax_probs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_masks(path):
    out, cur = {}, None
    for line in open(path, encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            cur = line[1:-1]
            out[cur] = []
        else:
            out[cur].append([c == "1" for c in line])
    return {k: np.array(v) for k, v in out.items()}


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _gqa_expand(k, H):
    """[B, N, Hkv, d] -> [B, N, H, d] repeating each kv head for its q heads."""
    rep = H // k.shape[2]
    return np.repeat(k, rep, axis=2)


def _sdpa(q, k, v, scale, causal=True, mask=None):
    """torch's fp64 CPU attention on [L, d] operands."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x))[None, None] for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal and mask is None,
                                         scale=scale)
    return out[0, 0].numpy()


# ---------------------------------------------------------------- masks ---------------

def test_masks_match_hand_worked_example():
    g = _read_masks(os.path.join(GOLDEN, "s2attn_mask_n8_g4.txt"))
    assert np.array_equal(O.s2attn_mask(8, 4, 0), g["unshifted"])
    assert np.array_equal(O.s2attn_mask(8, 4, 2, "R1"), g["shifted_R1"])
    assert np.array_equal(O.s2attn_mask(8, 4, 2, "R2"), g["shifted_R2"])


@pytest.mark.parametrize("N,G", [(8, 4), (16, 4), (16, 8), (32, 8), (32, 16), (64, 16)])
def test_roll_direction_is_immaterial(N, G):
    s = G // 2
    # rolling right by s is rolling left by N - s
    assert np.array_equal(O.s2attn_mask(N, G, s), O.s2attn_mask(N, G, N - s))


@pytest.mark.parametrize("N,G", [(8, 4), (16, 4), (16, 8), (32, 8), (48, 16), (64, 64)])
@pytest.mark.parametrize("reading", ["R1", "R2"])
def test_pair_count_closed_form(N, G, reading):
    for s in (0, G // 2):
        m = O.s2attn_mask(N, G, s, reading)
        assert m.sum() == (N // G) * G * (G + 1) // 2
        assert m.diagonal().all()


def test_wrap_group_sees_the_end_of_the_sequence():
    # under R1 the first s tokens of a shifted head attend to the last s tokens: (G/2)^2 pairs
    N, G = 32, 8
    s = G // 2
    m = O.s2attn_mask(N, G, s, "R1")
    assert m[:s, N - s:].all()
    assert m[:s, N - s:].sum() == s * s
    assert not m[N - s:, :s].any()


def test_groups_partition_tokens():
    N, G, s = 64, 16, 8
    seen = np.concatenate([O.group_tokens(N, G, s, g) for g in range(N // G)])
    assert np.array_equal(np.sort(seen), np.arange(N))


# ---------------------------------------------------------------- forward --------------

@pytest.mark.parametrize("N,G,H,Hkv", [(32, 8, 4, 4), (32, 16, 4, 2), (48, 16, 6, 2), (16, 16, 4, 4)])
def test_three_formulations_agree(N, G, H, Hkv):
    B, d = 2, 8
    q, k, v = _rand((B, N, H, d), 1), _rand((B, N, Hkv, d), 2), _rand((B, N, Hkv, d), 3)
    scale = d ** -0.5
    o1, l1 = O.s2attn_fwd_bruteforce(q, k, v, G, True, scale)
    o2, l2, *_ = O.s2attn_groups(q, k, v, None, G, True, scale)
    o3, l3 = O.s2attn_fwd_roll(q, k, v, G, True, scale)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o1, o3, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l3, rtol=0, atol=1e-12)


def test_R2_per_group_matches_bruteforce():
    B, N, G, H, Hkv, d = 1, 32, 8, 4, 2, 8
    q, k, v = _rand((B, N, H, d), 4), _rand((B, N, Hkv, d), 5), _rand((B, N, Hkv, d), 6)
    o1, l1 = O.s2attn_fwd_bruteforce(q, k, v, G, True, 0.3, reading="R2")
    o2, l2, *_ = O.s2attn_groups(q, k, v, None, G, True, 0.3, reading="R2")
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


@pytest.mark.parametrize("shift", [True, False])
@pytest.mark.parametrize("Hkv", [4, 2, 1])
def test_single_group_is_dense_causal_attention(shift, Hkv):
    B, N, H, d = 2, 24, 4, 8
    q, k, v = _rand((B, N, H, d), 7), _rand((B, N, Hkv, d), 8), _rand((B, N, Hkv, d), 9)
    scale = d ** -0.5
    o, lse, *_ = O.s2attn_groups(q, k, v, None, N, shift, scale)
    ke, ve = _gqa_expand(k, H), _gqa_expand(v, H)
    for b in range(B):
        for h in range(H):
            ref = _sdpa(q[b, :, h], ke[b, :, h], ve[b, :, h], scale)
            np.testing.assert_allclose(o[b, :, h], ref, atol=1e-12)


def test_unshifted_heads_are_per_group_causal_attention():
    B, N, G, H, d = 1, 32, 8, 4, 8
    q, k, v = _rand((B, N, H, d), 10), _rand((B, N, H, d), 11), _rand((B, N, H, d), 12)
    scale = 0.25
    o, *_ = O.s2attn_groups(q, k, v, None, G, False, scale)
    for h in range(H):
        for g in range(N // G):
            sl = slice(g * G, (g + 1) * G)
            ref = _sdpa(q[0, sl, h], k[0, sl, h], v[0, sl, h], scale)
            np.testing.assert_allclose(o[0, sl, h], ref, atol=1e-12)


def test_shifted_heads_are_causal_attention_on_the_rolled_sequence():
    # the short roll / attend / roll-back form, with torch's attention as the attention call
    B, N, G, H, d = 1, 32, 8, 4, 8
    s = G // 2
    q, k, v = _rand((B, N, H, d), 13), _rand((B, N, H, d), 14), _rand((B, N, H, d), 15)
    scale = 0.3
    o, lse, *_ = O.s2attn_groups(q, k, v, None, G, True, scale)
    for h in range(H // 2, H):
        qr, kr, vr = (np.roll(x[0, :, h], -s, axis=0) for x in (q, k, v))
        orr = np.concatenate([_sdpa(qr[g * G:(g + 1) * G], kr[g * G:(g + 1) * G], vr[g * G:(g + 1) * G], scale)
                              for g in range(N // G)])
        np.testing.assert_allclose(o[0, :, h], np.roll(orr, s, axis=0), atol=1e-12)


def test_softmax_rows_sum_to_one_and_lse_bounds():
    N, G, d = 32, 8, 8
    q, k = _rand((N, d), 16), _rand((N, d), 17)
    v = _rand((N, d), 18)
    m = O.s2attn_mask(N, G, G // 2)
    o, lse = masked_attention(q, k, v, m, 0.5)
    p = softmax_probs(q, k, m, 0.5, lse)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(p[~m] == 0)
    diag = 0.5 * np.einsum("td,td->t", q, k)
    assert np.all(lse >= diag - 1e-12)
    # LSE is at most the max visible logit plus log of the visible count
    s = np.where(m, 0.5 * q @ k.T, -np.inf)
    assert np.all(lse <= s.max(axis=1) + np.log(m.sum(axis=1)) + 1e-12)


def test_zero_queries_give_uniform_attention_closed_form():
    # q = 0: every visible key gets weight 1/|visible|, LSE = log |visible|
    N, G, d = 16, 8, 4
    v = _rand((N, d), 19)
    m = O.s2attn_mask(N, G, G // 2)
    o, lse = masked_attention(np.zeros((N, d)), _rand((N, d), 20), v, m, 1.0)
    cnt = m.sum(axis=1)
    np.testing.assert_allclose(lse, np.log(cnt), atol=1e-14)
    np.testing.assert_allclose(o, (m @ v) / cnt[:, None], atol=1e-14)


# ---------------------------------------------------------------- backward -------------

def _torch_masked_attention(q, k, v, masks, scale, kvmap):
    """Differentiable reference with torch autograd: per head, explicit boolean mask."""
    outs = []
    for h in range(q.shape[1]):
        s = scale * (q[:, h] @ k[:, kvmap[h]].T)
        s = s.masked_fill(~masks[h], float("-inf"))
        outs.append(torch.softmax(s, dim=-1) @ v[:, kvmap[h]])
    return torch.stack(outs, dim=1)


@pytest.mark.parametrize("N,G,H,Hkv", [(16, 4, 4, 4), (16, 8, 4, 2), (32, 8, 4, 1)])
def test_bwd_matches_torch_autograd(N, G, H, Hkv):
    d = 8
    q, k, v, do = _rand((1, N, H, d), 21), _rand((1, N, Hkv, d), 22), _rand((1, N, Hkv, d), 23), _rand((1, N, H, d), 24)
    scale = d ** -0.5
    _, _, dq, dk, dv = O.s2attn_bwd_bruteforce(q, k, v, do, G, True, scale)
    _, _, dq2, dk2, dv2 = O.s2attn_groups(q, k, v, do, G, True, scale)
    tq, tk, tv = (torch.tensor(x[0], requires_grad=True) for x in (q, k, v))
    masks = [torch.from_numpy(O.s2attn_mask(N, G, O.head_shift(h, H, N, G, True))) for h in range(H)]
    kvmap = [O.kv_head(h, H, Hkv) for h in range(H)]
    out = _torch_masked_attention(tq, tk, tv, masks, scale, kvmap)
    (out * torch.from_numpy(do[0])).sum().backward()
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine[0], ref.numpy(), atol=1e-12)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        np.testing.assert_allclose(a, b, atol=1e-12)


@pytest.mark.parametrize("G,Hkv", [(4, 4), (8, 2), (8, 4), (4, 2)])
def test_bwd_matches_finite_differences(G, Hkv):
    B, N, H, d = 1, 16, 4, 4
    q, k, v, do = _rand((B, N, H, d), 31), _rand((B, N, Hkv, d), 32), _rand((B, N, Hkv, d), 33), _rand((B, N, H, d), 34)
    scale = d ** -0.5
    _, _, dq, dk, dv = O.s2attn_groups(q, k, v, do, G, True, scale)

    def loss(q_, k_, v_):
        o, _ = O.s2attn_fwd_bruteforce(q_, k_, v_, G, True, scale)
        return float((o * do).sum())

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[i] = (loss(**{f"{a}_": b for a, b in args_p.items()}) -
                      loss(**{f"{a}_": b for a, b in args_m.items()})) / (2 * eps)
        rel = np.linalg.norm(num - g) / np.linalg.norm(g)
        assert rel < 1e-6, (name, rel)


def test_key_gradient_sums_to_zero_per_kv_head():
    # shifting every key of a kv head by one vector shifts each visible logit row by a
    # constant, which the softmax ignores: sum over tokens of dK is zero per kv head
    B, N, G, H, Hkv, d = 1, 32, 8, 4, 2, 8
    q, k, v, do = _rand((B, N, H, d), 41), _rand((B, N, Hkv, d), 42), _rand((B, N, Hkv, d), 43), _rand((B, N, H, d), 44)
    _, _, dq, dk, dv = O.s2attn_groups(q, k, v, do, G, True, 0.35)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    # adding one vector to every value adds it to every output row: sum_u dV = sum_t dO per kv
    for kv in range(Hkv):
        hs = [h for h in range(H) if O.kv_head(h, H, Hkv) == kv]
        np.testing.assert_allclose(dv[0, :, kv].sum(axis=0), do[0][:, hs].sum(axis=(0, 1)), atol=1e-12)


def test_zero_output_gradient_gives_zero_gradients():
    B, N, G, H, d = 1, 16, 8, 4, 4
    q, k, v = _rand((B, N, H, d), 51), _rand((B, N, H, d), 52), _rand((B, N, H, d), 53)
    _, _, dq, dk, dv = O.s2attn_groups(q, k, v, np.zeros((B, N, H, d)), G, True, 0.5)
    assert not dq.any() and not dk.any() and not dv.any()


def test_value_gradient_closed_form_uniform_attention():
    # q = 0 -> P[t, u] = mask[t, u] / |visible(t)|, so dV = P^T dO in closed form
    N, G, d = 16, 8, 4
    m = O.s2attn_mask(N, G, G // 2)
    k, v, do = _rand((N, d), 54), _rand((N, d), 55), _rand((N, d), 56)
    q = np.zeros((N, d))
    o, lse = masked_attention(q, k, v, m, 1.0)
    _, _, dv = masked_attention_bwd(q, k, v, m, 1.0, o, lse, do)
    p = m / m.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(dv, p.T @ do, atol=1e-14)


@pytest.mark.parametrize("G,shift,reading", [(8, True, "R1"), (8, True, "R2"), (32, True, "R1"), (16, False, "R1")])
def test_row_sampled_forward_matches_groups(G, shift, reading):
    B, N, H, Hkv, d = 1, 32, 4, 2, 8
    q, k, v = _rand((B, N, H, d), 61), _rand((B, N, Hkv, d), 62), _rand((B, N, Hkv, d), 63)
    o, lse, *_ = O.s2attn_groups(q, k, v, None, G, shift, 0.4, reading)
    rows = [0, 3, 4, 15, 16, 27, 31]
    for h in range(H):
        ro, rl = O.s2attn_rows(q, k, v, 0, h, rows, G, shift, 0.4, reading)
        np.testing.assert_allclose(ro, o[0, rows, h], atol=1e-12)
        np.testing.assert_allclose(rl, lse[0, h, rows], atol=1e-12)
