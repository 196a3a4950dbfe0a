"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every expected value comes from
a hand-worked example (tests/golden), a closed form, a library routine
(torch softmax, torch SDPA, numpy matmul) or brute force over the raw prefix
(Eq. 1 of "Retrofitting Linear Attention into Diffusion Language Models",
section 2.2, evaluated without the recurrent state).  CPU only.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_example.json")


# ---------------------------------------------------------------- helpers
def _val(s):
    s = str(s)
    if "ln(" in s:
        coef, arg = s.split("*ln(")
        return float(Fraction(coef)) * math.log(float(Fraction(arg.rstrip(")"))))
    return float(Fraction(s))


def _arr(rows):
    return np.array([[_val(x) for x in r] if isinstance(r, list) else _val(r) for r in rows],
                    dtype=np.float64)


def _golden():
    with open(GOLDEN) as fh:
        g = json.load(fh)
    d, F = g["d"], g["F"]
    W = _arr(g["W"]).reshape(1, d, F)
    pk = _arr(g["prefix_k"]).reshape(1, 1, -1, d)
    pv = _arr(g["prefix_v"]).reshape(1, 1, -1, d)
    q = _arr(g["block_q"]).reshape(1, 1, -1, d)
    k = _arr(g["block_k"]).reshape(1, 1, -1, d)
    v = _arr(g["block_v"]).reshape(1, 1, -1, d)
    return g, W, pk, pv, q, k, v


def lib_phi(x, W):
    """Hedgehog map through torch's softmax (library route): x [..., d], W [d, F]."""
    u = torch.from_numpy(np.asarray(x, dtype=np.float64)) @ torch.from_numpy(np.asarray(W, dtype=np.float64))
    return torch.cat([torch.softmax(u, -1), torch.softmax(-u, -1)], -1).numpy()


def empty_pool(slots, H, F, d):
    return np.zeros((slots, H, 2 * F, d)), np.zeros((slots, H, 2 * F))


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300))


def rand_case(rng, B, H, L, d, F, P):
    W = rng.normal(0, d ** -0.5, (H, d, F))
    q, k, v = (rng.normal(0, 1, (B, H, L, d)) for _ in range(3))
    pk, pv = (rng.normal(0, 1, (B, H, P, d)) for _ in range(2))
    return W, q, k, v, pk, pv


# ------------------------------------------------------- feature map pins
def test_phi_hand_worked():
    g, W, pk, pv, q, k, v = _golden()
    phi_k = oracle.feature_map(pk[0, 0][:, None, :], W)[:, 0]
    phi_q = oracle.feature_map(q[0, 0][:, None, :], W)[:, 0]
    np.testing.assert_allclose(phi_k, _arr(g["phi_prefix_k"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(phi_q, _arr(g["phi_block_q"]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("d,F", [(64, 64), (128, 128), (16, 8)])
def test_phi_matches_library_softmax(d, F):
    rng = np.random.default_rng(10 + d + F)
    H, n = 3, 17
    x = rng.normal(0, 1, (n, H, d))
    W = rng.normal(0, d ** -0.5, (H, d, F))
    got = oracle.feature_map(x, W)
    for h in range(H):
        np.testing.assert_allclose(got[:, h], lib_phi(x[:, h], W[h]), rtol=1e-13, atol=1e-16)


def test_phi_simplex_and_sign_swap():
    rng = np.random.default_rng(3)
    d, F, H, n = 32, 24, 2, 11
    x = rng.normal(0, 2, (n, H, d))
    W = rng.normal(0, 1, (H, d, F))
    p = oracle.feature_map(x, W)
    assert np.all(p > 0)
    np.testing.assert_allclose(p[..., :F].sum(-1), 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(p[..., F:].sum(-1), 1.0, rtol=0, atol=1e-14)
    pm = oracle.feature_map(-x, W)  # phi(-x) swaps the two halves
    np.testing.assert_allclose(pm[..., :F], p[..., F:], rtol=1e-13, atol=0)
    np.testing.assert_allclose(pm[..., F:], p[..., :F], rtol=1e-13, atol=0)


def test_phi_zero_W_is_uniform():
    x = np.random.default_rng(4).normal(0, 1, (5, 2, 8))
    p = oracle.feature_map(x, np.zeros((2, 8, 6)))
    np.testing.assert_allclose(p, 1.0 / 6, rtol=0, atol=1e-16)


def test_phi_large_logits_reach_one_hot():
    # softmax(c u) -> one-hot at argmax u as c grows; the stable form must not overflow
    rng = np.random.default_rng(5)
    d, F = 8, 5
    x = rng.normal(0, 1, (3, 1, d))
    W = rng.normal(0, 1, (1, d, F)) * 1e4
    p = oracle.feature_map(x, W)
    u = x[:, 0] @ W[0]
    assert np.all(np.isfinite(p))
    for r in range(3):
        hot_pos = np.eye(F)[np.argmax(u[r])]
        hot_neg = np.eye(F)[np.argmin(u[r])]
        np.testing.assert_allclose(p[r, 0, :F], hot_pos, atol=1e-12)
        np.testing.assert_allclose(p[r, 0, F:], hot_neg, atol=1e-12)


# ------------------------------------------------------------ commit pins
def test_commit_hand_worked():
    g, W, pk, pv, q, k, v = _golden()
    S0, Z0 = empty_pool(1, 1, g["F"], g["d"])
    S, Z = oracle.commit(S0, Z0, pk, pv, W)
    np.testing.assert_allclose(S[0, 0], _arr(g["S"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(Z[0, 0], _arr(g["Z"]), rtol=0, atol=1e-15)


def test_commit_equals_library_matmul():
    # S = Phi(K)^T V and Z = Phi(K)^T 1 with Phi from torch softmax and numpy matmul
    rng = np.random.default_rng(6)
    B, H, T, d, F = 2, 3, 19, 16, 12
    W = rng.normal(0, d ** -0.5, (H, d, F))
    k, v = rng.normal(0, 1, (B, H, T, d)), rng.normal(0, 1, (B, H, T, d))
    S0 = rng.normal(0, 1, (B, H, 2 * F, d))
    Z0 = rng.uniform(0, 1, (B, H, 2 * F))
    S, Z = oracle.commit(S0, Z0, k, v, W)
    for b in range(B):
        for h in range(H):
            Phi = lib_phi(k[b, h], W[h])                 # [T][2F]
            np.testing.assert_allclose(S[b, h], S0[b, h] + Phi.T @ v[b, h], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(Z[b, h], Z0[b, h] + Phi.sum(0), rtol=1e-13, atol=0)


def test_commit_zero_W_closed_form():
    rng = np.random.default_rng(7)
    B, H, T, d, F = 1, 2, 10, 6, 4
    k, v = rng.normal(0, 1, (B, H, T, d)), rng.normal(0, 1, (B, H, T, d))
    S, Z = oracle.commit(*empty_pool(B, H, F, d), k, v, np.zeros((H, d, F)))
    np.testing.assert_allclose(Z, T / F, rtol=1e-14)
    for h in range(H):
        expect = np.tile(v[0, h].sum(0) / F, (2 * F, 1))
        np.testing.assert_allclose(S[0, h], expect, rtol=1e-13, atol=1e-14)


def test_commit_chunking_and_order_invariance():
    rng = np.random.default_rng(8)
    B, H, T, d, F = 2, 2, 64, 16, 8
    W = rng.normal(0, d ** -0.5, (H, d, F))
    k, v = rng.normal(0, 1, (B, H, T, d)), rng.normal(0, 1, (B, H, T, d))
    S_all, Z_all = oracle.commit(*empty_pool(B, H, F, d), k, v, W)
    for chunk in (1, 8, 32):
        S, Z = empty_pool(B, H, F, d)
        for t0 in range(0, T, chunk):
            S, Z = oracle.commit(S, Z, k[:, :, t0:t0 + chunk], v[:, :, t0:t0 + chunk], W)
        assert rel(S, S_all) < 1e-12 and rel(Z, Z_all) < 1e-12
    perm = rng.permutation(T)
    S_p, Z_p = oracle.commit(*empty_pool(B, H, F, d), k[:, :, perm], v[:, :, perm], W)
    assert rel(S_p, S_all) < 1e-12 and rel(Z_p, Z_all) < 1e-12


def test_commit_ragged_and_slots():
    rng = np.random.default_rng(9)
    B, H, T, d, F, slots = 3, 2, 12, 8, 4, 5
    W = rng.normal(0, d ** -0.5, (H, d, F))
    k, v = rng.normal(0, 1, (B, H, T, d)), rng.normal(0, 1, (B, H, T, d))
    S0 = rng.normal(0, 1, (slots, H, 2 * F, d))
    Z0 = rng.uniform(0, 1, (slots, H, 2 * F))
    n_valid = np.array([12, 0, 5], np.int32)
    slot = np.array([4, 0, 2], np.int32)
    S, Z = oracle.commit(S0, Z0, k, v, W, n_valid=n_valid, slot=slot)
    for b in range(B):
        s, nv = slot[b], n_valid[b]
        for h in range(H):
            Phi = lib_phi(k[b, h, :nv], W[h])
            np.testing.assert_allclose(S[s, h], S0[s, h] + Phi.T @ v[b, h, :nv], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(Z[s, h], Z0[s, h] + Phi.sum(0), rtol=1e-13)
    for s in (1, 3):  # slots no request maps to are untouched
        assert np.array_equal(S[s], S0[s]) and np.array_equal(Z[s], Z0[s])
    with pytest.raises(oracle.OracleError):
        oracle.commit(S0, Z0, k, v, W, n_valid=np.array([13, 0, 0], np.int32), slot=slot)


# -------------------------------------------------------------- step pins
@pytest.mark.parametrize("gate_key,w", [("out_gate_1", 1.0), ("out_gate_1_2", 0.5)])
def test_step_hand_worked(gate_key, w):
    g, W, pk, pv, q, k, v = _golden()
    S, Z = oracle.commit(*empty_pool(1, 1, g["F"], g["d"]), pk, pv, W)
    out = oracle.step(q, k, v, W, S, Z, gate=np.array([w]))
    np.testing.assert_allclose(out[0, 0], _arr(g[gate_key]), rtol=0, atol=1e-14)


def test_step_empty_state_is_block_sdpa():
    # empty prefix: the ratio is exact softmax restricted to the active block (section 3.1)
    rng = np.random.default_rng(11)
    B, H, L, d, F = 2, 3, 32, 64, 16
    W, q, k, v, _, _ = rand_case(rng, B, H, L, d, F, 0)
    for gate in (None, np.array([0.3, 1.0, 2.5])):
        out = oracle.step(q, k, v, W, *empty_pool(B, H, F, d), gate=gate)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def _brute_force_hybrid(q, k, v, W, pk, pv, w):
    """Weighted average over block keys (weight w e^{q.k/sqrt d}) and raw prefix
    tokens (weight phi(q).phi(k_t), Eq. 1 kernel) -- no recurrent state."""
    L, d = q.shape
    a = w * np.exp(q @ k.T / math.sqrt(d))                 # [L][L]
    kap = lib_phi(q, W) @ lib_phi(pk, W).T if len(pk) else np.zeros((L, 0))
    weights = np.concatenate([a, kap], 1)
    vals = np.concatenate([v, pv], 0)
    return (weights @ vals) / weights.sum(1, keepdims=True)


@pytest.mark.parametrize("L,d,F,P", [(8, 64, 64, 32), (32, 32, 16, 100), (4, 16, 8, 1)])
def test_step_equals_brute_force_prefix(L, d, F, P):
    rng = np.random.default_rng(12 + P)
    B, H = 2, 2
    W, q, k, v, pk, pv = rand_case(rng, B, H, L, d, F, P)
    gate = np.array([1.0, 0.4])
    S, Z = oracle.commit(*empty_pool(B, H, F, d), pk, pv, W)
    out = oracle.step(q, k, v, W, S, Z, gate=gate)
    for b in range(B):
        for h in range(H):
            ref = _brute_force_hybrid(q[b, h], k[b, h], v[b, h], W[h], pk[b, h], pv[b, h], gate[h])
            np.testing.assert_allclose(out[b, h], ref, rtol=1e-11, atol=1e-12)


def test_step_gate_limits():
    rng = np.random.default_rng(13)
    B, H, L, d, F, P = 1, 2, 8, 16, 8, 40
    W, q, k, v, pk, pv = rand_case(rng, B, H, L, d, F, P)
    S, Z = oracle.commit(*empty_pool(B, H, F, d), pk, pv, W)
    # w -> 0: pure linear attention, Eq. 1 over the prefix (section 2.2)
    out0 = oracle.step(q, k, v, W, S, Z, gate=np.full(H, 1e-200))
    for h in range(H):
        kap = lib_phi(q[0, h], W[h]) @ lib_phi(pk[0, h], W[h]).T
        np.testing.assert_allclose(out0[0, h], kap @ pv[0, h] / kap.sum(1, keepdims=True), rtol=1e-11, atol=1e-12)
    # w -> infinity: block softmax
    outi = oracle.step(q, k, v, W, S, Z, gate=np.full(H, 1e200))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(outi, ref, rtol=1e-11, atol=1e-12)


def test_step_zero_W_closed_form():
    # W = 0: phi = 1/F everywhere, so lin_num = (2/F) sum_t v_t and lin_den = 2P/F
    rng = np.random.default_rng(14)
    B, H, L, d, F, P = 1, 1, 8, 16, 8, 24
    _, q, k, v, pk, pv = rand_case(rng, B, H, L, d, F, P)
    W = np.zeros((H, d, F))
    S, Z = oracle.commit(*empty_pool(B, H, F, d), pk, pv, W)
    out = oracle.step(q, k, v, W, S, Z)
    a = np.exp(q[0, 0] @ k[0, 0].T / math.sqrt(d))
    ref = (a @ v[0, 0] + (2 / F) * pv[0, 0].sum(0)) / (a.sum(1, keepdims=True) + 2 * P / F)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-12, atol=1e-13)


def test_step_convexity_affine_and_permutation():
    rng = np.random.default_rng(15)
    B, H, L, d, F, P = 2, 2, 16, 32, 16, 48
    W, q, k, v, pk, pv = rand_case(rng, B, H, L, d, F, P)
    S, Z = oracle.commit(*empty_pool(B, H, F, d), pk, pv, W)
    out = oracle.step(q, k, v, W, S, Z)
    # convex combination of the visible values
    lo = np.minimum(v.min(2), pv.min(2))[:, :, None, :]
    hi = np.maximum(v.max(2), pv.max(2))[:, :, None, :]
    assert np.all(out >= lo - 1e-12) and np.all(out <= hi + 1e-12)
    # constant values everywhere -> that constant
    c = rng.normal(0, 1, (d,))
    vc, pvc = np.broadcast_to(c, v.shape).copy(), np.broadcast_to(c, pv.shape).copy()
    Sc, Zc = oracle.commit(*empty_pool(B, H, F, d), pk, pvc, W)
    np.testing.assert_allclose(oracle.step(q, k, vc, W, Sc, Zc), np.broadcast_to(c, out.shape), rtol=1e-12)
    # affine equivariance in V
    alpha, shift = -1.7, rng.normal(0, 1, (d,))
    Sa, Za = oracle.commit(*empty_pool(B, H, F, d), pk, alpha * pv + shift, W)
    outa = oracle.step(q, k, alpha * v + shift, W, Sa, Za)
    np.testing.assert_allclose(outa, alpha * out + shift, rtol=1e-11, atol=1e-12)
    # committed tokens form a set: order does not matter
    perm = rng.permutation(P)
    Sp, Zp = oracle.commit(*empty_pool(B, H, F, d), pk[:, :, perm], pv[:, :, perm], W)
    np.testing.assert_allclose(oracle.step(q, k, v, W, Sp, Zp), out, rtol=1e-12, atol=1e-13)


def test_step_slot_indirection():
    rng = np.random.default_rng(16)
    B, H, L, d, F, slots = 3, 2, 8, 16, 8, 6
    W, q, k, v, _, _ = rand_case(rng, B, H, L, d, F, 0)
    S = rng.normal(0, 0.1, (slots, H, 2 * F, d))
    Z = rng.uniform(0.5, 2, (slots, H, 2 * F))
    slot = np.array([5, 1, 3], np.int32)
    out = oracle.step(q, k, v, W, S, Z, slot=slot)
    out_g = oracle.step(q, k, v, W, S[slot], Z[slot])
    np.testing.assert_array_equal(out, out_g)


def test_step_refuses_overflowing_scores():
    rng = np.random.default_rng(17)
    B, H, L, d, F = 1, 1, 4, 4, 2
    W, q, k, v, _, _ = rand_case(rng, B, H, L, d, F, 0)
    with pytest.raises(oracle.OracleError):
        oracle.step(q * 1e3, k * 1e3, v, W, *empty_pool(B, H, F, d))


# -------------------------------------------------------- comparator pins
def test_comparator_hand_worked():
    g, W, pk, pv, q, k, v = _golden()
    out = oracle.prefix_softmax(q, k, v, pk, pv)
    c = g["comparator_out"]
    e = math.exp(0.5)
    num = _arr(c["num_sqrt_e"]) * e + _arr(c["num_const"])
    den = _arr(c["den_sqrt_e"]) * e + _arr(c["den_const"])
    np.testing.assert_allclose(out[0, 0], num / den[:, None], rtol=0, atol=1e-14)


@pytest.mark.parametrize("P", [0, 1, 37, 200])
def test_comparator_is_sdpa_over_prefix_and_block(P):
    rng = np.random.default_rng(18 + P)
    B, H, L, d = 2, 2, 16, 32
    _, q, k, v, pk, pv = rand_case(rng, B, H, L, d, 4, P)
    out = oracle.prefix_softmax(q, k, v, pk, pv)
    K = torch.from_numpy(np.concatenate([pk, k], 2))
    V = torch.from_numpy(np.concatenate([pv, v], 2))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), K, V).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_comparator_ragged_prefix_and_empty_state_agreement():
    rng = np.random.default_rng(19)
    B, H, L, d, F, P = 3, 2, 8, 16, 8, 30
    W, q, k, v, pk, pv = rand_case(rng, B, H, L, d, F, P)
    plen = np.array([30, 0, 11], np.int32)
    out = oracle.prefix_softmax(q, k, v, pk, pv, prefix_len=plen)
    for b in range(B):
        one = oracle.prefix_softmax(q[b:b + 1], k[b:b + 1], v[b:b + 1],
                                    pk[b:b + 1, :, :plen[b]], pv[b:b + 1, :, :plen[b]])
        np.testing.assert_allclose(out[b], one[0], rtol=1e-13, atol=1e-14)
    # at P = 0 the comparator and the hybrid step with an empty state are both block softmax
    hyb = oracle.step(q[1:2], k[1:2], v[1:2], W, *empty_pool(1, H, F, d))
    np.testing.assert_allclose(out[1], hyb[0], rtol=1e-12, atol=1e-13)


# ------------------------------------------------- key/value head groups
# Query heads own W, the gate and the states (section 3.1; section 3.3 keeps
# the state per query head); consecutive groups of H / Hkv query heads read
# one key/value head.  The library route is torch SDPA's own grouped-query
# mode, and brute force indexes the key/value head by h // (H / Hkv).
def gqa_case(rng, B, H, Hkv, L, d, F, P):
    W = rng.normal(0, d ** -0.5, (H, d, F))
    q = rng.normal(0, 1, (B, H, L, d))
    k, v = (rng.normal(0, 1, (B, Hkv, L, d)) for _ in range(2))
    pk, pv = (rng.normal(0, 1, (B, Hkv, P, d)) for _ in range(2))
    return W, q, k, v, pk, pv


@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (6, 3)])
def test_gqa_step_empty_state_is_grouped_sdpa(H, Hkv):
    rng = np.random.default_rng(40 + H + Hkv)
    B, L, d, F = 2, 16, 32, 8
    W, q, k, v, _, _ = gqa_case(rng, B, H, Hkv, L, d, F, 0)
    out = oracle.step(q, k, v, W, *empty_pool(B, H, F, d))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), enable_gqa=True).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2)])
def test_gqa_commit_equals_library_matmul(H, Hkv):
    rng = np.random.default_rng(44 + Hkv)
    B, T, d, F = 2, 24, 16, 8
    W, _, k, v, _, _ = gqa_case(rng, B, H, Hkv, T, d, F, 0)
    S, Z = oracle.commit(*empty_pool(B, H, F, d), k, v, W)
    G = H // Hkv
    for b in range(B):
        for h in range(H):
            p = lib_phi(k[b, h // G], W[h])                   # [T][2F]
            np.testing.assert_allclose(S[b, h], p.T @ v[b, h // G], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(Z[b, h], p.sum(0), rtol=1e-12, atol=1e-13)


def test_gqa_step_equals_brute_force_prefix():
    rng = np.random.default_rng(46)
    B, H, Hkv, L, d, F, P = 2, 4, 2, 8, 16, 8, 40
    W, q, k, v, pk, pv = gqa_case(rng, B, H, Hkv, L, d, F, P)
    gate = np.array([1.0, 0.4, 2.0, 0.7])
    S, Z = oracle.commit(*empty_pool(B, H, F, d), pk, pv, W)
    out = oracle.step(q, k, v, W, S, Z, gate=gate)
    G = H // Hkv
    for b in range(B):
        for h in range(H):
            g = h // G
            ref = _brute_force_hybrid(q[b, h], k[b, g], v[b, g], W[h], pk[b, g], pv[b, g], gate[h])
            np.testing.assert_allclose(out[b, h], ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("P", [0, 45])
def test_gqa_comparator_is_grouped_sdpa(P):
    rng = np.random.default_rng(48 + P)
    B, H, Hkv, L, d = 2, 6, 2, 8, 16
    _, q, k, v, pk, pv = gqa_case(rng, B, H, Hkv, L, d, 4, P)
    out = oracle.prefix_softmax(q, k, v, pk, pv)
    K = torch.from_numpy(np.concatenate([pk, k], 2))
    V = torch.from_numpy(np.concatenate([pv, v], 2))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), K, V, enable_gqa=True).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_gqa_rejects_uneven_groups():
    rng = np.random.default_rng(50)
    W, q, k, v, _, _ = gqa_case(rng, 1, 4, 3, 4, 8, 4, 0)
    with pytest.raises(oracle.OracleError):
        oracle.step(q, k, v, W, *empty_pool(1, 4, 4, 8))
