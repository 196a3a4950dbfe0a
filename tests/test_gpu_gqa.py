"""Key/value head groups on the GPU: H query heads (own W, gate and state)
over Hkv key/value heads, query head h reading key/value head h // (H/Hkv).

Every call is compared with the fp64 oracle on the same seeded inputs.  A
second check holds at any size: a grouped call must give exactly the bits of
the same call with each key/value head repeated over its group, since the
kernels read the same values in the same order either way."""
import numpy as np
import pytest
import torch

import block_hybrid_attention_amd as hba
import oracle
from block_hybrid_attention_amd import workloads as wl
from parity import check, report, row_rel, state_rel

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gen(seed):
    return wl.generator(seed, DEV)


@pytest.fixture(scope="module", autouse=True)
def _library():
    hba.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def grouped(B, H, Hkv, L, d, dtype, g):
    q = wl.normal((B, H, L, d), 1, dtype, g, DEV)
    k = wl.normal((B, Hkv, L, d), 1, dtype, g, DEV)
    v = wl.normal((B, Hkv, L, d), 1, dtype, g, DEV)
    return q, k, v


def rep(t, G):
    """[B][Hkv][..] -> [B][Hkv*G][..], head h holding key/value head h // G."""
    return t.repeat_interleave(G, dim=1).contiguous()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d,F", [(128, 128), (64, 64)])
@pytest.mark.parametrize("Hkv", [1, 2, 4])
def test_gqa_step_and_commit_match_oracle(dtype, d, F, Hkv):
    g = gen(9600 + d + F + 7 * Hkv + (dtype == torch.bfloat16))
    B, H, L, P, slots = 3, 8, 32, 72, 5
    W = wl.feature_weights(H, d, F, dtype, g, DEV)
    pq, pk, pv = grouped(B, H, Hkv, P, d, dtype, g)
    q, k, v = grouped(B, H, Hkv, L, d, dtype, g)
    gate = wl.gate_from_alpha(H, g, DEV)
    slot = torch.tensor([4, 0, 2], dtype=torch.int32, device=DEV)
    plen = torch.tensor([P, 1, 40], dtype=torch.int32, device=DEV)
    S = torch.zeros((slots, H, 2 * F, d), device=DEV)
    Z = torch.zeros((slots, H, 2 * F), device=DEV)

    hba.commit(pk, pv, W, S, Z, n_valid=plen, slot=slot)
    out = hba.step(q, k, v, W, S, Z, gate=gate, slot=slot)

    Sr, Zr = oracle.commit(np.zeros((slots, H, 2 * F, d)), np.zeros((slots, H, 2 * F)), pk, pv, W,
                           n_valid=plen, slot=slot)
    ref = oracle.step(q, k, v, W, Sr, Zr, gate=gate, slot=slot)
    errs = dict(out=row_rel(out, ref), S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]))
    report(f"gqa step+commit {dtype} d={d} F={F} H={H} Hkv={Hkv}", **errs)
    check(errs, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d,F", [(128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("L", [7, 32])
def test_gqa_step_commit_matches_oracle(dtype, d, F, L):
    g = gen(9700 + d + F + L + (dtype == torch.bfloat16))
    B, H, Hkv, P = 4, 6, 2, 64
    W = wl.feature_weights(H, d, F, dtype, g, DEV)
    _, pk, pv = grouped(B, H, Hkv, P, d, dtype, g)
    q, k, v = grouped(B, H, Hkv, L, d, dtype, g)
    gate = wl.gate_from_alpha(H, g, DEV)
    n_valid = torch.tensor([L, 0, min(3, L), L // 2], dtype=torch.int32, device=DEV)
    S = torch.zeros((B, H, 2 * F, d), device=DEV)
    Z = torch.zeros((B, H, 2 * F), device=DEV)
    hba.commit(pk, pv, W, S, Z)
    out = hba.step_commit(q, k, v, W, S, Z, gate=gate, n_valid=n_valid)

    Sp, Zp = oracle.commit(np.zeros((B, H, 2 * F, d)), np.zeros((B, H, 2 * F)), pk, pv, W)
    ref = oracle.step(q, k, v, W, Sp, Zp, gate=gate)
    Sr, Zr = oracle.commit(Sp, Zp, k, v, W, n_valid=n_valid)
    errs = dict(out=row_rel(out, ref), S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]))
    report(f"gqa step_commit {dtype} d={d} F={F} L={L}", **errs)
    check(errs, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
def test_gqa_comparator_matches_oracle(dtype, d):
    g = gen(9800 + d + (dtype == torch.bfloat16))
    B, H, Hkv, L, P = 3, 8, 2, 32, 300
    q, k, v = grouped(B, H, Hkv, L, d, dtype, g)
    Kc = wl.normal((B, Hkv, P, d), 1, dtype, g, DEV)
    Vc = wl.normal((B, Hkv, P, d), 1, dtype, g, DEV)
    plen = torch.tensor([P, 0, 157], dtype=torch.int32, device=DEV)
    out = hba.prefix_softmax(q, k, v, Kc, Vc, prefix_len=plen)
    ref = oracle.prefix_softmax(q, k, v, Kc, Vc, prefix_len=plen)
    err = row_rel(out, ref)
    report(f"gqa comparator {dtype} d={d}", out=err)
    check(dict(out=err), dtype)


def test_gqa_serving_shape_equals_repeated_heads_bitwise():
    """32 requests, 16 query heads over 4 key/value heads, bf16, 1k-token
    prefixes: every call gives the same bits as the multi-head call on
    repeated key/value heads."""
    g = gen(9900)
    B, H, Hkv, L, d, F, P = 32, 16, 4, 32, 128, 128, 1024
    G = H // Hkv
    dtype = torch.bfloat16
    W = wl.feature_weights(H, d, F, dtype, g, DEV)
    _, pk, pv = grouped(B, H, Hkv, P, d, dtype, g)
    q, k, v = grouped(B, H, Hkv, L, d, dtype, g)
    gate = wl.gate_from_alpha(H, g, DEV)

    S1 = torch.zeros((B, H, 2 * F, d), device=DEV)
    Z1 = torch.zeros((B, H, 2 * F), device=DEV)
    hba.commit(pk, pv, W, S1, Z1)
    S2 = torch.zeros_like(S1)
    Z2 = torch.zeros_like(Z1)
    hba.commit(rep(pk, G), rep(pv, G), W, S2, Z2)
    assert torch.equal(S1, S2) and torch.equal(Z1, Z2)

    o1 = hba.step(q, k, v, W, S1, Z1, gate=gate)
    o2 = hba.step(q, rep(k, G), rep(v, G), W, S2, Z2, gate=gate)
    assert torch.equal(o1, o2)

    c1 = hba.prefix_softmax(q, k, v, pk, pv)
    c2 = hba.prefix_softmax(q, rep(k, G), rep(v, G), rep(pk, G), rep(pv, G))
    assert torch.equal(c1, c2)

    f1 = hba.step_commit(q, k, v, W, S1, Z1, gate=gate)
    f2 = hba.step_commit(q, rep(k, G), rep(v, G), W, S2, Z2, gate=gate)
    assert torch.equal(f1, f2) and torch.equal(S1, S2) and torch.equal(Z1, Z2)

    # a sample of (request, head) pairs against the oracle
    idx = [0, 13, 31]
    Sr, Zr = oracle.commit(np.zeros((len(idx), H, 2 * F, d)), np.zeros((len(idx), H, 2 * F)),
                           pk[idx], pv[idx], W)
    ref = oracle.step(q[idx], k[idx], v[idx], W, Sr, Zr, gate=gate)
    err = row_rel(o1[idx], ref)
    report("gqa serving-shape step sample", out=err)
    check(dict(out=err), dtype)
