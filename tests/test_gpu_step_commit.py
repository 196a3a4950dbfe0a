"""hba_step_commit: the block's last denoising step fused with the commit of
that block.  Every case builds a state from a seeded prefix on both sides
(hba_commit on the GPU, the oracle's commit on the host), then compares the
fused call with the oracle's step on that state followed by the oracle's
commit of the block."""
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


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d,F", [(128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("L", [1, 7, 32])
def test_step_commit_matches_oracle(dtype, d, F, L):
    """Slot map into a larger pool, a gate, n_valid with 0 and partial blocks.
    12 (request, head) pairs: the bf16 d = 128 kernel splits the value
    columns over two workgroups per pair."""
    g = gen(9100 + 7 * d + F + 31 * L + (dtype == torch.bfloat16))
    B, H, P, slots = 4, 3, 40, 6
    W = wl.feature_weights(H, d, F, dtype, g, DEV)
    pk, pv = wl.normal((B, H, P, d), 1, dtype, g, DEV), wl.normal((B, H, P, d), 1, dtype, g, DEV)
    q, k, v = wl.block_qkv(B, H, L, d, dtype, g, DEV)
    gate = wl.gate_from_alpha(H, g, DEV)
    slot = torch.tensor([5, 0, 2, 3], dtype=torch.int32, device=DEV)
    n_valid = torch.tensor([L, 0, min(3, L), L // 2], dtype=torch.int32, device=DEV)
    S = 0.01 * torch.randn((slots, H, 2 * F, d), generator=g, device=DEV)
    Z = torch.rand((slots, H, 2 * F), generator=g, device=DEV)
    S0, Z0 = S.clone(), Z.clone()

    hba.commit(pk, pv, W, S, Z, slot=slot)
    S1, Z1 = S.clone(), Z.clone()
    out = hba.step_commit(q, k, v, W, S, Z, gate=gate, slot=slot, n_valid=n_valid)

    Sp, Zp = oracle.commit(S0, Z0, pk, pv, W, slot=slot)
    ref = oracle.step(q, k, v, W, Sp, Zp, gate=gate, slot=slot)
    Sr, Zr = oracle.commit(Sp, Zp, k, v, W, n_valid=n_valid, slot=slot)

    for s in (1, 4):   # slots no request uses
        assert torch.equal(S[s], S0[s]) and torch.equal(Z[s], Z0[s])
    assert torch.equal(S[0], S1[0]) and torch.equal(Z[0], Z1[0])   # n_valid 0: untouched by the fused call
    errs = dict(out=row_rel(out, ref), S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]))
    report(f"step_commit {dtype} d={d} F={F} L={L}", **errs)
    check(errs, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_step_commit_agrees_with_separate_calls(dtype):
    g = gen(9300 + (dtype == torch.bfloat16))
    B, H, L, d, F, P = 6, 4, 32, 128, 128, 96
    W = wl.feature_weights(H, d, F, dtype, g, DEV)
    pk, pv = wl.normal((B, H, P, d), 1, dtype, g, DEV), wl.normal((B, H, P, d), 1, dtype, g, DEV)
    q, k, v = wl.block_qkv(B, H, L, d, dtype, g, DEV)
    S = torch.zeros((B, H, 2 * F, d), device=DEV)
    Z = torch.zeros((B, H, 2 * F), device=DEV)
    hba.commit(pk, pv, W, S, Z)
    S2, Z2 = S.clone(), Z.clone()
    out_f = hba.step_commit(q, k, v, W, S, Z)
    out_s = hba.step(q, k, v, W, S2, Z2)
    hba.commit(k, v, W, S2, Z2)
    errs = dict(out=row_rel(out_f, out_s), S=state_rel(S, S2), Z=state_rel(Z[..., None], Z2[..., None]))
    report(f"step_commit vs step + commit {dtype}", **errs)
    check(errs, dtype)


def test_step_commit_medium_bf16():
    """16 requests x 8 heads, 512-token prefixes of different lengths, every
    (request, head) compared with the oracle."""
    g = gen(9400)
    B, H, L, d, F, P = 16, 8, 32, 128, 128, 512
    dtype = torch.bfloat16
    W = wl.feature_weights(H, d, F, dtype, g, DEV)
    pk, pv = wl.normal((B, H, P, d), 1, dtype, g, DEV), wl.normal((B, H, P, d), 1, dtype, g, DEV)
    plen = torch.randint(1, P + 1, (B,), generator=g, device=DEV, dtype=torch.int32)
    q, k, v = wl.block_qkv(B, H, L, d, dtype, g, DEV)
    S = torch.zeros((B, H, 2 * F, d), device=DEV)
    Z = torch.zeros((B, H, 2 * F), device=DEV)
    hba.commit(pk, pv, W, S, Z, n_valid=plen)
    out = hba.step_commit(q, k, v, W, S, Z)
    Sp, Zp = oracle.commit(np.zeros((B, H, 2 * F, d)), np.zeros((B, H, 2 * F)), pk, pv, W, n_valid=plen)
    ref = oracle.step(q, k, v, W, Sp, Zp)
    Sr, Zr = oracle.commit(Sp, Zp, k, v, W)
    errs = dict(out=row_rel(out, ref), S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]))
    report("step_commit medium bf16", **errs)
    check(errs, dtype)


@pytest.mark.parametrize("F", [128, 64])
@pytest.mark.parametrize("L", [7, 32])
def test_step_commit_one_workgroup_per_pair(F, L):
    """bf16, d = 128 with more (request, head) pairs than half the CUs of a
    256-CU device (12 x 16 = 192), so each pair is one workgroup over all 128
    value columns: ragged n_valid with 0, a slot map and a gate, against the
    oracle's step and commit."""
    d, dtype = 128, torch.bfloat16
    g = gen(9300 + F + L)
    B, H, P = 12, 16, 40
    slots = B + 3
    W = wl.feature_weights(H, d, F, dtype, g, DEV)
    pk, pv = wl.normal((B, H, P, d), 1, dtype, g, DEV), wl.normal((B, H, P, d), 1, dtype, g, DEV)
    q, k, v = wl.block_qkv(B, H, L, d, dtype, g, DEV)
    gate = wl.gate_from_alpha(H, g, DEV)
    slot = torch.randperm(slots, generator=torch.Generator().manual_seed(F + L))[:B].to(torch.int32).to(DEV)
    n_valid = torch.tensor([L if b == B - 1 else (3 * b) % (L + 1) for b in range(B)], dtype=torch.int32, device=DEV)
    S = 0.01 * torch.randn((slots, H, 2 * F, d), generator=g, device=DEV)
    Z = torch.rand((slots, H, 2 * F), generator=g, device=DEV)
    S0, Z0 = S.clone(), Z.clone()

    hba.commit(pk, pv, W, S, Z, slot=slot)
    out = hba.step_commit(q, k, v, W, S, Z, gate=gate, slot=slot, n_valid=n_valid)

    Sp, Zp = oracle.commit(S0, Z0, pk, pv, W, slot=slot)
    ref = oracle.step(q, k, v, W, Sp, Zp, gate=gate, slot=slot)
    Sr, Zr = oracle.commit(Sp, Zp, k, v, W, n_valid=n_valid, slot=slot)
    used = set(slot.tolist())
    for s in range(slots):
        if s not in used:
            assert torch.equal(S[s], S0[s]) and torch.equal(Z[s], Z0[s])
    errs = dict(out=row_rel(out, ref), S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]))
    report(f"step_commit one workgroup per pair F={F} L={L}", **errs)
    check(errs, dtype)
