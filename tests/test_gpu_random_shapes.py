"""Seeded random shapes through every decode-path entry point, against the
fp64 oracle.

Each case draws, from its own seed, an input dtype, head_dim, feature width,
query heads and a key/value head count dividing them, a batch (some large
enough that the bf16 d = 128 kernels run one workgroup per pair, most small
enough for their two-workgroup split; the last cases 24 to 48 requests at 8
to 16 heads, more pairs than CUs), a block length in 1..32, a prefix of 0..100
tokens committed in one call (one chunk or several), ragged n_valid with
zeros, a slot map into a larger pool or none, a gate or none, and a ragged
comparator prefix with a key split of 1, 2, 3 or 5.  Every case runs, on the
same inputs: the commit, the step, the fused last step + commit, the feature
map of the queries, and the comparator (split and, with n_split = 1, not)."""
import numpy as np
import pytest
import torch

import block_hybrid_attention_amd as hba
import oracle
from block_hybrid_attention_amd import workloads as wl
from parity import check, report, row_rel, state_rel

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = 60
N_LARGE = 16   # cases N_CASES .. N_CASES + N_LARGE - 1: B = 24..48 at 8, 12 or 16 heads


@pytest.fixture(scope="module", autouse=True)
def _library():
    hba.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def draw(case):
    r = np.random.default_rng(12_000 + case)
    H = int(r.choice([1, 2, 3, 4, 6, 8, 16]))
    if case >= N_CASES:   # the large-batch cases: more (request, head) pairs than CUs
        H = int(r.choice([8, 12, 16]))
    divisors = [x for x in range(1, H + 1) if H % x == 0]
    if case >= N_CASES:
        B = int(r.integers(24, 49))
    else:
        B = int(r.integers(1, 25)) if r.random() < 0.8 else int(r.integers(16, 41))
    return dict(
        dtype=torch.bfloat16 if r.random() < 0.6 else torch.float32,
        d=int(r.choice([64, 128])), F=int(r.choice([64, 128])), H=H, Hkv=int(r.choice(divisors)), B=B,
        L=int(r.integers(1, 33)), T=int(r.integers(0, 101)), P=int(r.integers(0, 301)),
        ragged=bool(r.random() < 0.7), use_slot=bool(r.random() < 0.6), use_gate=bool(r.random() < 0.5),
        n_split=int(r.choice([1, 2, 3, 5])), seed=int(r.integers(1 << 30)))


@pytest.mark.parametrize("case", range(N_CASES + N_LARGE))
def test_random_shape_all_entry_points(case):
    c = draw(case)
    dt, d, F, H, Hkv, B, L, T, P = (c[k] for k in ("dtype", "d", "F", "H", "Hkv", "B", "L", "T", "P"))
    g = wl.generator(c["seed"], DEV)
    gr = torch.Generator().manual_seed(c["seed"])
    W = wl.feature_weights(H, d, F, dt, g, DEV)
    pk, pv = wl.normal((B, Hkv, T, d), 1, dt, g, DEV), wl.normal((B, Hkv, T, d), 1, dt, g, DEV)
    q = wl.normal((B, H, L, d), 1, dt, g, DEV)
    k, v = wl.normal((B, Hkv, L, d), 1, dt, g, DEV), wl.normal((B, Hkv, L, d), 1, dt, g, DEV)
    Kc, Vc = wl.normal((B, Hkv, P, d), 1, dt, g, DEV), wl.normal((B, Hkv, P, d), 1, dt, g, DEV)
    gate = wl.gate_from_alpha(H, g, DEV) if c["use_gate"] else None
    slots = B + (3 if c["use_slot"] else 0)
    slot = torch.randperm(slots, generator=gr)[:B].to(torch.int32).to(DEV) if c["use_slot"] else None
    nv_prefix = torch.randint(0, T + 1, (B,), generator=gr, dtype=torch.int32).to(DEV) if c["ragged"] else None
    nv_block = torch.randint(0, L + 1, (B,), generator=gr, dtype=torch.int32).to(DEV) if c["ragged"] else None
    plen = torch.randint(0, P + 1, (B,), generator=gr, dtype=torch.int32).to(DEV) if c["ragged"] else None
    S = 0.01 * torch.randn((slots, H, 2 * F, d), generator=g, device=DEV)
    Z = torch.rand((slots, H, 2 * F), generator=g, device=DEV)
    S0, Z0 = S.clone(), Z.clone()

    hba.commit(pk, pv, W, S, Z, n_valid=nv_prefix, slot=slot)
    out = hba.step(q, k, v, W, S, Z, gate=gate, slot=slot)
    S1, Z1 = S.clone(), Z.clone()
    out_f = hba.step_commit(q, k, v, W, S1, Z1, gate=gate, slot=slot, n_valid=nv_block)
    phi = hba.feature_map(q.transpose(1, 2).reshape(B * L, H, d).contiguous(), W)
    cmp = hba.prefix_softmax(q, k, v, Kc, Vc, prefix_len=plen, n_split=c["n_split"])
    torch.cuda.synchronize()

    Sr, Zr = oracle.commit(S0, Z0, pk, pv, W, n_valid=nv_prefix, slot=slot)
    ref = oracle.step(q, k, v, W, Sr, Zr, gate=gate, slot=slot)
    Sr1, Zr1 = oracle.commit(Sr, Zr, k, v, W, n_valid=nv_block, slot=slot)
    phi_ref = oracle.feature_map(q.transpose(1, 2).reshape(B * L, H, d), W)
    cmp_ref = oracle.prefix_softmax(q, k, v, Kc, Vc, prefix_len=plen)
    errs = dict(S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]), out=row_rel(out, ref),
                fused_out=row_rel(out_f, ref), fused_S=state_rel(S1, Sr1),
                fused_Z=state_rel(Z1[..., None], Zr1[..., None]), phi=row_rel(phi, phi_ref),
                comparator=row_rel(cmp, cmp_ref))
    shape = {k_: c[k_] for k_ in ("d", "F", "H", "Hkv", "B", "L", "T", "P", "n_split")}
    report(f"random case {case} {str(dt)[6:]} {shape}", **errs)
    check(errs, dt)
