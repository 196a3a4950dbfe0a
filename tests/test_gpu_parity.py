"""Parity of the HIP library with the fp64 oracle on the GPU.

Every case draws seeded inputs once (block_hybrid_attention_amd.workloads),
runs them through the C ABI and through the oracle, and compares element by
element within the tolerances of tests/parity.py.  Small cases compare every
output; the full-size workloads compare sampled (request, head) pairs that the
oracle recomputes from scratch, plus properties checked on every output.
"""
import numpy as np
import pytest
import torch

import block_hybrid_attention_amd as hba
import oracle
from block_hybrid_attention_amd import workloads as wl
from parity import TOL, host64, report, row_rel, state_rel

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _library():
    hba.load_library()          # a missing library fails loudly
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def gen(seed):
    return wl.generator(seed, DEV)


def zeros_pool(n_slots, H, F, d):
    return (torch.zeros((n_slots, H, 2 * F, d), device=DEV, dtype=torch.float32),
            torch.zeros((n_slots, H, 2 * F), device=DEV, dtype=torch.float32))


def host_pool(n_slots, H, F, d):
    return np.zeros((n_slots, H, 2 * F, d)), np.zeros((n_slots, H, 2 * F))


# ------------------------------------------------------------ feature map
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d,F", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_feature_map(dtype, d, F):
    g = gen(100 + d + F)
    H, n = 3, 45                                    # two 32-row tiles, ragged tail
    x = wl.normal((n, H, d), 1.0, dtype, g, DEV)
    W = wl.feature_weights(H, d, F, dtype, g, DEV)
    phi = hba.feature_map(x, W)
    err = row_rel(phi, oracle.feature_map(x, W))
    report(f"feature_map {dtype} d={d} F={F}", phi=err)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("d,F", [(128, 128), (64, 128)])
def test_feature_map_many_tiles(d, F):
    """Several workgroups of four 32-row tiles each, and a ragged last tile."""
    g = gen(170 + d + F)
    H, n = 3, 300
    x = wl.normal((n, H, d), 1.0, torch.bfloat16, g, DEV)
    W = wl.feature_weights(H, d, F, torch.bfloat16, g, DEV)
    phi = hba.feature_map(x, W)
    err = row_rel(phi, oracle.feature_map(x, W))
    report(f"feature_map bf16 n={n} d={d} F={F}", phi=err)
    assert err <= TOL[torch.bfloat16]


# ---------------------------------------------------- tiny fp32 workload
def test_tiny_fp32_workload():
    """1 request, 1 head, d = F = 64, 4 committed 8-token blocks, then a step."""
    c = wl.TINY_FP32
    g = gen(c.seed)
    B, H, L, d, F = c.batch, c.heads, c.block, c.head_dim, c.feat
    W = wl.feature_weights(H, d, F, c.dtype, g, DEV)
    S, Z = zeros_pool(B, H, F, d)
    Sr, Zr = host_pool(B, H, F, d)
    pk, pv = [], []
    for _ in range(c.prefix[0] // L):
        k, v = wl.normal((B, H, L, d), 1, c.dtype, g, DEV), wl.normal((B, H, L, d), 1, c.dtype, g, DEV)
        hba.commit(k, v, W, S, Z)
        Sr, Zr = oracle.commit(Sr, Zr, k, v, W)
        pk.append(k)
        pv.append(v)
    q, k, v = wl.block_qkv(B, H, L, d, c.dtype, g, DEV)
    out = hba.step(q, k, v, W, S, Z)
    ref = oracle.step(q, k, v, W, Sr, Zr)
    gate = torch.full((H,), 1e-3, device=DEV)       # linear branch dominates
    out_g = hba.step(q, k, v, W, S, Z, gate=gate)
    ref_g = oracle.step(q, k, v, W, Sr, Zr, gate=gate)
    Kc, Vc = torch.cat(pk, 2), torch.cat(pv, 2)
    cmp = hba.prefix_softmax(q, k, v, Kc, Vc)
    cmp_ref = oracle.prefix_softmax(q, k, v, Kc, Vc)
    phi = hba.feature_map(q[0].transpose(0, 1).contiguous(), W)
    phi_ref = oracle.feature_map(q[0].transpose(0, 1), W)
    errs = dict(S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]), out=row_rel(out, ref),
                out_gate=row_rel(out_g, ref_g), comparator=row_rel(cmp, cmp_ref), phi=row_rel(phi, phi_ref))
    report("tiny fp32", **errs)
    for e in errs.values():
        assert e <= TOL[torch.float32]


# ------------------------------------------------------------ bf16, B = 8
def test_bf16_b8_prefix2048():
    """B=8, H=16, d=F=128, L=32: 2048 prefix tokens in one commit, then a step;
    64 commits of 32 tokens must give the same state."""
    c = wl.BF16_B8
    g = gen(c.seed)
    B, H, L, d, F, P = c.batch, c.heads, c.block, c.head_dim, c.feat, c.prefix[0]
    W = wl.feature_weights(H, d, F, c.dtype, g, DEV)
    pk, pv = wl.normal((B, H, P, d), 1, c.dtype, g, DEV), wl.normal((B, H, P, d), 1, c.dtype, g, DEV)
    q, k, v = wl.block_qkv(B, H, L, d, c.dtype, g, DEV)
    S, Z = zeros_pool(B, H, F, d)
    hba.commit(pk, pv, W, S, Z)
    out = hba.step(q, k, v, W, S, Z)
    S2, Z2 = zeros_pool(B, H, F, d)
    for t0 in range(0, P, L):
        hba.commit(pk[:, :, t0:t0 + L].contiguous(), pv[:, :, t0:t0 + L].contiguous(), W, S2, Z2)
    out2 = hba.step(q, k, v, W, S2, Z2)
    Sr, Zr = oracle.commit(*host_pool(B, H, F, d), pk, pv, W)
    ref = oracle.step(q, k, v, W, Sr, Zr)
    errs = dict(S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]), out=row_rel(out, ref),
                S_chunked=state_rel(S2, Sr), out_chunked=row_rel(out2, ref),
                chunk_vs_whole=state_rel(S2, S))
    report("bf16 B=8 P=2048", **errs)
    for e in errs.values():
        assert e <= TOL[torch.bfloat16]
    # fp32 accumulation of exact bf16 products: far inside the bf16 bar
    assert errs["out"] <= 1e-4 and errs["S"] <= 1e-4


# --------------------------------------------------- serving step, B=128
def test_serving_b128_sampled():
    """128 requests, prefix 512..4096 (ragged, committed with n_valid), one step.
    The oracle recomputes 5 whole requests (80 pairs); every output is checked
    for finiteness and for lying in the convex hull of the visible values."""
    c = wl.serving_b128()
    g = gen(c.seed)
    B, H, L, d, F = c.batch, c.heads, c.block, c.head_dim, c.feat
    plen = torch.tensor(c.prefix, dtype=torch.int32)
    Pmax = int(plen.max())
    W = wl.feature_weights(H, d, F, c.dtype, g, DEV)
    pk, pv = wl.normal((B, H, Pmax, d), 1, c.dtype, g, DEV), wl.normal((B, H, Pmax, d), 1, c.dtype, g, DEV)
    q, k, v = wl.block_qkv(B, H, L, d, c.dtype, g, DEV)
    S, Z = zeros_pool(B, H, F, d)
    hba.commit(pk, pv, W, S, Z, n_valid=plen.to(DEV))
    out = hba.step(q, k, v, W, S, Z)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    # convex hull of block values and committed values, per (b, h, column)
    mask = (torch.arange(Pmax, device=DEV)[None, :] < plen.to(DEV)[:, None])[:, None, :, None]
    big = torch.tensor(float("inf"), device=DEV)
    lo = torch.minimum(torch.where(mask, pv.float(), big).amin(2), v.float().amin(2))
    hi = torch.maximum(torch.where(mask, pv.float(), -big).amax(2), v.float().amax(2))
    slack = 1e-5 * (hi - lo)
    assert bool((out >= lo[:, :, None] - slack[:, :, None]).all())
    assert bool((out <= hi[:, :, None] + slack[:, :, None]).all())
    del mask, lo, hi
    bs = sorted({int(plen.argmin()), int(plen.argmax()), 0, 63, 127})
    idx = torch.tensor(bs, device=DEV)
    Sr, Zr = oracle.commit(*host_pool(len(bs), H, F, d), pk[idx], pv[idx], W, n_valid=plen[bs])
    ref = oracle.step(q[idx], k[idx], v[idx], W, Sr, Zr)
    errs = dict(S=state_rel(S[idx], Sr), out=row_rel(out[idx], ref))
    report(f"serving B=128 requests {bs}", **errs)
    for e in errs.values():
        assert e <= TOL[torch.bfloat16]


# ---------------------------------------------------- decode loop, B=32
def test_decode_loop_b32_sampled():
    """B=32: 256 blocks x (8 denoising steps, then commit of the last step's
    k, v); seed of (block n, step s) is 4e6 + 16 n + s.  The oracle replays the
    loop for 2 requests x 4 heads and checks every block's final step and the
    final state."""
    B, H, L, d, F, nblk, nstep = 32, 16, 32, 128, 128, 256, 8
    dt = torch.bfloat16
    W = wl.feature_weights(H, d, F, dt, gen(wl.DECODE_B32_SEED - 1), DEV)
    S, Z = zeros_pool(B, H, F, d)
    bs, hs = [0, 31], [0, 5, 10, 15]
    bi, hi = torch.tensor(bs, device=DEV), torch.tensor(hs, device=DEV)
    Wh = W[hi]
    Sr, Zr = host_pool(len(bs), len(hs), F, d)
    worst = 0.0
    for n in range(nblk):
        for s in range(nstep):
            q, k, v = wl.block_qkv(B, H, L, d, dt, gen(wl.DECODE_B32_SEED + 16 * n + s), DEV)
            out = hba.step(q, k, v, W, S, Z)
        sel = lambda t: t[bi][:, hi]  # noqa: E731
        ref = oracle.step(sel(q), sel(k), sel(v), Wh, Sr, Zr)
        worst = max(worst, row_rel(sel(out), ref))
        hba.commit(k, v, W, S, Z)
        Sr, Zr = oracle.commit(Sr, Zr, sel(k), sel(v), Wh)
    errs = dict(out_worst_block=worst, S=state_rel(S[bi][:, hi], Sr),
                Z=state_rel(Z[bi][:, hi][..., None], Zr[..., None]))
    report("decode loop B=32, 256 blocks", **errs)
    for e in errs.values():
        assert e <= TOL[dt]


# --------------------------------------------------- comparator sweep
@pytest.mark.parametrize("P", wl.COMPARATOR_PREFIXES)
def test_comparator_sweep_sampled(P):
    """B=128, H=16, block 32 over a bf16 prefix cache of P tokens: full softmax
    comparator vs oracle on 6 sampled pairs; the hybrid step with the same
    cache committed is checked against the oracle where the oracle commit is
    cheap (P <= 4096) and for finiteness and the convex hull at any P."""
    B, H, L, d, F = 128, 16, 32, 128, 128
    dt = torch.bfloat16
    g = gen(5_000_000 + P)
    W = wl.feature_weights(H, d, F, dt, g, DEV)
    Kc, Vc = wl.normal((B, H, P, d), 1, dt, g, DEV), wl.normal((B, H, P, d), 1, dt, g, DEV)
    q, k, v = wl.block_qkv(B, H, L, d, dt, g, DEV)
    cmp = hba.prefix_softmax(q, k, v, Kc, Vc)
    S, Z = zeros_pool(B, H, F, d)
    hba.commit(Kc, Vc, W, S, Z)
    hyb = hba.step(q, k, v, W, S, Z)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(cmp).all()) and bool(torch.isfinite(hyb).all())
    lo = torch.minimum(Vc.amin(2), v.amin(2)).float()[:, :, None]
    hi = torch.maximum(Vc.amax(2), v.amax(2)).float()[:, :, None]
    for o in (cmp, hyb):
        assert bool((o >= lo - 1e-5).all()) and bool((o <= hi + 1e-5).all())
    bs, hs = [0, 77, 127], [0, 9]
    bi, hi_ = torch.tensor(bs, device=DEV), torch.tensor(hs, device=DEV)
    sel = lambda t: t[bi][:, hi_]  # noqa: E731
    errs = dict(comparator=row_rel(sel(cmp), oracle.prefix_softmax(sel(q), sel(k), sel(v), sel(Kc), sel(Vc))))
    if P <= 4096:
        Sr, Zr = oracle.commit(*host_pool(len(bs), len(hs), F, d), sel(Kc), sel(Vc), W[hi_])
        errs["hybrid"] = row_rel(sel(hyb), oracle.step(sel(q), sel(k), sel(v), W[hi_], Sr, Zr))
        errs["S"] = state_rel(sel(S), Sr)
    report(f"comparator sweep P={P}", **errs)
    for e in errs.values():
        assert e <= TOL[dt]
    del Kc, Vc
    torch.cuda.empty_cache()


# ---------------------------------------------------------- edge cases
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d,F", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("L", [1, 7, 17, 32])
def test_step_commit_shapes_slots_gate(dtype, d, F, L):
    """Ragged blocks, every (d, F), a slot map into a larger pool, ragged
    commits (n_valid incl. 0, T not a multiple of 32), a non-trivial gate."""
    g = gen(7000 + 97 * d + 13 * F + L + (0 if dtype == torch.float32 else 1))
    B, H, T, slots = 3, 2, 45, 5
    W = wl.feature_weights(H, d, F, dtype, g, DEV)
    pk, pv = wl.normal((B, H, T, d), 1, dtype, g, DEV), wl.normal((B, H, T, d), 1, dtype, g, DEV)
    q, k, v = wl.block_qkv(B, H, L, d, dtype, g, DEV)
    gate = wl.gate_from_alpha(H, g, DEV)
    slot = torch.tensor([4, 0, 2], dtype=torch.int32, device=DEV)
    n_valid = torch.tensor([45, 0, 13], dtype=torch.int32, device=DEV)
    S, Z = zeros_pool(slots, H, F, d)
    S += 0.01 * torch.randn(S.shape, generator=g, device=DEV)   # slot 1 and 3: untouched data
    Z += torch.rand(Z.shape, generator=g, device=DEV)
    S0, Z0 = S.clone(), Z.clone()
    hba.commit(pk, pv, W, S, Z, n_valid=n_valid, slot=slot)
    out = hba.step(q, k, v, W, S, Z, gate=gate, slot=slot)
    Sr, Zr = oracle.commit(S0, Z0, pk, pv, W, n_valid=n_valid, slot=slot)
    ref = oracle.step(q, k, v, W, Sr, Zr, gate=gate, slot=slot)
    assert torch.equal(S[1], S0[1]) and torch.equal(S[3], S0[3]) and torch.equal(Z[1], Z0[1])
    assert torch.equal(S[0], S0[0]) and torch.equal(Z[0], Z0[0])    # n_valid 0: untouched
    errs = dict(S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]), out=row_rel(out, ref))
    report(f"shapes {dtype} d={d} F={F} L={L}", **errs)
    for e in errs.values():
        assert e <= TOL[dtype]


@pytest.mark.parametrize("T", [32, 45])
def test_commit_grid_with_partial_group(T):
    """bf16 commit over 20 (request, head) pairs: the two state halves of each
    pair go to workgroups 8 apart in whole groups of 16 and to neighbours in
    the last, partial group (pairs 16..19); every state against the oracle,
    through a slot map that reverses the requests."""
    g = gen(7400 + T)
    B, H, d, F = 5, 4, 128, 128
    dt = torch.bfloat16
    W = wl.feature_weights(H, d, F, dt, g, DEV)
    pk, pv = wl.normal((B, H, T, d), 1, dt, g, DEV), wl.normal((B, H, T, d), 1, dt, g, DEV)
    slot = torch.arange(B - 1, -1, -1, dtype=torch.int32, device=DEV)
    S, Z = zeros_pool(B, H, F, d)
    S += 0.01 * torch.randn(S.shape, generator=g, device=DEV)
    Z += torch.rand(Z.shape, generator=g, device=DEV)
    S0, Z0 = S.clone(), Z.clone()
    hba.commit(pk, pv, W, S, Z, slot=slot)
    Sr, Zr = oracle.commit(S0, Z0, pk, pv, W, slot=slot)
    errs = dict(S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]))
    report(f"commit B={B} H={H} T={T}", **errs)
    for e in errs.values():
        assert e <= TOL[dt]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("L", [1, 32])
def test_empty_state_is_block_softmax_and_matches_comparator(dtype, L):
    g = gen(8100 + L)
    B, H, d, F = 4, 3, 128, 128
    W = wl.feature_weights(H, d, F, dtype, g, DEV)
    q, k, v = wl.block_qkv(B, H, L, d, dtype, g, DEV)
    S, Z = zeros_pool(B, H, F, d)
    out = hba.step(q, k, v, W, S, Z)
    empty = torch.empty((B, H, 0, d), dtype=dtype, device=DEV)
    cmp = hba.prefix_softmax(q, k, v, empty, empty)
    ref = oracle.step(q, k, v, W, host64(S), host64(Z))
    errs = dict(step=row_rel(out, ref), comparator=row_rel(cmp, ref), step_vs_cmp=row_rel(out, cmp))
    report(f"empty state {dtype} L={L}", **errs)
    for e in errs.values():
        assert e <= TOL[dtype]


def test_comparator_ragged_prefix_len():
    g = gen(8200)
    B, H, L, d, P = 4, 2, 17, 64, 300
    dt = torch.bfloat16
    q, k, v = wl.block_qkv(B, H, L, d, dt, g, DEV)
    Kc, Vc = wl.normal((B, H, P, d), 1, dt, g, DEV), wl.normal((B, H, P, d), 1, dt, g, DEV)
    plen = torch.tensor([300, 0, 1, 129], dtype=torch.int32, device=DEV)
    out = hba.prefix_softmax(q, k, v, Kc, Vc, prefix_len=plen)
    ref = oracle.prefix_softmax(q, k, v, Kc, Vc, prefix_len=plen)
    err = row_rel(out, ref)
    report("comparator ragged prefix", out=err)
    assert err <= TOL[dt]


def test_deterministic_and_resumable():
    """Same inputs give bitwise-equal states and outputs (no atomics); a state
    saved from one slot and restored into another continues bitwise equal."""
    g = gen(8300)
    B, H, L, d, F = 2, 4, 32, 128, 128
    dt = torch.bfloat16
    W = wl.feature_weights(H, d, F, dt, g, DEV)
    k1, v1 = wl.normal((B, H, 64, d), 1, dt, g, DEV), wl.normal((B, H, 64, d), 1, dt, g, DEV)
    k2, v2 = wl.normal((B, H, 32, d), 1, dt, g, DEV), wl.normal((B, H, 32, d), 1, dt, g, DEV)
    q, k, v = wl.block_qkv(B, H, L, d, dt, g, DEV)
    pool = hba.StatePool(6, H, d, F, device=DEV)
    a = pool.alloc(B)
    hba.commit(k1, v1, W, pool.S, pool.Z, slot=a)
    S_a, Z_a = pool.S.clone(), pool.Z.clone()
    pool2 = hba.StatePool(6, H, d, F, device=DEV)
    a2 = pool2.alloc(B)
    hba.commit(k1, v1, W, pool2.S, pool2.Z, slot=a2)
    assert torch.equal(pool2.S, S_a) and torch.equal(pool2.Z, Z_a)
    saved = pool.save(a)
    bslots = pool.alloc(B)
    pool.restore(bslots, saved)
    for s in (a, bslots):
        hba.commit(k2, v2, W, pool.S, pool.Z, slot=s)
    o1 = hba.step(q, k, v, W, pool.S, pool.Z, slot=a)
    o2 = hba.step(q, k, v, W, pool.S, pool.Z, slot=bslots)
    o3 = hba.step(q, k, v, W, pool.S, pool.Z, slot=a)
    assert torch.equal(pool.S[a.long()], pool.S[bslots.long()])
    assert torch.equal(o1, o2) and torch.equal(o1, o3)


def test_int64_state_offsets():
    """A slot whose state starts past 2^31 fp32 elements of the pool."""
    H, d, F = 16, 128, 128
    per_slot = H * 2 * F * d
    n_slots = (1 << 31) // per_slot + 4
    dt = torch.bfloat16
    g = gen(8400)
    W = wl.feature_weights(H, d, F, dt, g, DEV)
    k1, v1 = wl.normal((1, H, 96, d), 1, dt, g, DEV), wl.normal((1, H, 96, d), 1, dt, g, DEV)
    q, k, v = wl.block_qkv(1, H, 32, d, dt, g, DEV)
    S, Z = zeros_pool(n_slots, H, F, d)
    slot = torch.tensor([n_slots - 1], dtype=torch.int32, device=DEV)
    hba.commit(k1, v1, W, S, Z, slot=slot)
    out = hba.step(q, k, v, W, S, Z, slot=slot)
    Sr, Zr = oracle.commit(*host_pool(1, H, F, d), k1, v1, W)
    ref = oracle.step(q, k, v, W, Sr, Zr)
    errs = dict(S=state_rel(S[n_slots - 1:], Sr), out=row_rel(out, ref))
    # the fused last step + commit on the same far slot
    out2 = hba.step_commit(q, k, v, W, S, Z, slot=slot)
    Sr2, Zr2 = oracle.commit(Sr, Zr, k, v, W)
    errs.update(fused_out=row_rel(out2, ref), fused_S=state_rel(S[n_slots - 1:], Sr2),
                fused_Z=state_rel(Z[n_slots - 1:, :, :, None], Zr2[..., None]))
    report("int64 offsets", **errs)
    assert float(S[: n_slots - 1].abs().max()) == 0.0 and float(Z[: n_slots - 1].abs().max()) == 0.0
    for e in errs.values():
        assert e <= TOL[dt]
    del S, Z
    torch.cuda.empty_cache()


def test_zero_batch_noop_on_device():
    dt = torch.bfloat16
    q = torch.empty((0, 2, 32, 64), dtype=dt, device=DEV)
    W = torch.zeros((2, 64, 64), dtype=dt, device=DEV)
    S, Z = zeros_pool(1, 2, 64, 64)
    out = hba.step(q, q, q, W, S, Z)
    hba.commit(q, q, W, S, Z)
    assert out.shape == (0, 2, 32, 64) and float(S.abs().sum()) == 0.0
