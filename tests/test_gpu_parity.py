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
from parity import check, host64, report, row_rel, state_rel

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
    check(dict(phi=err), dtype)


def _device_cus() -> int:
    return int(torch.cuda.get_device_properties(0).multi_processor_count)


def _rows_for_tiles_per_group(kt: int, H: int) -> int:
    """Rows of one head that make the bf16 feature-map launcher pick kt 32-row
    tiles per workgroup (it takes the most tiles per workgroup that still fill
    one round of two workgroups per CU), with a last workgroup holding fewer
    tiles than the others and a ragged last tile of 13 rows."""
    rnd = 2 * _device_cus()
    tiles = -(-kt * rnd // H)                # fewest tiles that select kt
    tiles += 1 if kt == 2 else 2             # a short last workgroup
    assert tiles % kt and tiles * H < 2 * kt * rnd
    return 32 * tiles - 19


@pytest.mark.parametrize("kt", [1, 2, 4, 8])
@pytest.mark.parametrize("d,F", [(128, 128), (64, 128)])
def test_feature_map_tiles_per_workgroup(kt, d, F):
    """The bf16 feature map's 1-, 2-, 4- and 8-tile workgroups at 16 heads,
    each with a short last workgroup and a ragged last tile, every row
    against the oracle."""
    g = gen(170 + d + F + kt)
    H = 16
    n = 45 if kt == 1 else _rows_for_tiles_per_group(kt, H)
    x = wl.normal((n, H, d), 1.0, torch.bfloat16, g, DEV)
    W = wl.feature_weights(H, d, F, torch.bfloat16, g, DEV)
    phi = hba.feature_map(x, W)
    err = row_rel(phi, oracle.feature_map(x, W))
    report(f"feature_map bf16 n={n} H={H} d={d} F={F} ({kt} tiles per workgroup)", phi=err)
    check(dict(phi=err), torch.bfloat16)


@pytest.mark.parametrize("n", [4096, 32768])
def test_feature_map_serving_rows(n):
    """4096 rows x 16 heads (the rows of one serving step: 4 tiles per
    workgroup) compared in full, and 32768 x 16 (8 tiles per workgroup)
    compared on every 13th row and the whole last workgroup."""
    g = gen(180 + n)
    H, d, F = 16, 128, 128
    x = wl.normal((n, H, d), 1.0, torch.bfloat16, g, DEV)
    W = wl.feature_weights(H, d, F, torch.bfloat16, g, DEV)
    phi = hba.feature_map(x, W)
    rows = torch.arange(n) if n <= 4096 else torch.cat([torch.arange(0, n - 256, 13), torch.arange(n - 256, n)])
    err = row_rel(phi[rows.to(DEV)], oracle.feature_map(x[rows.to(DEV)], W))
    report(f"feature_map bf16 n={n} H={H} ({len(rows)} rows compared)", phi=err)
    check(dict(phi=err), torch.bfloat16)


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
    check(errs, torch.float32)


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
    check(errs, torch.bfloat16)


# --------------------------------------------------- serving step, B=128
def test_serving_b128_all_pairs():
    """128 requests, prefix 512..4096 (ragged, committed with n_valid), one step.
    The oracle commits every request's prefix itself and recomputes the step,
    so all 2048 (request, head) states and outputs are compared; every output
    is also checked for finiteness and for lying in the convex hull of the
    visible values."""
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
    errs = dict(S=0.0, Z=0.0, out=0.0)
    for b0 in range(0, B, 16):              # 16 requests at a time bounds host memory
        b1 = b0 + 16
        T = int(plen[b0:b1].max())
        Sr, Zr = oracle.commit(*host_pool(b1 - b0, H, F, d), pk[b0:b1, :, :T], pv[b0:b1, :, :T], W,
                               n_valid=plen[b0:b1])
        ref = oracle.step(q[b0:b1], k[b0:b1], v[b0:b1], W, Sr, Zr)
        errs["S"] = max(errs["S"], state_rel(S[b0:b1], Sr))
        errs["Z"] = max(errs["Z"], state_rel(Z[b0:b1, :, :, None], Zr[..., None]))
        errs["out"] = max(errs["out"], row_rel(out[b0:b1], ref))
    report("serving B=128, all 2048 pairs", **errs)
    check(errs, torch.bfloat16)


# ---------------------------------------------------- decode loop, B=32
def test_decode_loop_b32():
    """B=32: 256 blocks x (8 denoising steps, then commit of the last step's
    k, v); seed of (block n, step s) is 4e6 + 16 n + s.  Two loops run side by
    side on the same inputs: one calls hba_step eight times and then
    hba_commit, the other makes its eighth step hba_step_commit.  The oracle
    replays the loop for 4 requests x 16 heads (64 pairs) and checks, for both
    loops, the final step of every block, every step of every 32nd block and
    the states every 32 blocks."""
    B, H, L, d, F, nblk, nstep = 32, 16, 32, 128, 128, 256, 8
    dt = torch.bfloat16
    W = wl.feature_weights(H, d, F, dt, gen(wl.DECODE_B32_SEED - 1), DEV)
    S, Z = zeros_pool(B, H, F, d)
    S2, Z2 = zeros_pool(B, H, F, d)
    bs = [0, 11, 22, 31]
    bi = torch.tensor(bs, device=DEV)
    sel = lambda t: t[bi]  # noqa: E731
    Sr, Zr = host_pool(len(bs), H, F, d)
    errs = dict(out=0.0, out_fused=0.0, S=0.0, Z=0.0, S_fused=0.0, Z_fused=0.0)
    for n in range(nblk):
        every_step = n % 32 == 0
        for s in range(nstep):
            q, k, v = wl.block_qkv(B, H, L, d, dt, gen(wl.DECODE_B32_SEED + 16 * n + s), DEV)
            out = hba.step(q, k, v, W, S, Z)
            last = s == nstep - 1
            out2 = hba.step_commit(q, k, v, W, S2, Z2) if last else hba.step(q, k, v, W, S2, Z2)
            if last or every_step:
                ref = oracle.step(sel(q), sel(k), sel(v), W, Sr, Zr)
                errs["out"] = max(errs["out"], row_rel(sel(out), ref))
                errs["out_fused"] = max(errs["out_fused"], row_rel(sel(out2), ref))
        hba.commit(k, v, W, S, Z)
        Sr, Zr = oracle.commit(Sr, Zr, sel(k), sel(v), W)
        if n % 32 == 31:
            errs["S"] = max(errs["S"], state_rel(sel(S), Sr))
            errs["Z"] = max(errs["Z"], state_rel(sel(Z)[..., None], Zr[..., None]))
            errs["S_fused"] = max(errs["S_fused"], state_rel(sel(S2), Sr))
            errs["Z_fused"] = max(errs["Z_fused"], state_rel(sel(Z2)[..., None], Zr[..., None]))
    report("decode loop B=32, 256 blocks, 64 pairs, unfused and fused", **errs)
    check(errs, dt)


# --------------------------------------------------- comparator sweep
@pytest.mark.parametrize("P", wl.COMPARATOR_PREFIXES)
def test_comparator_sweep_sampled(P):
    """B=128, H=16, block 32 over a bf16 prefix cache of P tokens.  The same
    cache feeds the full-softmax comparator and the commit that builds the
    hybrid state; then the hybrid step runs on the same q, k, v.  The oracle
    recomputes the comparator, the commit of all P tokens and the hybrid step
    for 8 requests x 8 heads (64 pairs) at every P; every output is also
    checked for finiteness and for the convex hull."""
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
    bs, hs = [0, 18, 37, 55, 74, 92, 111, 127], [0, 3, 5, 7, 8, 10, 12, 15]
    bi, hi_ = torch.tensor(bs, device=DEV), torch.tensor(hs, device=DEV)
    sel = lambda t: t[bi][:, hi_]  # noqa: E731
    Kh, Vh = sel(Kc), sel(Vc)
    del Kc, Vc
    torch.cuda.empty_cache()
    errs = dict(comparator=row_rel(sel(cmp), oracle.prefix_softmax(sel(q), sel(k), sel(v), Kh, Vh)))
    Sr, Zr = oracle.commit(*host_pool(len(bs), len(hs), F, d), Kh, Vh, W[hi_])
    errs["hybrid"] = row_rel(sel(hyb), oracle.step(sel(q), sel(k), sel(v), W[hi_], Sr, Zr))
    errs["S"] = state_rel(sel(S), Sr)
    errs["Z"] = state_rel(sel(Z)[..., None], Zr[..., None])
    report(f"comparator sweep P={P}, 64 pairs", **errs)
    check(errs, dt)


# --------------------------------------------- one workgroup per pair, ragged L
@pytest.mark.parametrize("F", [128, 64])
@pytest.mark.parametrize("L", [1, 7, 17])
def test_step_ragged_block_one_workgroup_per_pair(L, F):
    """bf16, d = 128 with at least one (request, head) pair per CU, so the step
    runs one workgroup per pair (below that it splits the output columns over
    two): ragged blocks, a gate, a slot map and ragged commits, every pair
    against the oracle."""
    H, d = 16, 128
    B = max(16, -(-_device_cus() // H))
    assert B * H >= _device_cus()
    dt = torch.bfloat16
    g = gen(7600 + L + F)
    T = 45
    W = wl.feature_weights(H, d, F, dt, g, DEV)
    pk, pv = wl.normal((B, H, T, d), 1, dt, g, DEV), wl.normal((B, H, T, d), 1, dt, g, DEV)
    q, k, v = wl.block_qkv(B, H, L, d, dt, g, DEV)
    gate = wl.gate_from_alpha(H, g, DEV)
    slot = torch.randperm(B + 3, generator=g, device=DEV)[:B].to(torch.int32)
    n_valid = torch.randint(0, T + 1, (B,), generator=g, device=DEV, dtype=torch.int32)
    S, Z = zeros_pool(B + 3, H, F, d)
    S += 0.01 * torch.randn(S.shape, generator=g, device=DEV)
    Z += torch.rand(Z.shape, generator=g, device=DEV)
    S0, Z0 = S.clone(), Z.clone()
    hba.commit(pk, pv, W, S, Z, n_valid=n_valid, slot=slot)
    out = hba.step(q, k, v, W, S, Z, gate=gate, slot=slot)
    Sr, Zr = oracle.commit(S0, Z0, pk, pv, W, n_valid=n_valid, slot=slot)
    ref = oracle.step(q, k, v, W, Sr, Zr, gate=gate, slot=slot)
    errs = dict(S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]), out=row_rel(out, ref))
    report(f"one workgroup per pair B={B} H={H} L={L} F={F}", **errs)
    check(errs, dt)


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
    check(errs, dtype)


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
    check(errs, dt)


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
    check(errs, dtype)


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
    check(dict(out=err), dt)


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



@pytest.mark.parametrize("B,H", [(2, 4), (12, 16)])
def test_fused_step_commit_deterministic(B, H):
    """The fused step + commit, in both of its forms (two workgroups per pair
    at 8 pairs; at 192 pairs one workgroup per pair whose two feature halves
    add their partial sums in LDS), gives bitwise-equal outputs and states
    from bitwise-equal inputs, over two consecutive blocks."""
    L, d, F = 32, 128, 128
    dt = torch.bfloat16
    g = gen(8350 + B)
    W = wl.feature_weights(H, d, F, dt, g, DEV)
    S1, Z1 = zeros_pool(B, H, F, d)
    S1 += 0.01 * torch.randn(S1.shape, generator=g, device=DEV)
    Z1 += torch.rand(Z1.shape, generator=g, device=DEV)
    S2, Z2 = S1.clone(), Z1.clone()
    gate = wl.gate_from_alpha(H, g, DEV)
    for _ in range(2):
        q, k, v = wl.block_qkv(B, H, L, d, dt, g, DEV)
        o1 = hba.step_commit(q, k, v, W, S1, Z1, gate=gate)
        o2 = hba.step_commit(q, k, v, W, S2, Z2, gate=gate)
        assert torch.equal(o1, o2)
        assert torch.equal(S1, S2) and torch.equal(Z1, Z2)

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
    check(errs, dt)
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


# ------------------------------------------- one-block commit at serving shapes
@pytest.mark.parametrize("B,T,F,Hkv", [(128, 32, 128, 16), (37, 7, 128, 16), (64, 17, 64, 4), (40, 32, 128, 2)])
def test_commit_one_block_serving_shapes(B, T, F, Hkv):
    """The one-block bf16 commit at serving batch sizes (up to 128 requests x
    16 heads, two workgroups per pair): blocks shorter than 32, ragged n_valid
    with zeros, a slot map into a larger pool, grouped key/value heads; every
    state against the oracle, untouched slots and n_valid = 0 pairs bitwise."""
    H, d = 16, 128
    dt = torch.bfloat16
    g = gen(7700 + B + T + F + Hkv)
    W = wl.feature_weights(H, d, F, dt, g, DEV)
    k, v = wl.normal((B, Hkv, T, d), 1, dt, g, DEV), wl.normal((B, Hkv, T, d), 1, dt, g, DEV)
    slots = B + 5
    slot = torch.randperm(slots, generator=g, device=DEV)[:B].to(torch.int32)
    n_valid = torch.randint(0, T + 1, (B,), generator=g, device=DEV, dtype=torch.int32)
    n_valid[::9] = 0
    S, Z = zeros_pool(slots, H, F, d)
    S += 0.05 * torch.randn(S.shape, generator=g, device=DEV)
    Z += torch.rand(Z.shape, generator=g, device=DEV)
    S0, Z0 = S.clone(), Z.clone()
    hba.commit(k, v, W, S, Z, n_valid=n_valid, slot=slot)
    Sr, Zr = oracle.commit(S0, Z0, k, v, W, n_valid=n_valid, slot=slot)
    used = set(slot.tolist())
    for sl in range(slots):
        if sl not in used:
            assert torch.equal(S[sl], S0[sl]) and torch.equal(Z[sl], Z0[sl])
    for b in range(B):
        if int(n_valid[b]) == 0:
            sl = int(slot[b])
            assert torch.equal(S[sl], S0[sl]) and torch.equal(Z[sl], Z0[sl])
    errs = dict(S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]))
    report(f"one-block commit B={B} T={T} F={F} Hkv={Hkv}", **errs)
    check(errs, dt)


@pytest.mark.parametrize("B,T,F,Hkv,nvs", [
    (12, 192, 128, 16, [0, 1, 32, 33, 64, 65, 96, 97, 128, 160, 191, 192]),
    (12, 192, 64, 4, [192, 191, 160, 128, 97, 96, 65, 64, 33, 32, 1, 0]),
    (4, 2048, 128, 16, [2048, 2047, 1025, 33]),
    # 2 B H = 256 workgroups, at most one per CU on a 256-CU device: the
    # eight-wave form with 64-token chunks
    (8, 320, 128, 16, [0, 1, 64, 65, 128, 129, 257, 320]),
    (8, 320, 64, 4, [320, 319, 192, 191, 127, 64, 33, 0]),
])
def test_commit_multichunk_pipeline(B, T, F, Hkv, nvs):
    """The pipelined bf16 commit (more than one 32-token chunk, d = 128), in
    its four-wave (32-token chunks) and eight-wave (64-token chunks, grids of
    at most one workgroup per CU) forms: every chunk count over the requests,
    both parities of the two-chunk loop and its one-chunk tail, token counts
    that are not a multiple of the chunk, grouped key/value heads and a slot
    map into a larger pool; every state against the oracle, untouched slots
    and n_valid = 0 pairs bitwise."""
    H, d = 16, 128
    dt = torch.bfloat16
    g = gen(8800 + B + T + F + Hkv)
    W = wl.feature_weights(H, d, F, dt, g, DEV)
    k, v = wl.normal((B, Hkv, T, d), 1, dt, g, DEV), wl.normal((B, Hkv, T, d), 1, dt, g, DEV)
    slots = B + 3
    slot = torch.randperm(slots, generator=g, device=DEV)[:B].to(torch.int32)
    n_valid = torch.tensor(nvs, dtype=torch.int32, device=DEV)
    S, Z = zeros_pool(slots, H, F, d)
    S += 0.05 * torch.randn(S.shape, generator=g, device=DEV)
    Z += torch.rand(Z.shape, generator=g, device=DEV)
    S0, Z0 = S.clone(), Z.clone()
    hba.commit(k, v, W, S, Z, n_valid=n_valid, slot=slot)
    Sr, Zr = oracle.commit(S0, Z0, k, v, W, n_valid=n_valid, slot=slot)
    used = set(slot.tolist())
    for sl in range(slots):
        if sl not in used:
            assert torch.equal(S[sl], S0[sl]) and torch.equal(Z[sl], Z0[sl])
    for b in range(B):
        if nvs[b] == 0:
            sl = int(slot[b])
            assert torch.equal(S[sl], S0[sl]) and torch.equal(Z[sl], Z0[sl])
    errs = dict(S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]))
    report(f"multi-chunk commit B={B} T={T} F={F} Hkv={Hkv}", **errs)
    check(errs, dt)


# ------------------------------- both sides of the small-batch split threshold
@pytest.mark.parametrize("B", [8, 9])
@pytest.mark.parametrize("F", [128, 64])
def test_small_batch_split_threshold(B, F):
    """bf16, d = 128, 16 heads: at B = 8 the (request, head) pairs fill half
    of a 256-CU device and the step, the one-block commit and the fused step
    + commit each run two workgroups per pair; at B = 9 one.  Both sides
    against the oracle: a seeded prefix committed on both sides, then the
    step, the commit of a ragged block (n_valid with 0) and the fused call on
    a copy of the same states, through a slot map and with a gate."""
    H, L, d, P = 16, 32, 128, 40
    dt = torch.bfloat16
    g = gen(9600 + 10 * B + F)
    slots = B + 2
    slot = torch.randperm(slots, generator=torch.Generator().manual_seed(B + F))[:B].to(torch.int32).to(DEV)
    W = wl.feature_weights(H, d, F, dt, g, DEV)
    pk, pv = wl.normal((B, H, P, d), 1, dt, g, DEV), wl.normal((B, H, P, d), 1, dt, g, DEV)
    q, k, v = wl.block_qkv(B, H, L, d, dt, g, DEV)
    gate = wl.gate_from_alpha(H, g, DEV)
    n_valid = torch.tensor([(5 * b) % (L + 1) for b in range(B - 1)] + [L], dtype=torch.int32, device=DEV)
    S0, Z0 = zeros_pool(slots, H, F, d)
    S0 += 0.01 * torch.randn(S0.shape, generator=g, device=DEV)
    Z0 += torch.rand(Z0.shape, generator=g, device=DEV)
    S, Z = S0.clone(), Z0.clone()

    hba.commit(pk, pv, W, S, Z, slot=slot)
    Sp, Zp = oracle.commit(S0, Z0, pk, pv, W, slot=slot)
    S2, Z2 = S.clone(), Z.clone()
    out = hba.step(q, k, v, W, S, Z, gate=gate, slot=slot)
    hba.commit(k, v, W, S, Z, n_valid=n_valid, slot=slot)
    out_f = hba.step_commit(q, k, v, W, S2, Z2, gate=gate, slot=slot, n_valid=n_valid)

    ref = oracle.step(q, k, v, W, Sp, Zp, gate=gate, slot=slot)
    Sr, Zr = oracle.commit(Sp, Zp, k, v, W, n_valid=n_valid, slot=slot)
    errs = dict(out=row_rel(out, ref), S=state_rel(S, Sr), Z=state_rel(Z[..., None], Zr[..., None]),
                out_fused=row_rel(out_f, ref), S_fused=state_rel(S2, Sr), Z_fused=state_rel(Z2[..., None], Zr[..., None]))
    report(f"split threshold B={B} F={F}", **errs)
    check(errs, dt)
    used = set(slot.tolist())
    for s in range(slots):
        if s not in used:
            assert torch.equal(S[s], S0[s]) and torch.equal(S2[s], S0[s])
