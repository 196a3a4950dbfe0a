"""Benchmark: block-hybrid attention denoising step, 128 concurrent requests.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --comparator     # hybrid step vs full softmax over P-token caches
    python bench.py --decode-loop    # B=32 decode loop: 8 steps + 1 commit per block
    python bench.py --commit-sweep   # whole-prefix commits (pipelined kernel), B=8..128
    python bench.py --small-batch    # step, commit, fused step + commit at B=1..32 (HIP graphs)

Workload (one hybrid layer): 128 requests, 16 heads, head_dim 128, F = 128
(phi dim 256), active block 32 tokens, bf16 q/k/v/W ~ N(0,1) / N(0,1/d), fp32
states S [256][128] and Z [256] per (request, head) built by hba_commit from
seeded bf16 prefixes of 512..4096 tokens (uniform, whole 32-token blocks).

A timed step is one hba_step over the whole batch (feature map of q, block
softmax, linear readout of the states, gated shared-normaliser merge), with
inputs resident in HBM.  Four independent state/input sets (1.3 GB) rotate so
the 256 MB last-level cache cannot hold the state between steps.

Prints ONE JSON line: query tokens/s (B*L/t_step), the roofline of hba_step
(algorithmic bytes per launch / mean launch time, i.e. K back-to-back launches
between two HIP events on the launch stream, against the 8 TB/s HBM peak) and the fp64 oracle's rate on the host cores for a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "active-block query tokens/sec per hybrid layer at B=128; % of HBM peak"
HBM_PEAK_GBS = 8000.0
N_SETS = 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "step_serving_b128_traffic.json")
STEP_SOURCES = ["block_hybrid_attention_amd/csrc/hba_step.hip",
                "block_hybrid_attention_amd/csrc/hba_device.h"]


def step_source_hash() -> str:
    h = hashlib.sha256()
    for p in STEP_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def step_bytes(B, H, L, d, F, in_bytes=2) -> int:
    """Algorithmic HBM bytes of one hba_step launch: each input read once,
    the output written once (S and Z fp32, q/k/v/W in_dtype, out fp32)."""
    state = B * H * 2 * F * (d + 1) * 4
    qkv = 3 * B * H * L * d * in_bytes
    w = H * d * F * in_bytes
    out = B * H * L * d * 4
    return state + qkv + w + out


def commit_bytes(B, H, T, d, F, in_bytes=2) -> int:
    """Algorithmic bytes of one hba_commit: state read + written, k/v/W read."""
    return 2 * B * H * 2 * F * (d + 1) * 4 + 2 * B * H * T * d * in_bytes + H * d * F * in_bytes


def load_traffic(kernel_hash):
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_hash:
        return None       # counters were taken on an older kernel
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, W, pk_host, pv_host, plen, q, k, v, n_req: int, seconds: float):
    """fp64 oracle on the host cores: commit (untimed) then step for the first
    n_req requests of the workload, repeated for about `seconds`."""
    import numpy as np
    import oracle

    H, F, d = W.shape[0], W.shape[2], W.shape[1]
    S0, Z0 = np.zeros((n_req, H, 2 * F, d)), np.zeros((n_req, H, 2 * F))
    Sr, Zr = oracle.commit(S0, Z0, pk_host, pv_host, W, n_valid=plen[:n_req])
    qh, kh, vh = (oracle._f64(t[:n_req]) for t in (q, k, v))
    Wh = oracle._f64(W)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.step(qh, kh, vh, Wh, Sr, Zr)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    L = q.shape[2]
    return {"value": n_req * L * reps / el, "unit": "query tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": (f"fp64 C oracle step for the first {n_req} of 128 requests (all 16 heads, "
                       f"states from the oracle's own commit of their seeded prefixes), "
                       f"{reps} repetitions in {el:.1f} s")}


def _time_launches(torch, fn, warmup, iters, stream):
    """Mean time per launch (ms): `iters` back-to-back launches bracketed by
    two HIP events on the launch stream (an event pair around every launch
    would put its own packets between the kernels)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def _time_graph(torch, fn, n, reps, stream):
    """Mean time per call (ms) of `fn` captured `n` times in one HIP graph and
    replayed `reps` times between two events: the host is out of the loop,
    which matters for launches of a few microseconds."""
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / (n * reps)


def comparator_sweep(args, torch, hba, wl, dev, B=128):
    """Full softmax attention over a P-token bf16 KV cache (the layer the
    hybrid replaces) against the hybrid step reading the fixed-size state
    built from the same cache: B requests, 16 heads, d=128, block 32.  Below
    one (request, head) pair per compute unit the comparator is also timed
    with its keys split over workgroups (the library's choice, and a sweep)."""
    H, L, d, F = 16, 32, 128, 128
    dt = torch.bfloat16
    stream = torch.cuda.current_stream()
    rows = []
    for P in wl.COMPARATOR_PREFIXES:
        g = wl.generator(5_000_000 + P, dev)
        W = wl.feature_weights(H, d, F, dt, g, dev)
        Kc = wl.normal((B, H, P, d), 1.0, dt, g, dev)
        Vc = wl.normal((B, H, P, d), 1.0, dt, g, dev)
        q, k, v = wl.block_qkv(B, H, L, d, dt, g, dev)
        S = torch.zeros((B, H, 2 * F, d), device=dev)
        Z = torch.zeros((B, H, 2 * F), device=dev)
        hba.commit(Kc, Vc, W, S, Z)
        out_c = torch.empty((B, H, L, d), device=dev)
        out_h = torch.empty((B, H, L, d), device=dev)
        n = max(3, min(args.steps, 20 if P >= 16384 else 50))
        cm = _time_launches(torch, lambda: hba.prefix_softmax(q, k, v, Kc, Vc, out=out_c), 2, n, stream)
        hm = _time_launches(torch, lambda: hba.step(q, k, v, W, S, Z, out=out_h), 3, n, stream)
        hg = _time_graph(torch, lambda: hba.step(q, k, v, W, S, Z, out=out_h), 20, 5, stream)
        kv_bytes = 2 * B * H * P * d * 2
        c_bytes = kv_bytes + 3 * B * H * L * d * 2 + B * H * L * d * 4
        row = {"prefix": P, "comparator_ms": cm,
               "comparator_GBps": c_bytes / (cm * 1e-3) / 1e9,
               "hybrid_ms": hm,
               "hybrid_GBps": step_bytes(B, H, L, d, F) / (hm * 1e-3) / 1e9,
               "speedup": cm / hm, "comparator_kv_bytes": kv_bytes,
               "hybrid_graph_ms": hg, "speedup_vs_hybrid_graph": cm / hg}
        ns_auto = hba.prefix_softmax_auto_split(B, H, L, d, P)
        if ns_auto > 1:
            ws = torch.empty(hba.prefix_softmax_workspace_bytes(B, H, L, d, 64) // 4, device=dev)
            sweep = {}
            for ns in sorted({2, 4, 8, 16, 32, 64, ns_auto}):
                sweep[ns] = _time_launches(torch, lambda: hba.prefix_softmax(
                    q, k, v, Kc, Vc, out=out_c, n_split=ns, workspace=ws), 2, n, stream)
            ref = hba.prefix_softmax(q, k, v, Kc, Vc, n_split=1)
            hba.prefix_softmax(q, k, v, Kc, Vc, out=out_c, n_split=ns_auto, workspace=ws)
            torch.cuda.synchronize()
            err = float(((out_c - ref).norm(dim=-1) / ref.norm(dim=-1)).max())
            sm = sweep[ns_auto]
            row.update({"split_auto": ns_auto, "split_ms": sm,
                        "split_GBps": c_bytes / (sm * 1e-3) / 1e9, "split_speedup_vs_hybrid": sm / hm,
                        "split_speedup_vs_hybrid_graph": sm / hg,
                        "split_sweep_ms": sweep, "split_vs_unsplit_max_row_rel": err})
            del ws
        rows.append(row)
        del Kc, Vc, S, Z
        torch.cuda.empty_cache()
    print(json.dumps({"mode": "comparator_sweep", "batch": B, "heads": H, "block": L, "head_dim": d,
                      "feat": F, "dtype": "bf16 inputs, fp32 accumulate", "unit": "ms per 32-token block",
                      "rows": rows}), flush=True)


def transfer_flops(d, F, L) -> int:
    """Algorithmic flops of stage-1 attention transfer per (token, head):
    phi(q) and phi(k) (2 x 2dF), block scores and A V (2 x 2Ld), the linear
    readout and the commit (2 x 2(2F)d), dphi(q) and dphi(k) (2 x 2(2F)d),
    the suffix state G (2(2F)d), and dW from the query and key sides (2 x 2dF)."""
    return 2 * 2 * d * F + 2 * 2 * L * d + 5 * 2 * (2 * F) * d + 2 * 2 * d * F


def transfer_mfma_bf16(F) -> int:
    """v_mfma_f32_16x16x32_bf16 instructions the bf16 path of hba_transfer
    issues per 32-row token tile and head (all three sweeps; fp32 operands
    split into high and residual parts count once per part product):
    forward: projections 32 NFT, scores 16, P V 32, linear readout 24 NPT,
    commit 16 NPT; query sweep: projections 32 NFT, dphi 192 FW, fold 144 FW,
    dW 32 NWT; key sweep: projections 32 NFT, dphi 128 FW, fold 216 FW,
    dW 32 NWT (NFT = F/16, NPT = 2F/16, FW = NPT/8, NWT = F/16)."""
    nft, npt = F // 16, 2 * F // 16
    fw, nwt = npt // 8, F // 16
    fwd = 32 * nft + 16 + 32 + 24 * npt + 16 * npt
    qsw = 32 * nft + 192 * fw + 144 * fw + 32 * nwt
    ksw = 32 * nft + 128 * fw + 216 * fw + 32 * nwt
    return fwd + qsw + ksw


def transfer_bench(args, torch, hba, wl, dev):
    """Stage-1 attention transfer: loss and dW, dalpha for 16 sequences of
    2048 tokens (64 blocks of 32) x 16 heads, d = F = 128, bf16 inputs,
    fp32 accumulation (bf16 MFMA with split operands), against a synthetic
    teacher output."""
    B, H, L, nb, d, F = 16, 16, 32, 64, 128, 128
    N = nb * L
    g = wl.generator(6_000_000, dev)
    q, k, v = (wl.normal((B, H, N, d), 1.0, torch.bfloat16, g, dev) for _ in range(3))
    W = wl.feature_weights(H, d, F, torch.bfloat16, g, dev)
    alpha = torch.randn(H, generator=g, device=dev)
    target = 0.3 * torch.randn((B, H, N, d), generator=g, device=dev)
    ws = torch.empty(hba.transfer_workspace_bytes(B, H, L, d, F, nb) // 4, device=dev)
    stream = torch.cuda.current_stream()
    ms = _time_launches(torch, lambda: hba.transfer(q, k, v, W, alpha, target, L, workspace=ws), 2,
                        max(3, min(args.steps, 10)), stream)
    fl = transfer_flops(d, F, L) * B * H * N
    issued = transfer_mfma_bf16(F) * 16 * 16 * 32 * 2 * B * H * nb
    print(json.dumps({"mode": "transfer", "batch": B, "heads": H, "tokens": N, "block": L, "head_dim": d,
                      "feat": F, "dtype": "bf16 inputs; bf16 MFMA, fp32 operands split into high and residual "
                      "parts, fp32 accumulation", "ms": ms,
                      "tokens_per_s": B * N / (ms * 1e-3), "algorithmic_flops": fl,
                      "TFLOPs": fl / (ms * 1e-3) / 1e12, "bf16_mfma_peak_TFLOPs": 2500.0,
                      "frac_of_bf16_mfma_peak": fl / (ms * 1e-3) / 1e12 / 2500.0,
                      "bf16_mfma_issued_TFLOPs": issued / (ms * 1e-3) / 1e12,
                      "issued_frac_of_bf16_mfma_peak": issued / (ms * 1e-3) / 1e12 / 2500.0}), flush=True)


def commit_sweep(args, torch, hba, wl, dev):
    """hba_commit of whole prefixes in one call (bf16, H=16, d=F=128): the
    pipelined multi-chunk kernel.  Shapes: the 2048-token prefix of the
    B = 8 workload, and 512, 256 and 2048 tokens at B = 32 and 128.  Each
    call starts from its own state set (two or more rotate, > 600 MB in all
    when they fit); the state is read and written once, k and v read once."""
    H, d, F = 16, 128, 128
    rows = []
    for B, T in ((8, 2048), (32, 512), (128, 256), (128, 2048)):
        g = wl.generator(41 + B + T, dev)
        W = wl.feature_weights(H, d, F, torch.bfloat16, g, dev)
        k = wl.normal((B, H, T, d), 1.0, torch.bfloat16, g, dev)
        v = wl.normal((B, H, T, d), 1.0, torch.bfloat16, g, dev)
        per_set = B * H * (2 * F * d + 2 * F) * 4
        nsets = max(2, min(8, -(-600_000_000 // per_set)))
        sets = [(torch.zeros((B, H, 2 * F, d), device=dev), torch.zeros((B, H, 2 * F), device=dev))
                for _ in range(nsets)]
        it = [0]

        def fn():
            S, Z = sets[it[0] % nsets]
            it[0] += 1
            hba.commit(k, v, W, S, Z)

        n = max(4, min(args.steps, 40 if T <= 512 else 10))
        ms = _time_launches(torch, fn, 2, n, torch.cuda.current_stream())
        nb = commit_bytes(B, H, T, d, F)
        rows.append({"batch": B, "tokens": T, "us": ms * 1e3, "M_tokens_per_s": B * T / (ms * 1e-3) / 1e6,
                     "TBps": nb / (ms * 1e-3) / 1e12, "algorithmic_bytes": nb, "state_sets": nsets})
        print(json.dumps({"mode": "commit_sweep", **rows[-1]}), flush=True)
        del k, v, sets
        torch.cuda.empty_cache()
    return rows


def small_batch(args, torch, hba, wl, dev):
    """The decode-path calls at small batches (bf16, H=16, d=F=128, L=32):
    hba_step, the one-block hba_commit and hba_step_commit, each replayed
    from a HIP graph (a decode loop's launches; one launch takes a few
    microseconds, so the host is kept out of the timing) over rotating state
    sets.  Below half a workgroup per CU the library splits each (request,
    head) over two workgroups; these batch sizes show both sides of that."""
    H, L, d, F = 16, 32, 128, 128
    batches = [int(x) for x in (args.batch if args.batch != "128" else "1,4,8,12,16,32").split(",")]
    stream = torch.cuda.current_stream()
    rows = []
    for B in batches:
        g = wl.generator(57 + B, dev)
        W = wl.feature_weights(H, d, F, torch.bfloat16, g, dev)
        q, k, v = wl.block_qkv(B, H, L, d, torch.bfloat16, g, dev)
        per_set = B * H * (2 * F * d + 2 * F) * 4
        nsets = max(2, min(16, -(-600_000_000 // per_set)))
        sets = [(wl.normal((B, H, 2 * F, d), 0.01, torch.float32, g, dev),
                 torch.rand((B, H, 2 * F), generator=g, device=dev) * 20 + 1) for _ in range(nsets)]
        out = torch.empty((B, H, L, d), device=dev)
        it = [0]

        def nxt():
            S, Z = sets[it[0] % nsets]
            it[0] += 1
            return S, Z

        calls = {"step": lambda: hba.step(q, k, v, W, *nxt(), out=out),
                 "commit": lambda: hba.commit(k, v, W, *nxt()),
                 "step_commit": lambda: hba.step_commit(q, k, v, W, *nxt(), out=out)}
        row = {"batch": B, "items": B * H}
        for name, fn in calls.items():
            row[name + "_us"] = _time_graph(torch, fn, nsets, max(2, args.steps // nsets), stream) * 1e3
        rows.append(row)
        print(json.dumps({"mode": "small_batch", **row}), flush=True)
        del sets
        torch.cuda.empty_cache()
    return rows


def batch_sweep(args, torch, hba, wl, dev):
    """hba_step (bf16, H=16, d=F=128, L=32) over batch sizes, with enough
    rotating state sets (> 600 MB) that the 256 MB Infinity Cache holds none
    of them.  A least-squares line t = t0 + items / R over the batches that
    fill the CUs at least once splits the launch time into a fixed part t0
    (ramp-up, and the last workgroups' epilogue and output drain) and the
    marginal HBM rate R of the state stream."""
    H, L, d, F = 16, 32, 128, 128
    batches = [int(x) for x in (args.batch if args.batch != "128" else "16,32,48,64,96,112,128,144,160,192").split(",")]
    rows = []
    for B in batches:
        g = wl.generator(31 + B, dev)
        W = wl.feature_weights(H, d, F, torch.bfloat16, g, dev)
        q, k, v = wl.block_qkv(B, H, L, d, torch.bfloat16, g, dev)
        per_set = B * H * (2 * F * d + 2 * F) * 4
        nsets = max(2, -(-600_000_000 // per_set))
        sets = [(wl.normal((B, H, 2 * F, d), 0.01, torch.float32, g, dev),
                 torch.rand((B, H, 2 * F), generator=g, device=dev) * 20 + 1) for _ in range(nsets)]
        out = torch.empty((B, H, L, d), device=dev)
        it = [0]

        def fn():
            S, Z = sets[it[0] % nsets]
            it[0] += 1
            hba.step(q, k, v, W, S, Z, out=out)

        ms = _time_launches(torch, fn, max(args.warmup, nsets), args.steps, torch.cuda.current_stream())
        nb = step_bytes(B, H, L, d, F)
        rows.append({"batch": B, "items": B * H, "us": ms * 1e3, "TBps": nb / (ms * 1e-3) / 1e12,
                     "state_sets": nsets})
        print(json.dumps({"mode": "batch_sweep", **rows[-1]}), flush=True)
        del sets
        torch.cuda.empty_cache()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    # three step workgroups are resident per CU; below that the launch is one partial round
    fit = [r for r in rows if r["items"] >= 3 * cus]
    if len(fit) >= 2:
        n = len(fit)
        mx = sum(r["items"] for r in fit) / n
        my = sum(r["us"] for r in fit) / n
        slope = sum((r["items"] - mx) * (r["us"] - my) for r in fit) / sum((r["items"] - mx) ** 2 for r in fit)
        t0 = my - slope * mx
        item_bytes = (step_bytes(128, H, L, d, F) - H * d * F * 2) / (128 * H)
        print(json.dumps({"mode": "batch_sweep_fit", "batches": [r["batch"] for r in fit],
                          "fixed_us": t0, "us_per_item": slope,
                          "marginal_TBps": item_bytes / (slope * 1e-6) / 1e12,
                          "marginal_frac_of_8TBps": item_bytes / (slope * 1e-6) / 8e12}), flush=True)


def decode_loop(args, torch, hba, wl, dev):
    """One hybrid layer through a block-diffusion decode: per 32-token block,
    8 denoising steps (hba_step) then hba_commit of the block; 32 requests."""
    B, H, L, d, F, nsteps = 32, 16, 32, 128, 128, 8
    dt = torch.bfloat16
    stream = torch.cuda.current_stream()
    W = wl.feature_weights(H, d, F, dt, wl.generator(wl.DECODE_B32_SEED - 1, dev), dev)
    pool = [wl.block_qkv(B, H, L, d, dt, wl.generator(wl.DECODE_B32_SEED + i, dev), dev) for i in range(16)]
    S = torch.zeros((B, H, 2 * F, d), device=dev)
    Z = torch.zeros((B, H, 2 * F), device=dev)
    out = torch.empty((B, H, L, d), device=dev)

    def block(n):
        for s_ in range(nsteps):
            q, k, v = pool[(n * nsteps + s_) % len(pool)]
            hba.step(q, k, v, W, S, Z, out=out)
        hba.commit(k, v, W, S, Z)

    def block_fused(n):   # the last step and the commit as one call
        for s_ in range(nsteps - 1):
            q, k, v = pool[(n * nsteps + s_) % len(pool)]
            hba.step(q, k, v, W, S, Z, out=out)
        q, k, v = pool[(n * nsteps + nsteps - 1) % len(pool)]
        hba.step_commit(q, k, v, W, S, Z, out=out)

    for n in range(2):
        block(n)
    S.zero_()
    Z.zero_()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for n in range(args.blocks):
        block(n)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)

    # the same loop with the last step of each block fused with its commit
    S.zero_()
    Z.zero_()
    for n in range(2):
        block_fused(n)
    S.zero_()
    Z.zero_()
    torch.cuda.synchronize()
    e0.record(stream)
    for n in range(args.blocks):
        block_fused(n)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_f = e0.elapsed_time(e1)
    final_eager = (S.clone(), Z.clone(), out.clone())

    # the fused loop replayed from a HIP graph of two blocks (the input pool
    # repeats every two blocks), starting from the same zero state.  The
    # state is cleared outside the graph.  Replays are checked against the
    # eager loop after 2 and 4 blocks (with eager work and synchronisation
    # between the replays) and after the full loop.
    def eager_from_zero(nblocks):
        S.zero_()
        Z.zero_()
        for n in range(nblocks):
            block_fused(n)
        torch.cuda.synchronize()
        return S.clone(), Z.clone(), out.clone()

    def same(a, b):
        return all(bool(torch.equal(x, y)) for x, y in zip(a, b))

    ref2, ref4 = eager_from_zero(2), eager_from_zero(4)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        block_fused(0)
        block_fused(1)
    S.zero_()
    Z.zero_()
    graph.replay()
    torch.cuda.synchronize()
    ok = same((S, Z, out), ref2)
    _ = float(out.abs().sum())   # eager work between replays
    graph.replay()
    torch.cuda.synchronize()
    ok = ok and same((S, Z, out), ref4)
    reps = args.blocks // 2
    S.zero_()
    Z.zero_()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_g = e0.elapsed_time(e1)
    ok = ok and (2 * reps != args.blocks or same((S, Z, out), final_eager))
    print(json.dumps({"mode": "decode_loop", "batch": B, "heads": H, "block": L, "steps_per_block": nsteps,
                      "blocks": args.blocks, "total_ms": ms, "us_per_block": ms * 1e3 / args.blocks,
                      "generated_tokens_per_s": B * L * args.blocks / (ms * 1e-3),
                      "query_tokens_per_s": B * L * nsteps * args.blocks / (ms * 1e-3),
                      "fused_last_step": {"us_per_block": ms_f * 1e3 / args.blocks,
                                          "generated_tokens_per_s": B * L * args.blocks / (ms_f * 1e-3)},
                      "fused_graph": {"blocks": 2 * reps, "us_per_block": ms_g * 1e3 / (2 * reps),
                                      "generated_tokens_per_s": B * L * 2 * reps / (ms_g * 1e-3),
                                      "matches_eager": ok}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--comparator", action="store_true",
                    help="time hba_prefix_softmax against hba_step at B=128 for P = 1k/4k/16k/32k")
    ap.add_argument("--batch", default="128",
                    help="comma-separated batch sizes for --comparator (e.g. 8,32,128)")
    ap.add_argument("--decode-loop", action="store_true",
                    help="time the B=32 decode loop (8 steps + 1 commit per 32-token block)")
    ap.add_argument("--blocks", type=int, default=256)
    ap.add_argument("--transfer", action="store_true",
                    help="time stage-1 attention transfer (loss, dW, dalpha) at 16 x 16 heads x 2048 tokens")
    ap.add_argument("--batch-sweep", action="store_true",
                    help="time hba_step over batch sizes (--batch, default 16..192) and fit fixed + marginal cost")
    ap.add_argument("--commit-sweep", action="store_true",
                    help="hba_commit of whole prefixes (8 x 2048 .. 128 x 2048 tokens)")
    ap.add_argument("--small-batch", action="store_true",
                    help="hba_step, one-block hba_commit and hba_step_commit at small batches "
                         "(--batch, default 1..32), each replayed from a HIP graph")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB read + 1 GiB write elementwise kernel (torch.neg) "
                         "10 times, to calibrate HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: the benchmark runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the step shards by request, with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_hybrid_attention_amd as hba
    from block_hybrid_attention_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        n = (1 << 30) // 4
        x = torch.ones(n, device=dev)
        y = torch.empty_like(x)
        for _ in range(10):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "torch.neg fp32", "read_bytes": 4 * n, "write_bytes": 4 * n,
                          "launches": 10}), flush=True)
        return
    if args.comparator:
        for B in (int(x) for x in args.batch.split(",")):
            comparator_sweep(args, torch, hba, wl, dev, B)
        return
    if args.decode_loop:
        return decode_loop(args, torch, hba, wl, dev)
    if args.transfer:
        return transfer_bench(args, torch, hba, wl, dev)
    if args.commit_sweep:
        return commit_sweep(args, torch, hba, wl, dev)
    if args.batch_sweep:
        return batch_sweep(args, torch, hba, wl, dev)
    if args.small_batch:
        return small_batch(args, torch, hba, wl, dev)
    c = wl.serving_b128()
    B, H, L, d, F = c.batch, c.heads, c.block, c.head_dim, c.feat
    plen = torch.tensor(c.prefix, dtype=torch.int32)
    Pmax = int(plen.max())
    g = wl.generator(c.seed, dev)
    W = wl.feature_weights(H, d, F, c.dtype, g, dev)

    sets = []
    keep_host = None
    # the prefixes are committed with hba_commit in one call per set (the
    # pipelined multi-chunk kernel); sets after the first are timed for
    # context, the first call of the process being excluded
    pre_ev = []
    for s in range(N_SETS):
        gs = wl.generator(c.seed * 1000 + s, dev)
        pk = wl.normal((B, H, Pmax, d), 1.0, c.dtype, gs, dev)
        pv = wl.normal((B, H, Pmax, d), 1.0, c.dtype, gs, dev)
        S = torch.zeros((B, H, 2 * F, d), device=dev)
        Z = torch.zeros((B, H, 2 * F), device=dev)
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        ev[0].record()
        hba.commit(pk, pv, W, S, Z, n_valid=plen.to(dev))
        ev[1].record()
        if s > 0:
            pre_ev.append(ev)
        q, k, v = wl.block_qkv(B, H, L, d, c.dtype, gs, dev)
        out = torch.empty((B, H, L, d), device=dev)
        if s == 0 and not args.no_cpu_baseline:
            n_req = 16
            keep_host = (pk[:n_req].cpu(), pv[:n_req].cpu())
        del pk, pv
        sets.append((q, k, v, S, Z, out))
    torch.cuda.synchronize()

    prefix_us = statistics.mean(a_.elapsed_time(b_) for a_, b_ in pre_ev) * 1e3 if pre_ev else None
    prefix_tokens = int(plen.sum())
    prefix_bytes = prefix_tokens * H * 2 * d * 2 + B * H * 2 * F * (d + 1) * 4 * 2

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        q, k, v, S, Z, out = sets[i % N_SETS]
        hba.step(q, k, v, W, S, Z, out=out)
    torch.cuda.synchronize()

    # timed region: K back-to-back steps on the launch stream, with a HIP
    # event between segments of at least 5 launches (at most 20 segments;
    # never an event between every launch: those packets would sit between
    # the kernels and add to every step).  The mean launch duration is
    # total / K; the spread is that of the segment means.
    nseg = max(1, min(20, args.steps // 5))
    bounds = [round(i * args.steps / nseg) for i in range(nseg + 1)]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(nseg + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for sgi in range(nseg):
        for i in range(bounds[sgi], bounds[sgi + 1]):
            q, k, v, S, Z, out = sets[i % N_SETS]
            hba.step(q, k, v, W, S, Z, out=out)
        marks[sgi + 1].record(stream)
    torch.cuda.synchronize()
    total_ms = marks[0].elapsed_time(marks[-1])
    ms_per_step = total_ms / args.steps
    mean_launch_ms = ms_per_step
    seg_ms = [marks[i].elapsed_time(marks[i + 1]) / (bounds[i + 1] - bounds[i])
              for i in range(nseg) if bounds[i + 1] > bounds[i]]
    if len(seg_ms) >= 2:
        dec = statistics.quantiles(seg_ms, n=10)
        q10, q50, q90 = dec[0], statistics.median(seg_ms), dec[-1]
    else:
        q10 = q50 = q90 = ms_per_step

    nbytes = step_bytes(B, H, L, d, F)
    achieved = nbytes / (mean_launch_ms * 1e-3) / 1e9
    khash = step_source_hash()
    traffic = load_traffic(khash)

    # one block commit (32 tokens) for context: state read-modify-write,
    # rotating over the state sets (the step timing above is done, so the
    # commits may change them) so that the Infinity Cache holds none of them
    rot = [0]

    def commit_next():
        q_, k_, v_, S_, Z_, _ = sets[rot[0] % N_SETS]
        rot[0] += 1
        hba.commit(k_, v_, W, S_, Z_)

    commit_us = _time_launches(torch, commit_next, 4, 20, stream) * 1e3
    cbytes = commit_bytes(B, H, L, d, F)

    # the fused last step + commit (hba_step_commit) at the same shape, rotating likewise
    def step_commit_next():
        q_, k_, v_, S_, Z_, o_ = sets[rot[0] % N_SETS]
        rot[0] += 1
        hba.step_commit(q_, k_, v_, W, S_, Z_, out=o_)

    sc_ms = _time_launches(torch, step_commit_next, 4, 20, stream)
    sc_bytes = step_bytes(B, H, L, d, F) + B * H * 2 * F * (d + 1) * 4
    q, k, v, S, Z, out = sets[0]

    # the standalone feature map (hba_feature_map) of the step's B*L query
    # rows for all heads: x [B*L][H][d] bf16 -> phi [B*L][H][2F] fp32
    xq = q.permute(0, 2, 1, 3).reshape(B * L, H, d).contiguous()
    phi = torch.empty((B * L, H, 2 * F), device=dev)
    fm_ms = _time_launches(torch, lambda: hba.feature_map(xq, W, out=phi), 3, 20, stream)
    fm_bytes = B * L * H * d * 2 + H * d * F * 2 + B * L * H * 2 * F * 4
    del xq, phi

    # the B = 8 workload (a 2048-token prefix committed in one call, then the
    # step): the pipelined commit, and the step replayed from a HIP graph of
    # 20 launches, which takes the host out of a launch this short
    B8, T8 = 8, 2048
    g8 = wl.generator(c.seed * 1000 + 99, dev)
    k8p = wl.normal((B8, H, T8, d), 1.0, c.dtype, g8, dev)
    v8p = wl.normal((B8, H, T8, d), 1.0, c.dtype, g8, dev)
    S8 = torch.zeros((B8, H, 2 * F, d), device=dev)
    Z8 = torch.zeros((B8, H, 2 * F), device=dev)
    c8_ms = _time_launches(torch, lambda: hba.commit(k8p, v8p, W, S8, Z8), 2, 10, stream)
    q8, k8, v8 = wl.block_qkv(B8, H, L, d, c.dtype, g8, dev)
    o8 = torch.empty((B8, H, L, d), device=dev)
    s8_us = _time_graph(torch, lambda: hba.step(q8, k8, v8, W, S8, Z8, out=o8), 20, 5, stream) * 1e3
    del k8p, v8p

    base = None
    if not args.no_cpu_baseline:
        q0, k0, v0 = sets[0][0], sets[0][1], sets[0][2]
        base = cpu_baseline(wl, W, keep_host[0], keep_host[1], plen, q0, k0, v0, 16, args.cpu_seconds)

    tokens = B * L
    line = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in; split-bf16 MFMA; fp32 accumulate and state",
        "data": "synthetic",
        "config": {"workload": "serving_b128: 128 requests x 16 heads, d=128, F=128 (phi 256), block 32, "
                               "prefix 32*U{16..128} tokens committed with hba_commit; one hba_step",
                   "batch": B, "heads": H, "block": L, "head_dim": d, "feat": F,
                   "inputs": "bf16 q/k/v/W", "state": "fp32 S,Z", "accumulate": "fp32",
                   "rotating_sets": N_SETS, "hbm_pct": 100.0 * achieved / HBM_PEAK_GBS},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": "hba_step (step_kernel<bf16,128,128>)",
                     "algorithmic_bytes_per_launch": nbytes,
                     "launch_ms": {"mean": mean_launch_ms, "p10": q10, "median": q50, "p90": q90,
                                   "timing": (f"{args.steps} back-to-back launches on the launch stream, HIP "
                                              f"events between {len(seg_ms)} segments; p10/median/p90 "
                                              "of the segment means")},
                     "source_hash": khash},
        "cpu_baseline": base,
        "components": {"commit_block_us": commit_us,
                       "commit_block_GBps": cbytes / (commit_us * 1e-6) / 1e9,
                       "commit_algorithmic_bytes": cbytes,
                       "step_commit_us": sc_ms * 1e3,
                       "step_commit_GBps": sc_bytes / (sc_ms * 1e-3) / 1e9,
                       "step_commit_algorithmic_bytes": sc_bytes,
                       "feature_map_us": fm_ms * 1e3,
                       "feature_map_GBps": fm_bytes / (fm_ms * 1e-3) / 1e9,
                       "feature_map_algorithmic_bytes": fm_bytes,
                       "prefix_commit_us": prefix_us,
                       "prefix_commit_tokens": prefix_tokens,
                       "prefix_commit_M_tokens_per_s": (prefix_tokens / (prefix_us * 1e-6) / 1e6
                                                        if prefix_us else None),
                       "prefix_commit_GBps": prefix_bytes / (prefix_us * 1e-6) / 1e9 if prefix_us else None,
                       "prefix_commit_algorithmic_bytes": prefix_bytes,
                       "b8_prefix_commit_us": c8_ms * 1e3,
                       "b8_prefix_commit_tokens": B8 * T8,
                       "b8_step_us_graph": s8_us},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
