"""hba_transfer (stage-1 attention transfer: loss and gradients for W and
alpha) against the fp64 oracle on the same seeded inputs.

Measures: the loss and each head's dW by relative error (Frobenius norm for
dW), dalpha by its error relative to the norm of the dalpha vector, the
layer output by the usual per-row relative error.  fp32 inputs run on fp32
matrix cores; bf16 inputs on bf16 matrix cores with fp32 operands split into
high and residual parts and fp32 accumulation.  The forward values meet the
fp32 bar for both, the gradients the bar of their input dtype."""
import numpy as np
import pytest
import torch

import block_hybrid_attention_amd as hba
import oracle
from block_hybrid_attention_amd import workloads as wl
from parity import DESIGN_TOL, TOL, host64, report, row_rel

pytestmark = pytest.mark.gpu
DEV = "cuda"
GRAD_TOL = {torch.float32: 1e-5, torch.bfloat16: 3e-3}


def check_grads(e, dtype):
    """Gradients within their dtype's bar and the split-bf16 design guard."""
    for name in ("dW", "dalpha"):
        assert e[name] <= GRAD_TOL[dtype] and e[name] <= DESIGN_TOL[dtype], (name, e[name])


@pytest.fixture(scope="module", autouse=True)
def _library():
    hba.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def make(seed, B, H, Hkv, nb, L, F, dtype):
    g = wl.generator(seed, DEV)
    d, N = 128, nb * L
    q = wl.normal((B, H, N, d), 1, dtype, g, DEV)
    k = wl.normal((B, Hkv, N, d), 1, dtype, g, DEV)
    v = wl.normal((B, Hkv, N, d), 1, dtype, g, DEV)
    W = wl.feature_weights(H, d, F, dtype, g, DEV)
    alpha = torch.randn(H, generator=g, device=DEV)
    target = 0.3 * torch.randn((B, H, N, d), generator=g, device=DEV)
    return q, k, v, W, alpha, target


def errors(got, ref):
    loss, dW, da, out = got
    rl, rout, rdW, rda = ref[1], ref[0], ref[2], ref[3]
    e = dict(loss=abs(float(loss[0]) - rl) / rl,
             dW=max(float(np.linalg.norm(host64(dW[h]) - rdW[h]) / np.linalg.norm(rdW[h])) for h in range(len(rdW))),
             dalpha=float(np.linalg.norm(host64(da) - rda) / np.linalg.norm(rda)))
    if out is not None:
        e["out"] = row_rel(out, rout)
    return e


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("F", [128, 64])
@pytest.mark.parametrize("L,nb,Hkv", [(32, 4, 2), (7, 5, 1), (32, 1, 2), (19, 3, 2), (16, 3, 1), (8, 4, 2),
                                      (1, 9, 2)])
def test_transfer_matches_oracle(dtype, F, L, nb, Hkv):
    B, H = 2, 2
    q, k, v, W, alpha, target = make(9700 + F + L + nb + (dtype == torch.bfloat16), B, H, Hkv, nb, L, F, dtype)
    out = torch.empty((B, H, nb * L, 128), device=DEV)
    got = hba.transfer(q, k, v, W, alpha, target, L, out=out)
    ref = oracle.transfer(q, k, v, W, alpha, target, L)
    if nb == 1:
        # one block: no committed context, so both gradients are exactly zero (up to rounding)
        assert float(got[1].abs().max()) <= 1e-5 * float(got[0][0]) and float(got[2].abs().max()) <= 1e-5 * float(got[0][0])
        e = dict(loss=abs(float(got[0][0]) - ref[1]) / ref[1], out=row_rel(out, ref[0]))
        report(f"transfer {dtype} F={F} L={L} nb=1", **e)
        assert all(x <= TOL[dtype] for x in e.values())
        return
    e = errors(got, ref)
    report(f"transfer {dtype} F={F} L={L} nb={nb} Hkv={Hkv}", **e)
    assert e["loss"] <= TOL[torch.float32] and e["out"] <= TOL[torch.float32]
    check_grads(e, dtype)


def test_transfer_deterministic_and_empty():
    B, H, L, nb, F = 2, 4, 32, 3, 128
    q, k, v, W, alpha, target = make(9750, B, H, 4, nb, L, F, torch.bfloat16)
    a = hba.transfer(q, k, v, W, alpha, target, L)
    b = hba.transfer(q, k, v, W, alpha, target, L)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    z = hba.transfer(q[:, :, :0], k[:, :, :0], v[:, :, :0], W, alpha, target[:, :, :0], L)
    assert float(z[0][0]) == 0.0 and not z[1].any() and not z[2].any()


def test_transfer_medium_bf16():
    """4 requests x 8 heads over 2 key/value heads, 16 blocks of 32 tokens."""
    B, H, Hkv, L, nb, F = 4, 8, 2, 32, 16, 128
    q, k, v, W, alpha, target = make(9760, B, H, Hkv, nb, L, F, torch.bfloat16)
    got = hba.transfer(q, k, v, W, alpha, target, L)
    ref = oracle.transfer(q, k, v, W, alpha, target, L)
    e = errors(got, ref)
    report("transfer medium bf16", **e)
    assert e["loss"] <= TOL[torch.float32]
    check_grads(e, torch.bfloat16)


def test_transfer_bench_size_bf16():
    """The launch bench.py --transfer times: 16 requests x 16 heads x 2048
    tokens (64 blocks of 32), d = F = 128, bf16.  The layer output of a
    sampled request from that launch against the oracle, element by element;
    that request's loss and gradients (a one-request launch) against the
    oracle; and the full-batch gradients against the ordered sum of the 16
    one-request launches (the gradient is a sum over requests)."""
    B, H, L, nb, F = 16, 16, 32, 64, 128
    q, k, v, W, alpha, target = make(9800, B, H, H, nb, L, F, torch.bfloat16)
    out = torch.empty((B, H, nb * L, 128), device=DEV)
    full = hba.transfer(q, k, v, W, alpha, target, L, out=out)
    b = 11
    one = [hba.transfer(q[i:i + 1], k[i:i + 1], v[i:i + 1], W, alpha, target[i:i + 1], L) for i in range(B)]
    ref = oracle.transfer(q[b:b + 1], k[b:b + 1], v[b:b + 1], W, alpha, target[b:b + 1], L)
    e = errors(one[b], ref)
    e["out"] = row_rel(out[b:b + 1], ref[0])
    report("transfer bench size bf16 (request 11)", **e)
    assert e["loss"] <= TOL[torch.float32] and e["out"] <= TOL[torch.float32]
    check_grads(e, torch.bfloat16)
    # a sum over requests: the full launch equals the sum of the one-request launches
    sl = sum(float(o[0][0]) for o in one)
    sdW = sum(host64(o[1]) for o in one)
    sda = sum(host64(o[2]) for o in one)
    assert abs(float(full[0][0]) - sl) <= 1e-6 * sl
    assert np.linalg.norm(host64(full[1]) - sdW) <= 1e-6 * np.linalg.norm(sdW)
    assert np.linalg.norm(host64(full[2]) - sda) <= 1e-6 * np.linalg.norm(sda)
