"""Pins of the oracle's stage-1 attention transfer (loss and gradients with
respect to W and alpha; "Retrofitting Linear Attention into Diffusion
Language Models", section 3.2, over the layer of section 3.1).

None of these compares the oracle with itself:
  - the output is brute force over raw tokens (block softmax weights
    w exp(q.k/sqrt d) inside the block, the Eq. 1 kernel phi(q).phi(k) on
    every token of an earlier block, one shared normaliser) with no state;
  - the gradients are torch autograd (fp64) through that brute force;
  - central finite differences of the loss, and closed forms (a single
    block has no linear branch, so both gradients vanish; a target equal
    to the output gives zero loss and zero gradients).
CPU only.
"""
import numpy as np
import pytest
import torch

import oracle


def case(rng, B, H, Hkv, nb, L, d, F):
    N = nb * L
    q = rng.normal(0, 1, (B, H, N, d))
    k, v = (rng.normal(0, 1, (B, Hkv, N, d)) for _ in range(2))
    W = rng.normal(0, d ** -0.5, (H, d, F))
    alpha = rng.normal(0, 1, H)
    t = rng.normal(0, 0.3, (B, H, N, d))
    return q, k, v, W, alpha, t


def brute(q, k, v, W, alpha, t, L):
    """Loss of the block-hybrid layer written over raw tokens, in torch fp64
    (autograd-capable: W and alpha may require grad)."""
    q, k, v, t = (torch.as_tensor(x, dtype=torch.float64) for x in (q, k, v, t))
    B, H, N, d = q.shape
    G = H // k.shape[1]
    kk, vv = k.repeat_interleave(G, 1), v.repeat_interleave(G, 1)

    def phi(x):
        u = torch.matmul(x, W[None])                         # [B][H][N][F]
        return torch.cat([torch.softmax(u, -1), torch.softmax(-u, -1)], -1)

    blk = torch.arange(N) // L
    same = (blk[:, None] == blk[None, :]).double()
    earlier = (blk[None, :] < blk[:, None]).double()
    w = torch.sigmoid(alpha)[None, :, None, None]
    a = torch.exp(torch.matmul(q, kk.transpose(-1, -2)) / d ** 0.5) * same
    kap = torch.matmul(phi(q), phi(kk).transpose(-1, -2)) * earlier
    wt = w * a + kap
    o = torch.matmul(wt, vv) / wt.sum(-1, keepdim=True)
    return ((o - t) ** 2).sum(), o


def autograd(q, k, v, W, alpha, t, L):
    Wt = torch.tensor(W, requires_grad=True)
    at = torch.tensor(alpha, requires_grad=True)
    loss, o = brute(q, k, v, Wt, at, t, L)
    loss.backward()
    return float(loss.detach()), o.detach().numpy(), Wt.grad.numpy(), at.grad.numpy()


@pytest.mark.parametrize("B,H,Hkv,nb,L,d,F", [(2, 2, 2, 4, 4, 8, 4), (1, 4, 2, 3, 8, 16, 8), (2, 3, 1, 5, 3, 8, 8)])
def test_transfer_matches_brute_force_and_autograd(B, H, Hkv, nb, L, d, F):
    rng = np.random.default_rng(60 + nb + L)
    q, k, v, W, alpha, t = case(rng, B, H, Hkv, nb, L, d, F)
    out, loss, dW, da = oracle.transfer(q, k, v, W, alpha, t, L)
    ref_loss, ref_out, ref_dW, ref_da = autograd(q, k, v, W, alpha, t, L)
    np.testing.assert_allclose(out, ref_out, rtol=1e-11, atol=1e-12)
    assert abs(loss - ref_loss) <= 1e-11 * ref_loss
    np.testing.assert_allclose(dW, ref_dW, rtol=1e-9, atol=1e-11 * np.abs(ref_dW).max())
    np.testing.assert_allclose(da, ref_da, rtol=1e-9, atol=1e-12)


def test_transfer_finite_differences():
    rng = np.random.default_rng(70)
    L = 4
    q, k, v, W, alpha, t = case(rng, 1, 2, 2, 3, L, 8, 4)
    _, _, dW, da = oracle.transfer(q, k, v, W, alpha, t, L)
    eps = 1e-6
    for (h, r, f) in [(0, 0, 0), (1, 3, 2), (0, 7, 3)]:
        Wp, Wm = W.copy(), W.copy()
        Wp[h, r, f] += eps
        Wm[h, r, f] -= eps
        fd = (oracle.transfer(q, k, v, Wp, alpha, t, L)[1] - oracle.transfer(q, k, v, Wm, alpha, t, L)[1]) / (2 * eps)
        assert abs(fd - dW[h, r, f]) <= 1e-6 * max(1.0, abs(fd))
    for h in range(2):
        ap, am = alpha.copy(), alpha.copy()
        ap[h] += eps
        am[h] -= eps
        fd = (oracle.transfer(q, k, v, W, ap, t, L)[1] - oracle.transfer(q, k, v, W, am, t, L)[1]) / (2 * eps)
        assert abs(fd - da[h]) <= 1e-6 * max(1.0, abs(fd))


def test_transfer_single_block_has_no_gradient():
    # one block: no committed context, o is block softmax whatever W and w are
    rng = np.random.default_rng(71)
    L = 8
    q, k, v, W, alpha, t = case(rng, 2, 2, 2, 1, L, 8, 4)
    out, loss, dW, da = oracle.transfer(q, k, v, W, alpha, t, L)
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(out, sdpa, rtol=1e-12, atol=1e-13)
    assert abs(loss - ((sdpa - t) ** 2).sum()) <= 1e-12 * loss
    assert np.abs(dW).max() <= 1e-12 and np.abs(da).max() <= 1e-12


def test_transfer_target_equal_to_output_is_stationary():
    rng = np.random.default_rng(72)
    L = 4
    q, k, v, W, alpha, t = case(rng, 1, 2, 1, 4, L, 8, 4)
    out, _, _, _ = oracle.transfer(q, k, v, W, alpha, t, L)
    _, loss, dW, da = oracle.transfer(q, k, v, W, alpha, out, L)
    assert loss <= 1e-25
    assert np.abs(dW).max() <= 1e-12 and np.abs(da).max() <= 1e-12


def test_transfer_request_order_and_head_split():
    # the per-head gradient is the sum of per-request gradients
    rng = np.random.default_rng(73)
    L = 4
    q, k, v, W, alpha, t = case(rng, 3, 2, 2, 3, L, 8, 4)
    _, loss, dW, da = oracle.transfer(q, k, v, W, alpha, t, L)
    parts = [oracle.transfer(q[b:b + 1], k[b:b + 1], v[b:b + 1], W, alpha, t[b:b + 1], L) for b in range(3)]
    assert abs(loss - sum(p[1] for p in parts)) <= 1e-12 * loss
    np.testing.assert_allclose(dW, sum(p[2] for p in parts), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(da, sum(p[3] for p in parts), rtol=1e-12, atol=1e-14)
