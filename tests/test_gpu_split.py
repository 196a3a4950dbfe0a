"""The comparator with its keys split over several workgroups per (request,
head): hba_prefix_softmax_split against the fp64 oracle, including splits
that receive no keys (short prefixes, many splits) and grouped key/value
heads, and against the unsplit call at a small-batch, long-prefix shape."""
import pytest
import torch

import block_hybrid_attention_amd as hba
import oracle
from block_hybrid_attention_amd import workloads as wl
from parity import check, report, row_rel

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _library():
    hba.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_split", [2, 3, 7, 64])
def test_split_comparator_matches_oracle(dtype, d, n_split):
    g = wl.generator(9950 + d + n_split + (dtype == torch.bfloat16), DEV)
    B, H, Hkv, L, P = 4, 4, 2, 32, 700
    q = wl.normal((B, H, L, d), 1, dtype, g, DEV)
    k, v = (wl.normal((B, Hkv, L, d), 1, dtype, g, DEV) for _ in range(2))
    Kc, Vc = (wl.normal((B, Hkv, P, d), 1, dtype, g, DEV) for _ in range(2))
    # 0: the block's own keys only (most splits empty); 33: one tile plus a tail
    plen = torch.tensor([P, 0, 33, 517], dtype=torch.int32, device=DEV)
    out = hba.prefix_softmax(q, k, v, Kc, Vc, prefix_len=plen, n_split=n_split)
    ref = oracle.prefix_softmax(q, k, v, Kc, Vc, prefix_len=plen)
    err = row_rel(out, ref)
    report(f"split comparator {dtype} d={d} n_split={n_split}", out=err)
    check(dict(out=err), dtype)


@pytest.mark.parametrize("L", [1, 7])
def test_split_comparator_short_blocks(L):
    g = wl.generator(9990 + L, DEV)
    B, H, d, P = 2, 3, 128, 300
    dtype = torch.bfloat16
    q, k, v = wl.block_qkv(B, H, L, d, dtype, g, DEV)
    Kc, Vc = (wl.normal((B, H, P, d), 1, dtype, g, DEV) for _ in range(2))
    out = hba.prefix_softmax(q, k, v, Kc, Vc, n_split=5)
    ref = oracle.prefix_softmax(q, k, v, Kc, Vc)
    err = row_rel(out, ref)
    report(f"split comparator L={L}", out=err)
    check(dict(out=err), dtype)


def test_split_comparator_small_batch_long_prefix():
    """8 requests x 16 heads with an 8k-token cache, the library's own split
    choice: agrees with the unsplit kernel, and sampled pairs with the oracle."""
    g = wl.generator(9999, DEV)
    B, H, L, d, P = 8, 16, 32, 128, 8192
    dtype = torch.bfloat16
    q, k, v = wl.block_qkv(B, H, L, d, dtype, g, DEV)
    Kc, Vc = (wl.normal((B, H, P, d), 1, dtype, g, DEV) for _ in range(2))
    ns = hba.prefix_softmax_auto_split(B, H, L, d, P)
    assert ns > 1
    out = hba.prefix_softmax(q, k, v, Kc, Vc, n_split=None)
    one = hba.prefix_softmax(q, k, v, Kc, Vc, n_split=1)
    agree = row_rel(out, one)
    idx = [0, 5]
    ref = oracle.prefix_softmax(q[idx], k[idx], v[idx], Kc[idx], Vc[idx])
    err = row_rel(out[idx], ref)
    report(f"split comparator B=8 P=8192 auto n_split={ns}", vs_unsplit=agree, out=err)
    check(dict(vs_unsplit=agree, out=err), dtype)


def test_split_workspace_reuse_and_size_check():
    g = wl.generator(9998, DEV)
    B, H, L, d, P = 2, 2, 32, 64, 400
    dtype = torch.bfloat16
    q, k, v = wl.block_qkv(B, H, L, d, dtype, g, DEV)
    Kc, Vc = (wl.normal((B, H, P, d), 1, dtype, g, DEV) for _ in range(2))
    need = hba.prefix_softmax_workspace_bytes(B, H, L, d, 4)
    ws = torch.full(((need + 3) // 4,), float("nan"), device=DEV)   # contents on entry do not matter
    a = hba.prefix_softmax(q, k, v, Kc, Vc, n_split=4, workspace=ws)
    b = hba.prefix_softmax(q, k, v, Kc, Vc, n_split=4, workspace=ws)
    assert torch.equal(a, b)
    with pytest.raises(ValueError, match="workspace"):
        hba.prefix_softmax(q, k, v, Kc, Vc, n_split=4, workspace=ws[:-1])
