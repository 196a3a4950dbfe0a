"""hba_prefix_softmax_split_noalloc: the split comparator with its partials
in the library's fixed per-device scratch array instead of a caller
workspace.  Through the C ABI, two calls in a row (the second smaller, with
ragged prefixes and another split count) must equal hba_prefix_softmax_split
with a caller workspace, and meet the oracle on sampled pairs; a shape whose
partials exceed the array is refused on the host."""
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


def _inputs(seed, B, H, L, d, P):
    g = wl.generator(seed, DEV)
    dt = torch.bfloat16
    q, k, v = wl.block_qkv(B, H, L, d, dt, g, DEV)
    Kc, Vc = wl.normal((B, H, P, d), 1, dt, g, DEV), wl.normal((B, H, P, d), 1, dt, g, DEV)
    return q, k, v, Kc, Vc


def test_noalloc_matches_workspace_call_twice():
    dt = torch.bfloat16
    # first call: the small-batch comparator shape, the library's split choice
    B, H, L, d, P = 8, 16, 32, 128, 8192
    q, k, v, Kc, Vc = _inputs(9900, B, H, L, d, P)
    ns = hba.prefix_softmax_auto_split(B, H, L, d, P)
    assert ns > 1 and hba.prefix_softmax_workspace_bytes(B, H, L, d, ns) <= hba.NOALLOC_SCRATCH_BYTES
    out = torch.empty((B, H, L, d), device=DEV)
    hba.prefix_softmax_noalloc(q, k, v, Kc, Vc, out, n_split=ns)
    ref = hba.prefix_softmax(q, k, v, Kc, Vc, n_split=ns)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    idx = torch.tensor([0, 5], device=DEV)
    hs = torch.tensor([0, 7, 15], device=DEV)
    sel = lambda t: t[idx][:, hs]  # noqa: E731
    err1 = row_rel(sel(out), oracle.prefix_softmax(sel(q), sel(k), sel(v), sel(Kc), sel(Vc)))
    # second call, smaller: fewer requests, ragged prefixes, more splits
    B2, L2, P2 = 2, 17, 3000
    q2, k2, v2, Kc2, Vc2 = _inputs(9901, B2, H, L2, d, P2)
    plen = torch.tensor([3000, 1234], dtype=torch.int32, device=DEV)
    out2 = torch.empty((B2, H, L2, d), device=DEV)
    hba.prefix_softmax_noalloc(q2, k2, v2, Kc2, Vc2, out2, n_split=8, prefix_len=plen)
    ref2 = hba.prefix_softmax(q2, k2, v2, Kc2, Vc2, prefix_len=plen, n_split=8)
    torch.cuda.synchronize()
    assert torch.equal(out2, ref2)
    err2 = row_rel(out2, oracle.prefix_softmax(q2, k2, v2, Kc2, Vc2, prefix_len=plen))
    report("comparator no-alloc, two calls", first=err1, second=err2)
    check(dict(first=err1, second=err2), dt)


def test_noalloc_refuses_oversized_partials():
    """Partials beyond the array: HBA_ERR_CAPACITY, checked on the host before
    any launch (the output stays untouched)."""
    B, H, L, d, P = 64, 16, 32, 128, 64
    q, k, v, Kc, Vc = _inputs(9902, B, H, L, d, P)
    assert hba.prefix_softmax_workspace_bytes(B, H, L, d, 16) > hba.NOALLOC_SCRATCH_BYTES
    out = torch.full((B, H, L, d), 7.0, device=DEV)
    with pytest.raises(hba.HbaError) as exc:
        hba.prefix_softmax_noalloc(q, k, v, Kc, Vc, out, n_split=16)
    assert exc.value.status == 6
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
