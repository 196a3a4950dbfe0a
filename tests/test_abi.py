"""The C ABI: the library loads, exports every call the header declares, and
rejects bad arguments on the host before anything reaches a GPU.

Every call here is built so that host validation fails (or the call is an
explicit no-op), so nothing is ever launched -- the fake pointers below are
never dereferenced.  Calls with fake pointers are skipped when a GPU is
present, as a second guard.
"""
import ctypes
import os
import re

import pytest
import torch

import block_hybrid_attention_amd as hba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hba.h")
OK, ENULL, ESHAPE, EUNSUP, EDTYPE, EALIGN, ECAP = 0, 1, 2, 3, 4, 5, 6
no_gpu_only = pytest.mark.skipif(torch.cuda.is_available(),
                                 reason="fake-pointer validation tests run only without a GPU")


def lib():
    if not os.path.exists(hba.library_path()):
        import block_hybrid_attention_amd.build as b
        b.build()
    return hba.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:hba_status|const char \*|int32_t|int64_t)\s*\**\s*(hba_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"hba_feature_map", "hba_step", "hba_commit", "hba_prefix_softmax", "hba_step_commit",
            "hba_prefix_softmax_split", "hba_prefix_softmax_auto_split", "hba_prefix_softmax_workspace_bytes",
            "hba_transfer", "hba_transfer_workspace_bytes", "hba_prefix_softmax_split_noalloc",
            "hba_status_string", "hba_abi_version"} <= set(names)
    L = lib()
    for n in names:
        assert hasattr(L, n), n
    assert hba.abi_version() == 6


def test_status_strings():
    L = lib()
    for code in range(8):
        s = L.hba_status_string(code)
        assert s and s != b"unknown status"
    assert L.hba_status_string(99) == b"unknown status"


def shape(batch=2, heads=4, block=32, d=128, F=128, dtype=1, slots=8, kv_heads=0):
    return hba.Shape(batch, heads, block, d, F, dtype, slots, kv_heads)


A = ctypes.c_void_p(0x10000)      # aligned, never dereferenced
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10004)    # 4-byte aligned only


def step_call(sh, q=A, k=A, v=A, W=A, gate=None, S=A2, Z=A2, slot=None, out=A2):
    return lib().hba_step(ctypes.byref(sh) if sh is not None else None, q, k, v, W, gate, S, Z, slot, out, None)


@no_gpu_only
def test_step_validation():
    assert step_call(None) == ENULL
    assert step_call(shape(dtype=7)) == EDTYPE
    assert step_call(shape(d=96)) == EUNSUP
    assert step_call(shape(F=32)) == EUNSUP
    assert step_call(shape(block=0)) == ESHAPE
    assert step_call(shape(block=33)) == EUNSUP
    assert step_call(shape(heads=0)) == ESHAPE
    assert step_call(shape(batch=-1)) == ESHAPE
    assert step_call(shape(slots=-1)) == ESHAPE
    assert step_call(shape(), q=None) == ENULL
    assert step_call(shape(), S=None) == ENULL
    assert step_call(shape(batch=9, slots=8)) == ECAP         # no slot map, too many requests
    assert step_call(shape(), k=MIS) == EALIGN
    assert step_call(shape(), out=MIS) == EALIGN
    assert step_call(shape(), gate=ctypes.c_void_p(0x10001), slot=A) == EALIGN


def test_zero_batch_is_a_noop():
    # batch == 0 returns before touching any pointer, on any machine
    assert step_call(shape(batch=0), q=None, k=None, v=None, W=None, S=None, Z=None, out=None) == OK
    L = lib()
    sh = shape(batch=0)
    assert L.hba_commit(ctypes.byref(sh), 32, None, None, None, None, None, None, None, None) == OK
    assert L.hba_prefix_softmax(ctypes.byref(sh), 64, None, None, None, None, None, None, None, None) == OK
    assert L.hba_feature_map(ctypes.byref(shape()), 0, None, None, None, None) == OK


@no_gpu_only
def test_step_commit_validation():
    L = lib()

    def call(sh, q=A, k=A, v=A, W=A, gate=None, S=A2, Z=A2, slot=None, out=A2, n_valid=None):
        return L.hba_step_commit(ctypes.byref(sh) if sh is not None else None, n_valid, q, k, v, W, gate,
                                 S, Z, slot, out, None)

    assert call(None) == ENULL
    assert call(shape(dtype=3)) == EDTYPE
    assert call(shape(d=96)) == EUNSUP
    assert call(shape(block=0)) == ESHAPE
    assert call(shape(block=40)) == EUNSUP
    assert call(shape(), v=None) == ENULL
    assert call(shape(), Z=None) == ENULL
    assert call(shape(batch=9, slots=8)) == ECAP
    assert call(shape(), S=MIS) == EALIGN
    assert call(shape(), n_valid=ctypes.c_void_p(0x10002), slot=A) == EALIGN
    assert call(shape(batch=0), q=None, k=None, v=None, W=None, S=None, Z=None, out=None) == OK


@no_gpu_only
def test_commit_validation():
    L = lib()

    def call(sh, n_tok=32, k=A, v=A, W=A, S=A2, Z=A2, n_valid=None, slot=None):
        return L.hba_commit(ctypes.byref(sh), n_tok, n_valid, k, v, W, S, Z, slot, None)

    assert call(shape(), n_tok=-1) == ESHAPE
    assert call(shape(), n_tok=0, k=None) == OK               # nothing to fold
    assert call(shape(d=32)) == EUNSUP
    assert call(shape(), v=None) == ENULL
    assert call(shape(batch=9, slots=8)) == ECAP
    assert call(shape(), Z=MIS) == EALIGN
    assert call(shape(), n_valid=ctypes.c_void_p(0x10002), slot=A) == EALIGN


@no_gpu_only
def test_prefix_and_feature_map_validation():
    L = lib()

    def pcall(sh, P=128, Kc=A, Vc=A, out=A2):
        return L.hba_prefix_softmax(ctypes.byref(sh), P, None, A, A, A, Kc, Vc, out, None)

    assert pcall(shape(), P=-1) == ESHAPE
    assert pcall(shape(), Kc=None) == ENULL
    assert pcall(shape(block=40)) == EUNSUP
    assert pcall(shape(), Vc=MIS) == EALIGN
    sh = shape()
    assert L.hba_feature_map(ctypes.byref(sh), -1, A, A, A2, None) == ESHAPE
    assert L.hba_feature_map(ctypes.byref(sh), 1 << 31, A, A, A2, None) == ESHAPE
    assert L.hba_feature_map(ctypes.byref(sh), 10, None, A, A2, None) == ENULL
    assert L.hba_feature_map(ctypes.byref(shape(F=96)), 10, A, A, A2, None) == EUNSUP
    assert L.hba_feature_map(ctypes.byref(sh), 10, A, MIS, A2, None) == EALIGN


@no_gpu_only
def test_kv_heads_validation():
    # kv_heads must divide heads (0 means heads); checked before any pointer
    L = lib()
    for bad in (-1, 3, 8):
        sh = shape(heads=4, kv_heads=bad)
        assert step_call(sh) == ESHAPE
        assert L.hba_commit(ctypes.byref(sh), 32, None, A, A, A, A2, A2, None, None) == ESHAPE
        assert L.hba_step_commit(ctypes.byref(sh), None, A, A, A, A, None, A2, A2, None, A2, None) == ESHAPE
        assert L.hba_prefix_softmax(ctypes.byref(sh), 64, None, A, A, A, A, A, A2, None) == ESHAPE
    # the feature map has no key/value heads and ignores the field
    assert L.hba_feature_map(ctypes.byref(shape(kv_heads=3)), 0, None, None, None, None) == OK
    for good in (1, 2, 4):
        assert step_call(shape(batch=0, heads=4, kv_heads=good), q=None) == OK


def test_python_binding_refuses_uneven_head_groups():
    lib()
    q = torch.zeros(1, 4, 8, 64)
    k = torch.zeros(1, 3, 8, 64)
    with pytest.raises(ValueError, match="key/value heads"):
        hba.step(q, k, k, torch.zeros(4, 64, 64), torch.zeros(1, 4, 128, 64), torch.zeros(1, 4, 128))


@no_gpu_only
def test_split_comparator_validation():
    L = lib()

    def call(sh, P=128, ns=4, ws=A2, wsb=1 << 30, Kc=A, out=A2):
        return L.hba_prefix_softmax_split(ctypes.byref(sh), P, ns, None, A, A, A, Kc, A, ws, wsb, out, None)

    sh = shape()
    need = L.hba_prefix_softmax_workspace_bytes(ctypes.byref(sh), 4)
    assert need == 4 * 2 * 4 * 4 * 32 * (128 + 2)
    assert L.hba_prefix_softmax_workspace_bytes(ctypes.byref(sh), 1) == 0
    assert L.hba_prefix_softmax_workspace_bytes(ctypes.byref(sh), 0) == -1
    assert L.hba_prefix_softmax_workspace_bytes(ctypes.byref(sh), 65) == -1
    assert call(sh, ns=0) == ESHAPE
    assert call(sh, ns=65) == ESHAPE
    assert call(sh, ws=None) == ENULL
    assert call(sh, wsb=need - 1) == ECAP
    assert call(sh, ws=MIS) == EALIGN
    assert call(sh, Kc=None) == ENULL
    assert call(shape(kv_heads=3)) == ESHAPE
    assert call(shape(batch=0), ws=None) == OK
    # without a device the choice falls back to one split; bad shapes give 1 too
    assert L.hba_prefix_softmax_auto_split(ctypes.byref(sh), 1 << 15) == 1
    assert L.hba_prefix_softmax_auto_split(None, 128) == 1


@no_gpu_only
def test_noalloc_comparator_validation():
    """The allocation-free comparator: host checks as the split comparator's,
    partials beyond the library's scratch array refused with
    HBA_ERR_CAPACITY before any device call; with no device, a call that
    passes every host check fails with HBA_ERR_HIP and launches nothing."""
    L = lib()
    EHIP = 7

    def call(sh, P=128, ns=4, Kc=A, out=A2, q=A):
        return L.hba_prefix_softmax_split_noalloc(ctypes.byref(sh), P, ns, None, q, A, A, Kc, A, out, None)

    sh = shape()
    assert call(sh, ns=0) == ESHAPE
    assert call(sh, ns=65) == ESHAPE
    assert call(sh, Kc=None) == ENULL
    assert call(sh, out=None) == ENULL
    assert call(sh, q=MIS) == EALIGN
    assert call(shape(kv_heads=3)) == ESHAPE
    assert call(shape(batch=0)) == OK
    big = shape(batch=64, heads=16)
    assert L.hba_prefix_softmax_workspace_bytes(ctypes.byref(big), 16) > 16 * 1024 * 1024
    assert call(big, ns=16) == ECAP
    assert call(sh, ns=4) == EHIP


@no_gpu_only
def test_transfer_validation():
    L = lib()

    def call(sh, nb=4, q=A, W=A, alpha=A, loss=A2, ws=A2, wsb=1 << 40, target=A):
        return L.hba_transfer(ctypes.byref(sh), nb, q, A, A, W, alpha, target, None, loss, A2, A2, ws, wsb, None)

    sh = shape()
    need = L.hba_transfer_workspace_bytes(ctypes.byref(sh), 4)
    N = 4 * 32
    # dnum, dden, phi(q) and phi(k), two dW parts, four scalars per (request, head)
    assert need == 4 * (2 * 4 * N * 128 + 2 * 4 * N + 2 * 2 * 4 * N * 256 + 2 * 2 * 4 * 128 * 128 + 4 * 2 * 4)
    assert L.hba_transfer_workspace_bytes(ctypes.byref(shape(d=64)), 4) == -1
    assert call(shape(d=64)) == EUNSUP
    assert call(shape(F=96)) == EUNSUP
    assert call(sh, nb=-1) == ESHAPE
    assert call(shape(kv_heads=3)) == ESHAPE
    assert call(sh, q=None) == ENULL
    assert call(sh, ws=None) == ENULL
    assert call(sh, loss=None) == ENULL
    assert call(sh, wsb=need - 4) == ECAP
    assert call(sh, W=MIS) == EALIGN
    assert call(sh, target=MIS) == EALIGN
    assert call(shape(batch=65536, slots=1 << 17)) == ESHAPE
    # one sequence is indexed in 32 bits: N * 128 < 2^31 (block 32 here)
    assert call(sh, nb=(1 << 24) // 32) == ESHAPE


def test_python_binding_refuses_host_tensors():
    # no CPU fallback: host tensors are rejected before any call
    lib()
    q = torch.zeros(1, 1, 8, 64)
    W = torch.zeros(1, 64, 64)
    S = torch.zeros(1, 1, 128, 64)
    Z = torch.zeros(1, 1, 128)
    with pytest.raises(ValueError, match="GPU"):
        hba.step(q, q, q, W, S, Z)
    with pytest.raises(ValueError, match="shape"):
        hba.step(q, q, q, torch.zeros(1, 64, 32), S, Z)
    with pytest.raises(ValueError, match="dtype"):
        hba.step(q, q.bfloat16(), q, W, S, Z)
