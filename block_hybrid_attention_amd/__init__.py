"""Block-hybrid attention for AMD Instinct MI355X (gfx950).

Python binding of ``libhba.so`` through ctypes.  This module only checks
tensor shapes, dtypes and devices and passes raw device pointers plus the
current HIP stream to the C ABI declared in ``include/hba.h``; every step of
the computation runs in the library's HIP kernels.  There is no fallback: if
the library is not built, every call raises.

The method: "Retrofitting Linear Attention into Diffusion Language Models",
section 3.1 (block-hybrid attention: exact softmax inside the active block,
Hedgehog linear attention over committed blocks through fixed-size states,
one shared normaliser) and section 2.2 (the softmax attention it replaces,
exposed here as the ``prefix_softmax`` comparator).
"""
from __future__ import annotations

import ctypes
import os

import torch

from .pool import StatePool  # noqa: F401  (re-exported)

__all__ = ["feature_map", "step", "commit", "prefix_softmax", "StatePool", "HbaError",
           "library_path", "load_library", "abi_version", "step_commit", "prefix_softmax_workspace_bytes",
           "prefix_softmax_auto_split", "transfer", "transfer_workspace_bytes", "prefix_softmax_noalloc",
           "NOALLOC_SCRATCH_BYTES"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libhba.so")

HBA_F32, HBA_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024   # HBA_NOALLOC_SCRATCH_BYTES in include/hba.h
_DTYPE = {torch.float32: HBA_F32, torch.bfloat16: HBA_BF16}
_STATUS = {0: "HBA_OK", 1: "HBA_ERR_NULL", 2: "HBA_ERR_SHAPE", 3: "HBA_ERR_UNSUPPORTED",
           4: "HBA_ERR_DTYPE", 5: "HBA_ERR_ALIGN", 6: "HBA_ERR_CAPACITY", 7: "HBA_ERR_HIP"}


class HbaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = load_library().hba_status_string(status).decode()
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({msg})")


class Shape(ctypes.Structure):
    """Mirror of ``hba_shape``."""
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("block", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("feat", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("n_slots", ctypes.c_int64), ("kv_heads", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


_lib = None


def load_library():
    """Load libhba.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m block_hybrid_attention_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, sp = ctypes.c_void_p, ctypes.POINTER(Shape)
        lib.hba_status_string.argtypes = [ctypes.c_int]
        lib.hba_status_string.restype = ctypes.c_char_p
        lib.hba_abi_version.argtypes = []
        lib.hba_abi_version.restype = ctypes.c_int32
        lib.hba_feature_map.argtypes = [sp, ctypes.c_int64, vp, vp, vp, vp]
        lib.hba_step.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.hba_prefix_softmax_split.argtypes = [sp, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp]
        lib.hba_prefix_softmax_split_noalloc.argtypes = [sp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.hba_prefix_softmax_auto_split.argtypes = [sp, i32]
        lib.hba_prefix_softmax_auto_split.restype = i32
        lib.hba_prefix_softmax_workspace_bytes.argtypes = [sp, i32]
        lib.hba_prefix_softmax_workspace_bytes.restype = i64
        lib.hba_transfer.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp]
        lib.hba_transfer_workspace_bytes.argtypes = [sp, i32]
        lib.hba_transfer_workspace_bytes.restype = i64
        lib.hba_commit.argtypes = [sp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.hba_prefix_softmax.argtypes = [sp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.hba_step_commit.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        for fn in (lib.hba_feature_map, lib.hba_step, lib.hba_commit, lib.hba_prefix_softmax,
                   lib.hba_step_commit, lib.hba_prefix_softmax_split, lib.hba_transfer):
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def abi_version() -> int:
    return int(load_library().hba_abi_version())


# ----------------------------------------------------------------- helpers
def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("block-hybrid attention tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("block-hybrid attention tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors of one call must be on the same device")
    return dev


def _in_dtype(*ts):
    dt = ts[0].dtype
    if dt not in _DTYPE:
        raise ValueError(f"input dtype {dt} not supported (float32 or bfloat16)")
    for t in ts:
        if t is not None and t.dtype != dt:
            raise ValueError("q, k, v, x, W, Kc and Vc must share one dtype")
    return _DTYPE[dt]


def _check(t, shape, dtype, name):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _call(fn, name, *args):
    st = fn(*args)
    if st != 0:
        raise HbaError(st, name)


# --------------------------------------------------------------- the calls
def feature_map(x: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """phi(x) = [softmax(xW), softmax(-xW)] per head (section 3.1).

    x [n][H][d], W [H][d][F] (same dtype) -> phi [n][H][2F] fp32."""
    lib = load_library()
    n, H, d = x.shape
    F = W.shape[2]
    dt = _in_dtype(x, W)
    _check(W, (H, d, F), x.dtype, "W")
    if out is None:
        out = torch.empty((n, H, 2 * F), device=x.device, dtype=torch.float32)
    _check(out, (n, H, 2 * F), torch.float32, "out")
    _dev(x, W, out)
    shape = Shape(0, H, 1, d, F, dt, 0)
    _call(lib.hba_feature_map, "hba_feature_map", ctypes.byref(shape), n, _p(x), _p(W), _p(out), _stream(stream))
    return out


def _kv_heads(H, k):
    """Key/value heads of k [B][Hkv][..][d]; H must be a multiple of it."""
    Hkv = k.shape[1]
    if Hkv <= 0 or H % Hkv:
        raise ValueError(f"k: {Hkv} key/value heads do not divide {H} query heads")
    return Hkv


def step(q, k, v, W, S_pool, Z_pool, gate=None, slot=None, out=None, stream=None):
    """One block-hybrid denoising step (section 3.1).

    q [B][H][L][d]; k, v [B][Hkv][L][d] with Hkv dividing H (query head h
    reads key/value head h // (H // Hkv)); W [H][d][F]; S_pool [n_slots][H][2F][d] fp32;
    Z_pool [n_slots][H][2F] fp32; gate [H] fp32 (w = sigma(alpha)) or None;
    slot [B] int32 or None (request b uses slot b) -> out [B][H][L][d] fp32."""
    lib = load_library()
    B, H, L, d = q.shape
    F = W.shape[2]
    dt = _in_dtype(q, k, v, W)
    Hkv = _kv_heads(H, k)
    for t, nm in ((k, "k"), (v, "v")):
        _check(t, (B, Hkv, L, d), q.dtype, nm)
    _check(W, (H, d, F), q.dtype, "W")
    n_slots = S_pool.shape[0]
    _check(S_pool, (n_slots, H, 2 * F, d), torch.float32, "S_pool")
    _check(Z_pool, (n_slots, H, 2 * F), torch.float32, "Z_pool")
    _check(gate, (H,), torch.float32, "gate")
    _check(slot, (B,), torch.int32, "slot")
    if out is None:
        out = torch.empty((B, H, L, d), device=q.device, dtype=torch.float32)
    _check(out, (B, H, L, d), torch.float32, "out")
    _dev(q, k, v, W, S_pool, Z_pool, gate, slot, out)
    shape = Shape(B, H, L, d, F, dt, n_slots, Hkv)
    _call(lib.hba_step, "hba_step", ctypes.byref(shape), _p(q), _p(k), _p(v), _p(W), _p(gate),
          _p(S_pool), _p(Z_pool), _p(slot), _p(out), _stream(stream))
    return out


def step_commit(q, k, v, W, S_pool, Z_pool, gate=None, slot=None, n_valid=None, out=None, stream=None):
    """The block's last denoising step fused with its commit (sections 3.1, 3.3):
    out = step(q, k, v) on the states as they are, then S += sum_t phi(k_t) v_t^T,
    Z += sum_t phi(k_t) over the first n_valid[b] tokens (all L when None).
    Shapes as for step(); S_pool and Z_pool are updated in place."""
    lib = load_library()
    B, H, L, d = q.shape
    F = W.shape[2]
    dt = _in_dtype(q, k, v, W)
    Hkv = _kv_heads(H, k)
    for t, nm in ((k, "k"), (v, "v")):
        _check(t, (B, Hkv, L, d), q.dtype, nm)
    _check(W, (H, d, F), q.dtype, "W")
    n_slots = S_pool.shape[0]
    _check(S_pool, (n_slots, H, 2 * F, d), torch.float32, "S_pool")
    _check(Z_pool, (n_slots, H, 2 * F), torch.float32, "Z_pool")
    _check(gate, (H,), torch.float32, "gate")
    _check(slot, (B,), torch.int32, "slot")
    _check(n_valid, (B,), torch.int32, "n_valid")
    if out is None:
        out = torch.empty((B, H, L, d), device=q.device, dtype=torch.float32)
    _check(out, (B, H, L, d), torch.float32, "out")
    _dev(q, k, v, W, S_pool, Z_pool, gate, slot, n_valid, out)
    shape = Shape(B, H, L, d, F, dt, n_slots, Hkv)
    _call(lib.hba_step_commit, "hba_step_commit", ctypes.byref(shape), _p(n_valid), _p(q), _p(k), _p(v),
          _p(W), _p(gate), _p(S_pool), _p(Z_pool), _p(slot), _p(out), _stream(stream))
    return out


def commit(k, v, W, S_pool, Z_pool, n_valid=None, slot=None, stream=None):
    """Fold k, v [B][Hkv][T][d] into the states of the H = W.shape[0] query
    heads in place (section 3.1): S += sum_t phi(k_t) v_t^T, Z += sum_t phi(k_t)
    over the first n_valid[b] tokens of each request (all T when n_valid is
    None); query head h absorbs key/value head h // (H // Hkv)."""
    lib = load_library()
    B, Hkv, T, d = k.shape
    H, F = W.shape[0], W.shape[2]
    dt = _in_dtype(k, v, W)
    _kv_heads(H, k)
    _check(v, (B, Hkv, T, d), k.dtype, "v")
    _check(W, (H, d, F), k.dtype, "W")
    n_slots = S_pool.shape[0]
    _check(S_pool, (n_slots, H, 2 * F, d), torch.float32, "S_pool")
    _check(Z_pool, (n_slots, H, 2 * F), torch.float32, "Z_pool")
    _check(n_valid, (B,), torch.int32, "n_valid")
    _check(slot, (B,), torch.int32, "slot")
    _dev(k, v, W, S_pool, Z_pool, n_valid, slot)
    shape = Shape(B, H, 1, d, F, dt, n_slots, Hkv)
    _call(lib.hba_commit, "hba_commit", ctypes.byref(shape), T, _p(n_valid), _p(k), _p(v), _p(W),
          _p(S_pool), _p(Z_pool), _p(slot), _stream(stream))


def prefix_softmax(q, k, v, Kc, Vc, prefix_len=None, out=None, stream=None, n_split=1, workspace=None):
    """Comparator: full softmax attention (section 2.2) of the block queries
    over [prefix cache ; block].  q [B][H][L][d]; k, v [B][Hkv][L][d];
    Kc, Vc [B][Hkv][P][d] (same dtype), Hkv dividing H; prefix_len [B] int32
    or None (all P).

    n_split > 1 splits each (request, head)'s keys over that many workgroups
    (hba_prefix_softmax_split); None takes the library's choice for the
    current device.  The split needs a device workspace of
    prefix_softmax_workspace_bytes(...) bytes, allocated here when not given."""
    lib = load_library()
    B, H, L, d = q.shape
    P = Kc.shape[2]
    dt = _in_dtype(q, k, v, Kc, Vc)
    Hkv = _kv_heads(H, k)
    for t, nm in ((k, "k"), (v, "v")):
        _check(t, (B, Hkv, L, d), q.dtype, nm)
    _check(Kc, (B, Hkv, P, d), q.dtype, "Kc")
    _check(Vc, (B, Hkv, P, d), q.dtype, "Vc")
    _check(prefix_len, (B,), torch.int32, "prefix_len")
    if out is None:
        out = torch.empty((B, H, L, d), device=q.device, dtype=torch.float32)
    _check(out, (B, H, L, d), torch.float32, "out")
    _dev(q, k, v, Kc, Vc, prefix_len, out)
    shape = Shape(B, H, L, d, 64, dt, 0, Hkv)
    kc = _p(Kc) if P > 0 else None
    vc = _p(Vc) if P > 0 else None
    if n_split is None:
        n_split = int(lib.hba_prefix_softmax_auto_split(ctypes.byref(shape), P))
    if n_split == 1:
        _call(lib.hba_prefix_softmax, "hba_prefix_softmax", ctypes.byref(shape), P, _p(prefix_len), _p(q),
              _p(k), _p(v), kc, vc, _p(out), _stream(stream))
        return out
    need = int(lib.hba_prefix_softmax_workspace_bytes(ctypes.byref(shape), n_split))
    if need < 0:
        raise ValueError(f"n_split={n_split} is outside 1..64")
    if workspace is None:
        workspace = torch.empty((need + 3) // 4, device=q.device, dtype=torch.float32)
    if workspace.dtype != torch.float32 or not workspace.is_contiguous() or workspace.numel() * 4 < need:
        raise ValueError(f"workspace: need a contiguous fp32 tensor of at least {need} bytes")
    _dev(workspace)
    _call(lib.hba_prefix_softmax_split, "hba_prefix_softmax_split", ctypes.byref(shape), P, n_split,
          _p(prefix_len), _p(q), _p(k), _p(v), kc, vc, _p(workspace), workspace.numel() * 4, _p(out),
          _stream(stream))
    return out


def prefix_softmax_noalloc(q, k, v, Kc, Vc, out, n_split=None, prefix_len=None, stream=None):
    """The split comparator through hba_prefix_softmax_split_noalloc: the
    partials go to the library's fixed per-device scratch array, so the call
    allocates nothing (``out`` is the caller's).  n_split None takes the
    library's choice.  Calls that overlap on one device race."""
    lib = load_library()
    B, H, L, d = q.shape
    P = Kc.shape[2]
    dt = _in_dtype(q, k, v, Kc, Vc)
    Hkv = _kv_heads(H, k)
    for t, nm in ((k, "k"), (v, "v")):
        _check(t, (B, Hkv, L, d), q.dtype, nm)
    _check(Kc, (B, Hkv, P, d), q.dtype, "Kc")
    _check(Vc, (B, Hkv, P, d), q.dtype, "Vc")
    _check(prefix_len, (B,), torch.int32, "prefix_len")
    _check(out, (B, H, L, d), torch.float32, "out")
    _dev(q, k, v, Kc, Vc, prefix_len, out)
    shape = Shape(B, H, L, d, 64, dt, 0, Hkv)
    if n_split is None:
        n_split = int(lib.hba_prefix_softmax_auto_split(ctypes.byref(shape), P))
    _call(lib.hba_prefix_softmax_split_noalloc, "hba_prefix_softmax_split_noalloc", ctypes.byref(shape), P,
          n_split, _p(prefix_len), _p(q), _p(k), _p(v), _p(Kc) if P > 0 else None, _p(Vc) if P > 0 else None,
          _p(out), _stream(stream))
    return out


def prefix_softmax_workspace_bytes(B, H, L, d, n_split, dtype=torch.bfloat16) -> int:
    """Workspace bytes of the split comparator (0 for n_split = 1)."""
    shape = Shape(B, H, L, d, 64, _DTYPE[dtype], 0, 0)
    need = int(load_library().hba_prefix_softmax_workspace_bytes(ctypes.byref(shape), n_split))
    if need < 0:
        raise ValueError("invalid shape or n_split")
    return need


def prefix_softmax_auto_split(B, H, L, d, max_prefix, dtype=torch.bfloat16) -> int:
    """The library's key-split choice for the current device."""
    shape = Shape(B, H, L, d, 64, _DTYPE[dtype], 0, 0)
    return int(load_library().hba_prefix_softmax_auto_split(ctypes.byref(shape), max_prefix))


def transfer_workspace_bytes(B, H, block, d, F, n_blocks, dtype=torch.bfloat16) -> int:
    """Workspace bytes of transfer() for this shape."""
    shape = Shape(B, H, block, d, F, _DTYPE[dtype], 0, 0)
    need = int(load_library().hba_transfer_workspace_bytes(ctypes.byref(shape), n_blocks))
    if need < 0:
        raise ValueError("unsupported shape for the transfer kernels (head_dim must be 128)")
    return need


def transfer(q, k, v, W, alpha, target, block, out=None, workspace=None, stream=None):
    """Stage-1 attention transfer (section 3.2) of the hybrid layer (section
    3.1) over whole sequences of N = n_blocks * block tokens: the summed
    squared error against ``target`` and its gradients for W and alpha.

    q, target [B][H][N][128] (target fp32); k, v [B][Hkv][N][128]; W [H][128][F];
    alpha [H] fp32 (w = sigma(alpha)).  Returns (loss [1], dW [H][128][F],
    dalpha [H], out) with out [B][H][N][128] fp32 when given (else None)."""
    lib = load_library()
    B, H, N, d = q.shape
    F = W.shape[2]
    dt = _in_dtype(q, k, v, W)
    Hkv = _kv_heads(H, k)
    if N % block:
        raise ValueError(f"{N} tokens are not whole blocks of {block}")
    nb = N // block
    for t, nm in ((k, "k"), (v, "v")):
        _check(t, (B, Hkv, N, d), q.dtype, nm)
    _check(W, (H, d, F), q.dtype, "W")
    _check(alpha, (H,), torch.float32, "alpha")
    _check(target, (B, H, N, d), torch.float32, "target")
    _check(out, (B, H, N, d), torch.float32, "out")
    shape = Shape(B, H, block, d, F, dt, 0, Hkv)
    need = int(lib.hba_transfer_workspace_bytes(ctypes.byref(shape), nb))
    if need < 0:
        raise ValueError("unsupported shape for the transfer kernels (head_dim must be 128)")
    if workspace is None:
        workspace = torch.empty((need + 3) // 4, device=q.device, dtype=torch.float32)
    if workspace.dtype != torch.float32 or not workspace.is_contiguous() or workspace.numel() * 4 < need:
        raise ValueError(f"workspace: need a contiguous fp32 tensor of at least {need} bytes")
    loss = torch.empty(1, device=q.device, dtype=torch.float32)
    dW = torch.empty((H, d, F), device=q.device, dtype=torch.float32)
    dalpha = torch.empty(H, device=q.device, dtype=torch.float32)
    _dev(q, k, v, W, alpha, target, out, workspace, loss)
    _call(lib.hba_transfer, "hba_transfer", ctypes.byref(shape), nb, _p(q), _p(k), _p(v), _p(W), _p(alpha),
          _p(target), _p(out), _p(loss), _p(dW), _p(dalpha), _p(workspace), workspace.numel() * 4,
          _stream(stream))
    return loss, dW, dalpha, out
