"""fp64 CPU oracle for block-hybrid attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never touches it, and it never touches the product path.

The arithmetic lives in ``hba_oracle.c`` (plain C, fp64, written from
"Retrofitting Linear Attention into Diffusion Language Models", sections 2.2
and 3.1).  This module only compiles that file with gcc and marshals numpy
arrays to it.  Every array handed in is converted to contiguous fp64, which is
exact for bf16 and fp32 inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hba_oracle.c")
# HBA_ORACLE_LIB points the loader at another build of hba_oracle.c (the
# pin-sensitivity test loads builds with a planted mistake this way)
_LIB = os.environ.get("HBA_ORACLE_LIB") or os.path.join(_HERE, "libhba_oracle.so")

_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (host only, OpenMP over independent pairs)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.orc_threads.argtypes = [ctypes.c_int]
        lib.orc_threads.restype = ctypes.c_int
        lib.orc_feature_map.argtypes = [i64, i32, i32, i32, _f64p, _f64p, _f64p, ctypes.c_int]
        lib.orc_commit.argtypes = [i32, i32, i32, i32, i32, i32, _i32p, _f64p, _f64p, _f64p,
                                   _f64p, _f64p, _i32p, ctypes.c_int]
        lib.orc_step.argtypes = [i32, i32, i32, i32, i32, i32, _f64p, _f64p, _f64p, _f64p, _f64p,
                                 _f64p, _f64p, _i32p, _f64p, ctypes.c_int]
        lib.orc_prefix_softmax.argtypes = [i32, i32, i32, i32, i32, i32, _i32p, _f64p, _f64p, _f64p,
                                           _f64p, _f64p, _f64p, ctypes.c_int]
        lib.orc_transfer.argtypes = [i32, i32, i32, i32, i32, i32, i32, _f64p, _f64p, _f64p, _f64p, _f64p,
                                     _f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_int]
        for fn in (lib.orc_feature_map, lib.orc_commit, lib.orc_step, lib.orc_prefix_softmax, lib.orc_transfer):
            fn.restype = ctypes.c_int
        _lib_handle = lib
    return _lib_handle


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor: widen exactly on the host
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a, t=_f64p):
    return None if a is None else a.ctypes.data_as(t)


def threads(nthreads: int = 0) -> int:
    """Threads an oracle call with ``nthreads`` (0 = OpenMP default) uses."""
    return int(_lib().orc_threads(nthreads))


def feature_map(x, W, nthreads: int = 0) -> np.ndarray:
    """phi = [softmax(xW), softmax(-xW)] per head.  x [n][H][d], W [H][d][F]
    -> phi [n][H][2F] (section 3.1, Hedgehog feature map)."""
    x, W = _f64(x), _f64(W)
    n, H, d = x.shape
    F = W.shape[2]
    assert W.shape == (H, d, F)
    phi = np.zeros((n, H, 2 * F))
    rc = _lib().orc_feature_map(n, H, d, F, _p(x), _p(W), _p(phi), nthreads)
    if rc:
        raise OracleError(f"orc_feature_map rc={rc}")
    return phi


def _kv_heads(H: int, Hkv: int) -> int:
    if Hkv <= 0 or H % Hkv:
        raise OracleError(f"{H} query heads cannot share {Hkv} key/value heads evenly")
    return Hkv


def commit(S_pool, Z_pool, k, v, W, n_valid=None, slot=None, nthreads: int = 0):
    """Fold k, v [B][Hkv][T][d] into the pool states of the H = W.shape[0]
    query heads (section 3.1, state update); query head h reads key/value head
    h // (H // Hkv).  Returns the (fp64) S_pool, Z_pool arrays it updated."""
    S_pool, Z_pool = _f64(S_pool).copy(), _f64(Z_pool).copy()
    k, v, W = _f64(k), _f64(v), _f64(W)
    B, Hkv, T, d = k.shape
    H, _, F = W.shape
    _kv_heads(H, Hkv)
    assert v.shape == k.shape and W.shape == (H, d, F)
    assert S_pool.shape[1:] == (H, 2 * F, d) and Z_pool.shape[1:] == (H, 2 * F)
    nv, sl = _i32(n_valid), _i32(slot)
    rc = _lib().orc_commit(B, H, Hkv, T, d, F, _p(nv, _i32p), _p(k), _p(v), _p(W),
                           _p(S_pool), _p(Z_pool), _p(sl, _i32p), nthreads)
    if rc:
        raise OracleError(f"orc_commit rc={rc}")
    return S_pool, Z_pool


def step(q, k, v, W, S_pool, Z_pool, gate=None, slot=None, nthreads: int = 0) -> np.ndarray:
    """One block-hybrid denoising step; q [B][H][L][d], k, v [B][Hkv][L][d]
    -> out [B][H][L][d] (section 3.1: within-block softmax, linear readout,
    gated merge).  Query head h reads key/value head h // (H // Hkv)."""
    q, k, v, W = _f64(q), _f64(k), _f64(v), _f64(W)
    S_pool, Z_pool = _f64(S_pool), _f64(Z_pool)
    B, H, L, d = q.shape
    F = W.shape[2]
    Hkv = _kv_heads(H, k.shape[1])
    assert k.shape == (B, Hkv, L, d) and v.shape == k.shape and W.shape == (H, d, F)
    assert S_pool.shape[1:] == (H, 2 * F, d) and Z_pool.shape[1:] == (H, 2 * F)
    g = None if gate is None else _f64(gate)
    sl = _i32(slot)
    out = np.zeros((B, H, L, d))
    rc = _lib().orc_step(B, H, Hkv, L, d, F, _p(q), _p(k), _p(v), _p(W), _p(g),
                         _p(S_pool), _p(Z_pool), _p(sl, _i32p), _p(out), nthreads)
    if rc:
        raise OracleError(f"orc_step rc={rc}")
    return out


def prefix_softmax(q, k, v, Kc, Vc, prefix_len=None, nthreads: int = 0) -> np.ndarray:
    """Full softmax attention of block queries over [prefix cache ; block]
    (section 2.2, softmax attention): the comparator.  k, v [B][Hkv][L][d],
    Kc, Vc [B][Hkv][P][d]; query head h reads key/value head h // (H // Hkv)."""
    q, k, v, Kc, Vc = _f64(q), _f64(k), _f64(v), _f64(Kc), _f64(Vc)
    B, H, L, d = q.shape
    P = Kc.shape[2]
    Hkv = _kv_heads(H, k.shape[1])
    assert k.shape == (B, Hkv, L, d) and v.shape == k.shape
    assert Kc.shape == (B, Hkv, P, d) and Vc.shape == Kc.shape
    pl = _i32(prefix_len)
    out = np.zeros((B, H, L, d))
    rc = _lib().orc_prefix_softmax(B, H, Hkv, L, d, P, _p(pl, _i32p), _p(q), _p(k), _p(v),
                                   _p(Kc), _p(Vc), _p(out), nthreads)
    if rc:
        raise OracleError(f"orc_prefix_softmax rc={rc}")
    return out


def transfer(q, k, v, W, alpha, target, block: int, nthreads: int = 0):
    """Stage-1 attention transfer (section 3.2) for one layer: the hybrid
    output over whole sequences of N = n_blocks * block tokens (section 3.1:
    block softmax plus the states of all earlier blocks), the summed squared
    error against ``target`` and its gradient with respect to W and alpha.
    q, target [B][H][N][d]; k, v [B][Hkv][N][d]; W [H][d][F]; alpha [H].
    Returns (out, loss, dW, dalpha)."""
    q, k, v, W = _f64(q), _f64(k), _f64(v), _f64(W)
    alpha, target = _f64(alpha), _f64(target)
    B, H, N, d = q.shape
    F = W.shape[2]
    Hkv = _kv_heads(H, k.shape[1])
    if N % block:
        raise OracleError(f"{N} tokens are not whole blocks of {block}")
    assert k.shape == (B, Hkv, N, d) and v.shape == k.shape and target.shape == q.shape
    assert W.shape == (H, d, F) and alpha.shape == (H,)
    out = np.zeros((B, H, N, d))
    loss = np.zeros(1)
    dW = np.zeros((H, d, F))
    dalpha = np.zeros(H)
    rc = _lib().orc_transfer(B, H, Hkv, N // block, block, d, F, _p(q), _p(k), _p(v), _p(W), _p(alpha),
                             _p(target), _p(out), _p(loss), _p(dW), _p(dalpha), nthreads)
    if rc:
        raise OracleError(f"orc_transfer rc={rc}")
    return out, float(loss[0]), dW, dalpha
