"""Error measures and tolerances shared by the GPU parity tests.

Tolerances (the bar every GPU result must meet against the fp64 oracle):
  fp32 inputs                           : relative error <= 1e-5
  bf16 inputs, fp32 state/accumulation  : relative error <= 3e-3
Relative error of an output is the max over query rows of
||o - o_ref||_2 / ||o_ref||_2; of a state, the max over (request, head) of the
Frobenius-norm ratio; of phi, the max over rows of the L2 ratio.

The bf16 paths also carry a tighter guard, DESIGN_TOL = 1e-4.  Products of two
bf16 inputs are exact, and every fp32 operand that meets bf16 matrix cores
(phi, softmax weights, the fp32 states) is split into a bf16 high part and a
bf16 residual, so the design keeps about 16 mantissa bits per product
(measured errors are a few 1e-6).  A state or operand rounded to plain bf16
instead gives errors of a few 1e-4: that passes 3e-3 but fails the guard, so a
lost residual term cannot pass unnoticed.
"""
import numpy as np
import torch

TOL = {torch.float32: 1e-5, torch.bfloat16: 3e-3}
DESIGN_TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-4}


def host64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").double().numpy()


def row_rel(out, ref) -> float:
    o, r = host64(out), host64(ref)
    num = np.linalg.norm(o - r, axis=-1)
    den = np.maximum(np.linalg.norm(r, axis=-1), 1e-300)
    return float(np.max(num / den)) if num.size else 0.0


def state_rel(S, Sref) -> float:
    """Max over leading (slot/request, head) entries of the relative Frobenius error."""
    s, r = host64(S), host64(Sref)
    lead = s.shape[:2]
    s = s.reshape(*lead, -1)
    r = r.reshape(*lead, -1)
    num = np.linalg.norm(s - r, axis=-1)
    den = np.maximum(np.linalg.norm(r, axis=-1), 1e-300)
    return float(np.max(num / den)) if num.size else 0.0


def report(name, **errs):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)


def check(errs: dict, dtype) -> None:
    """Every error within the stated bar and within the design's precision guard."""
    for name, e in errs.items():
        assert e <= TOL[dtype], f"{name}: {e:.3e} exceeds the bar {TOL[dtype]:g}"
        assert e <= DESIGN_TOL[dtype], f"{name}: {e:.3e} exceeds the split-bf16 guard {DESIGN_TOL[dtype]:g}"
