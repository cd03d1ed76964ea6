"""Element-by-element check of a verify-GEMM output against the fp64 oracle,
computed in column slices so that full-size products (the lm-head's 29 M
outputs, the M = 1024 sweep point) fit in host memory.

Tolerance: per element |y - y_ref| <= 1e-2 * max(|y_ref|, rms(Y_ref)), with
rms over the whole output; the relative Frobenius error is also bounded.
A pure per-element relative test is meaningless where y_ref ~ 0, since fp32
accumulation over K terms leaves an absolute error of order
1e-7 * sqrt(K) * |x||w|.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = 1e-2
FRO_TOL = 5e-3


def reference_sliced(X: torch.Tensor, W: torch.Tensor, cols: int = 8192) -> np.ndarray:
    """The fp64 oracle product of device bf16 operands, one column slice of W
    at a time (the operands are widened exactly to fp32 on the way)."""
    Xh = X.float().cpu().numpy()
    N = W.shape[1]
    out = np.empty((X.shape[0], N), np.float64)
    for c0 in range(0, N, cols):
        c1 = min(N, c0 + cols)
        out[:, c0:c1] = oracle.verify_linear(Xh, W[:, c0:c1].float().cpu().numpy())
    return out


def check_full(Y: torch.Tensor, ref: np.ndarray, label) -> dict:
    """Every element of Y against ref; returns the worst scaled error and the
    relative Frobenius error."""
    Yh = Y.float().cpu().numpy().astype(np.float64)
    assert Yh.shape == ref.shape, (label, Yh.shape, ref.shape)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    lim = TOL * np.maximum(np.abs(ref), rms)
    err = np.abs(Yh - ref)
    bad = err > lim
    if bad.any() or not np.all(np.isfinite(Yh)):
        i = int(np.argmax(np.where(np.isfinite(err), err / lim, np.inf)))
        raise AssertionError(f"{label}: {int(bad.sum())} elements out of tolerance; worst at flat "
                             f"index {i}: got {Yh.flat[i]!r} ref {ref.flat[i]!r} rms {rms:.4g}")
    fro = float(np.linalg.norm(Yh - ref) / max(np.linalg.norm(ref), 1e-300))
    assert fro < FRO_TOL, (label, fro)
    return dict(worst_scaled=float(np.max(err / np.maximum(np.abs(ref), rms))), fro=fro,
                elements=int(ref.size))
