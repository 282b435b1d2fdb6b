"""Reference matrix-vector product (test infrastructure only).

The fused kernel's result has a plain definition: y[b, r] = sum_c W_val[r, c] *
x_val[b, c], with W_val the decoded weight values (lossless decoding gives exactly
the encoded tensor: MINE page abstract and Section 4.1; DFloat11 page's
bit-identical outputs) and x_val the real value of each fp16 / bf16 activation.
It is evaluated here in float64 with numpy's matmul.

Acceptance bound, per output: |y - y_ref| <= 1e-3 * sum_c |W_val[r, c] * x_val[b, c]|.
"""
from __future__ import annotations

import numpy as np

REL_TOL = 1e-3


def x_values(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp16 array, or bf16 bit patterns (uint16) -> float64 values."""
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        b = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return b.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def gemv_f64(w_val: np.ndarray, x_val: np.ndarray) -> np.ndarray:
    """[N, K] x [B, K] -> [B, N] in float64."""
    return np.asarray(x_val, np.float64) @ np.asarray(w_val, np.float64).T


def abs_bound(w_val: np.ndarray, x_val: np.ndarray) -> np.ndarray:
    return np.abs(np.asarray(x_val, np.float64)) @ np.abs(np.asarray(w_val, np.float64)).T


def check(y: np.ndarray, w_val: np.ndarray, x_val: np.ndarray):
    """-> (pass, worst ratio |err| / (1e-3 * bound))."""
    ref = gemv_f64(w_val, x_val)
    bnd = abs_bound(w_val, x_val)
    err = np.abs(np.asarray(y, np.float64) - ref)
    allowed = REL_TOL * bnd
    ratio = np.where(allowed > 0, err / np.where(allowed > 0, allowed, 1), np.where(err > 0, np.inf, 0))
    worst = float(ratio.max()) if ratio.size else 0.0
    return worst <= 1.0, worst
