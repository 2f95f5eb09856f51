"""fp64 GEMV / skinny GEMM, grouped MoE expert GEMV and the error metric (oracle).

The hot path computes y[b][m] = sum_k W[m][k] * x[b][k] for a weight that is
decoded on the fly ([Bolt], background: at decode time every weight is read once
per token, so the weight bytes set the speed).  The oracle forms the same
product from the dequantized fp64 weight with numpy's float64 matmul.

MoE ([Bolt] describes per-token routing to a subset of experts; the synthetic
workload routes each token to 8 of 64 experts): for token t and slot j the up
projection is W_up[route[t][j]] @ x[t] and the down projection is
W_down[route[t][j]] @ a[t][j] with an independent input per (token, slot).  No
nonlinearity or gate weighting is defined on the pages, so the two stages are
independent GEMVs and the output keeps the [T][slot][M] shape.
"""
from __future__ import annotations

import numpy as np

from .bits import bf16_value


def gemv(w: np.ndarray, x_bits: np.ndarray) -> np.ndarray:
    """fp64 [B][M] = x @ w.T for fp64 weight [M][K] and bf16 bits x [B][K]."""
    x = bf16_value(x_bits)
    return x @ w.T


def rel_l2(y, ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(y - ref) / den) if den > 0 else float(np.linalg.norm(y))


def worst_row(y, ref) -> float:
    """Largest single-element error, relative to the RMS of its own output row:
    max over b, m of |y[b][m] - ref[b][m]| / rms(ref[b]).  The whole-output rel_l2
    spreads one wrong element over all M outputs (a factor sqrt(M) smaller); this
    reports it at full size.  Rows whose reference is all zero are measured in
    absolute terms."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    ref = np.atleast_2d(np.asarray(ref, dtype=np.float64))
    y = y.reshape(-1, y.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    rms = np.sqrt(np.mean(ref * ref, axis=1))
    err = np.abs(y - ref).max(axis=1)
    return float(np.max(np.where(rms > 0, err / np.where(rms > 0, rms, 1.0), err)))


def moe(deq_up: dict, deq_down: dict, routes: np.ndarray, x_bits: np.ndarray,
        a_bits: np.ndarray):
    """(y_up [T][k][M_up], y_down [T][k][M_down]) from per-expert fp64 weights."""
    T, k = routes.shape
    x = bf16_value(x_bits)
    a = bf16_value(a_bits)
    mu = next(iter(deq_up.values())).shape[0]
    md = next(iter(deq_down.values())).shape[0]
    yu = np.zeros((T, k, mu))
    yd = np.zeros((T, k, md))
    for t in range(T):
        for j in range(k):
            e = int(routes[t, j])
            yu[t, j] = deq_up[e] @ x[t]
            yd[t, j] = deq_down[e] @ a[t, j]
    return yu, yd
