"""fp64 masked softmax attention, forward and explicit backward (oracle; test infrastructure only).

The operator is the one benchmarked on "LongCA-bench: 长上下文注意力基准测试"
(xllm-io blog), sections 三 "密集注意力内核" / "稀疏注意力内核" and 四 "实验设置":
softmax(Q K^T / sqrt(d) + mask) V with GQA head groups (64 query heads sharing 8 KV
heads) or MHA, head dim 128, forward and backward. The page fixes no formulas; this
file writes out the textbook definition of masked softmax attention and of its
gradient, in fp64, one query head at a time:

  S   = scale * Q_h K_g^T,  S[i, j] = -inf where the mask hides key j from query i
  m_i = max_j S[i, j],  l_i = sum_j exp(S[i, j] - m_i)
  P   = exp(S - m) / l,  O_h = P V_g,  LSE_i = m_i + ln l_i
  D_i = sum_c dO[i, c] O[i, c]
  dP  = dO_h V_g^T,  dS = P * (dP - D)
  dQ_h = scale * dS K_g,  dK_g += scale * dS^T Q_h,  dV_g += P^T dO_h

with g = h // (Hq / Hk) (contiguous head groups). A row with no visible key has
O = 0, LSE = -inf and zero gradient. Rows are processed in independent chunks (each
row's softmax involves all keys), so any subset of rows can be computed exactly.
"""
from __future__ import annotations

import numpy as np

from .masks import mask_block


def _group(Hq: int, Hk: int) -> int:
    if Hk <= 0 or Hq % Hk != 0:
        raise ValueError("Hq must be a multiple of Hk")
    return Hq // Hk


def _row_softmax(S: np.ndarray, M: np.ndarray):
    """Masked row softmax of one chunk: returns P, m (row max, -inf if empty), l."""
    S = np.where(M, S, -np.inf)
    any_vis = M.any(axis=1)
    m = np.where(any_vis, S.max(axis=1, initial=-np.inf), -np.inf)
    m_safe = np.where(any_vis, m, 0.0)
    E = np.exp(S - m_safe[:, None])          # exp(-inf) = 0 on hidden keys
    l = E.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        P = np.where(any_vis[:, None], E / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return P, m, l, any_vis


def attention_forward(q, k, v, spec, *, scale=None, heads=None, rows=None, keep=None,
                      chunk=1024):
    """Forward pass.

    q : float64 [T][Hq][d];  k, v : float64 [T][Hk][d]
    heads : query heads to compute (default all);  rows : query positions (default all)
    returns O float64 [len(rows)][len(heads)][d], LSE float64 [len(heads)][len(rows)]
    """
    T, Hq, d = q.shape
    Hk = k.shape[1]
    G = _group(Hq, Hk)
    scale = (1.0 / np.sqrt(d)) if scale is None else float(scale)
    heads = list(range(Hq)) if heads is None else list(heads)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(T)
    O = np.zeros((len(rows), len(heads), d))
    LSE = np.empty((len(heads), len(rows)))
    for hi, h in enumerate(heads):
        g = h // G
        Kg = np.ascontiguousarray(k[:, g, :])
        Vg = np.ascontiguousarray(v[:, g, :])
        for c0 in range(0, len(rows), chunk):
            R = rows[c0:c0 + chunk]
            S = scale * (q[R, h, :] @ Kg.T)
            M = mask_block(spec, T, R, cols, h, keep)
            P, m, l, any_vis = _row_softmax(S, M)
            O[c0:c0 + len(R), hi, :] = P @ Vg
            with np.errstate(divide="ignore"):
                LSE[hi, c0:c0 + len(R)] = np.where(any_vis, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return O, LSE


def attention_backward(q, k, v, do, spec, *, scale=None, heads=None, rows=None, keep=None,
                       key_cols=None, chunk=1024):
    """Forward and explicit backward.

    Returns a dict with
      o    float64 [len(rows)][len(heads)][d]
      lse  float64 [len(heads)][len(rows)]
      dq   float64 [len(rows)][len(heads)][d]
      dk, dv float64 [len(key_cols)][Hk][d]: the contributions of the given heads and
           rows only (pass all rows that see key_cols to obtain the exact gradient).
    """
    T, Hq, d = q.shape
    Hk = k.shape[1]
    G = _group(Hq, Hk)
    scale = (1.0 / np.sqrt(d)) if scale is None else float(scale)
    heads = list(range(Hq)) if heads is None else list(heads)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    key_cols = np.arange(T) if key_cols is None else np.asarray(key_cols, dtype=np.int64)
    cols = np.arange(T)
    O = np.zeros((len(rows), len(heads), d))
    LSE = np.empty((len(heads), len(rows)))
    dQ = np.zeros((len(rows), len(heads), d))
    dK = np.zeros((len(key_cols), Hk, d))
    dV = np.zeros((len(key_cols), Hk, d))
    for hi, h in enumerate(heads):
        g = h // G
        Kg = np.ascontiguousarray(k[:, g, :])
        Vg = np.ascontiguousarray(v[:, g, :])
        for c0 in range(0, len(rows), chunk):
            R = rows[c0:c0 + chunk]
            n = len(R)
            Qh = q[R, h, :]
            dOh = do[R, h, :]
            S = scale * (Qh @ Kg.T)
            M = mask_block(spec, T, R, cols, h, keep)
            P, m, l, any_vis = _row_softmax(S, M)
            Oh = P @ Vg
            O[c0:c0 + n, hi, :] = Oh
            with np.errstate(divide="ignore"):
                LSE[hi, c0:c0 + n] = np.where(any_vis, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
            D = np.sum(dOh * Oh, axis=1)
            dP = dOh @ Vg.T
            dS = P * (dP - D[:, None])
            dQ[c0:c0 + n, hi, :] = scale * (dS @ Kg)
            dS_c = dS[:, key_cols]
            P_c = P[:, key_cols]
            dK[:, g, :] += scale * (dS_c.T @ Qh)
            dV[:, g, :] += P_c.T @ dOh
    return {"o": O, "lse": LSE, "dq": dQ, "dk": dK, "dv": dV}
