"""Context-parallel building block, in fp64 (oracle; test infrastructure only).

The ring and hybrid context-parallel methods benchmarked on "LongCA-bench: 长上下文注意力
基准测试" (xllm-io blog), section 三 "分布式注意力机制" and section 四 "分布式注意力性能",
split one long sequence into chunks, compute attention between a query chunk and one
key chunk at a time, and combine the partial results. The page gives no formulas; this
file writes out the definitions:

  partial forward of query chunk [q0, q0 + n) over key chunk [k0, k0 + n): the masked
  softmax attention restricted to that key chunk, mask = the global predicate at the
  global positions (O_part normalised over the chunk, LSE_part = ln of the chunk's sum
  of exp(scores); a row with no visible key there has O_part = 0, LSE_part = -inf);

  merge of two partials over disjoint key sets:
      LSE = ln(exp(LSE_1) + exp(LSE_2)),   O = exp(LSE_1 - LSE) O_1 + exp(LSE_2 - LSE) O_2,
  which is the attention over the union of the key sets;

  backward share of a chunk pair, given the whole rows' O and LSE: P = exp(S - LSE) on
  the pair's visible entries, D = rowsum(dO * O), dS = P * (dP - D),
      dQ_share = scale dS K_chunk,  dK_share = scale dS^T Q_chunk,  dV_share = P^T dO_chunk,
  which sum over key chunks (dQ) and over query chunks (dK, dV) to the full gradients.

Heads map to KV heads contiguously (g = h // (Hq / Hk)), as in oracle/attention.py.
"""
from __future__ import annotations

import numpy as np

from .masks import mask_block


def _lse_rows(S, M):
    """Per-row max and log-sum-exp of the visible entries of S (-inf for empty rows)."""
    any_vis = M.any(axis=1)
    Sm = np.where(M, S, -np.inf)
    m = np.where(any_vis, Sm.max(axis=1, initial=-np.inf), -np.inf)
    m_safe = np.where(any_vis, m, 0.0)
    E = np.where(M, np.exp(Sm - m_safe[:, None]), 0.0)
    l = E.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(any_vis, m_safe + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return lse, E, l, any_vis


def chunk_forward(q, k, v, spec, T, q0, k0, scale=None):
    """Partial attention of a query chunk over a key chunk.

    q : float64 [n][Hq][d] (global rows q0 .. q0+n-1);  k, v : float64 [n][Hk][d] (keys k0 ..)
    returns O_part float64 [n][Hq][d], LSE_part float64 [Hq][n]
    """
    n, Hq, d = q.shape
    Hk = k.shape[1]
    G = Hq // Hk
    scale = (1.0 / np.sqrt(d)) if scale is None else float(scale)
    M = mask_block(spec, T, np.arange(q0, q0 + n), np.arange(k0, k0 + k.shape[0]))
    O = np.zeros((n, Hq, d))
    LSE = np.empty((Hq, n))
    for h in range(Hq):
        g = h // G
        S = scale * (q[:, h, :] @ k[:, g, :].T)
        lse, E, l, any_vis = _lse_rows(S, M)
        P = np.where(any_vis[:, None], E / np.where(l > 0, l, 1.0)[:, None], 0.0)
        O[:, h, :] = P @ v[:, g, :]
        LSE[h] = lse
    return O, LSE


def lse_merge(o1, lse1, o2, lse2):
    """Combine partial results over disjoint key sets (O [n][Hq][d], LSE [Hq][n])."""
    m = np.maximum(lse1, lse2)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w1 = np.where(empty, 0.0, np.exp(lse1 - m_safe))
    w2 = np.where(empty, 0.0, np.exp(lse2 - m_safe))
    s = w1 + w2
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(s > 0, s, 1.0)))
        a1 = np.where(empty, 0.0, w1 / np.where(s > 0, s, 1.0))
        a2 = np.where(empty, 0.0, w2 / np.where(s > 0, s, 1.0))
    o = a1.T[:, :, None] * o1 + a2.T[:, :, None] * o2
    return o, lse


def chunk_backward(q, k, v, do, o_rows, lse_rows, spec, T, q0, k0, scale=None):
    """Backward share of the chunk pair, given the whole rows' O [n][Hq][d] and LSE [Hq][n].

    returns dq_share [n][Hq][d], dk_share, dv_share [n][Hk][d]
    """
    n, Hq, d = q.shape
    Hk = k.shape[1]
    G = Hq // Hk
    scale = (1.0 / np.sqrt(d)) if scale is None else float(scale)
    M = mask_block(spec, T, np.arange(q0, q0 + n), np.arange(k0, k0 + k.shape[0]))
    dq = np.zeros((n, Hq, d))
    dk = np.zeros((k.shape[0], Hk, d))
    dv = np.zeros((k.shape[0], Hk, d))
    for h in range(Hq):
        g = h // G
        S = scale * (q[:, h, :] @ k[:, g, :].T)
        lse = lse_rows[h]
        finite = np.isfinite(lse)
        P = np.where(M & finite[:, None], np.exp(S - np.where(finite, lse, 0.0)[:, None]), 0.0)
        D = np.sum(do[:, h, :] * o_rows[:, h, :], axis=1)
        dP = do[:, h, :] @ v[:, g, :].T
        dS = P * (dP - D[:, None])
        dq[:, h, :] = scale * (dS @ k[:, g, :])
        dk[:, g, :] += scale * (dS.T @ q[:, h, :])
        dv[:, g, :] += P.T @ do[:, h, :]
    return dq, dk, dv
