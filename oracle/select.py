"""Dynamic block selection (TopK / TopP) and the Variable Block expansion, in fp64
(oracle; test infrastructure only).

"LongCA-bench: 长上下文注意力基准测试" (xllm-io blog) lists two dynamic block masks in
section 三 "注意力掩码模式" (动态掩码: Uniform Block with a fixed block size such as
64 x 64, Variable Block with variable block sizes) and, in its review of the paper's
limitations, names TopK / TopP as the selection criterion of dynamic block-sparse
attention. The page defines neither; this file writes out the plainest readings:

  block score   s[h][qb][kb] = scale * mean(Q_h rows of query block qb) .
                                       mean(K_g rows of key block kb),   g = h // G,
                the means over the block's rows that exist (the last block may be short);
                by bilinearity this is the mean of the scaled scores over the block;
  order         per (h, qb): the diagonal block kb = qb first when keep_diagonal is set,
                then the other blocks by descending score, equal scores by ascending kb;
  TopK          keep the first min(k, nb) blocks of the order;
  TopP          keep the shortest prefix of the order whose softmax mass (over all nb
                blocks of the row, natural exp) reaches p;
  Variable Block with block edges on multiples of 64: keep64[h][qt][kt] =
                keep_var[h][r][c] for the row block r holding query tile qt and the
                column block c holding key tile kt.
"""
from __future__ import annotations

import numpy as np


def block_means(x, b):
    """x float64 [T][H][d] -> float64 [H][nb][d]: the mean of every block of b rows."""
    T, H, d = x.shape
    nb = -(-T // b)
    out = np.empty((H, nb, d))
    for blk in range(nb):
        out[:, blk, :] = x[blk * b:min(T, (blk + 1) * b)].mean(axis=0)
    return out


def block_scores(q, k, b, scale=None):
    """q float64 [T][Hq][d], k [T][Hk][d] -> block scores float64 [Hq][nb][nb]."""
    T, Hq, d = q.shape
    Hk = k.shape[1]
    G = Hq // Hk
    scale = (1.0 / np.sqrt(d)) if scale is None else float(scale)
    qm, km = block_means(q, b), block_means(k, b)
    return np.stack([scale * (qm[h] @ km[h // G].T) for h in range(Hq)])


def selection_order(row, qb, keep_diagonal):
    """Key blocks of one row of scores in selection order."""
    nb = len(row)
    rest = sorted((kb for kb in range(nb) if not (keep_diagonal and kb == qb)),
                  key=lambda kb: (-row[kb], kb))
    return ([qb] if keep_diagonal and qb < nb else []) + rest


def select_topk(scores, k, keep_diagonal=True):
    """scores [Hq][nqb][nkb] -> keep uint8 of the same shape."""
    keep = np.zeros(scores.shape, dtype=np.uint8)
    for h in range(scores.shape[0]):
        for qb in range(scores.shape[1]):
            for kb in selection_order(scores[h, qb], qb, keep_diagonal)[:k]:
                keep[h, qb, kb] = 1
    return keep


def softmax_row(row):
    e = np.exp(np.asarray(row, dtype=np.float64) - np.max(row))
    return e / e.sum()


def select_topp(scores, p, keep_diagonal=True):
    """scores [Hq][nqb][nkb] -> keep uint8: the shortest prefix of the order with mass >= p."""
    keep = np.zeros(scores.shape, dtype=np.uint8)
    for h in range(scores.shape[0]):
        for qb in range(scores.shape[1]):
            prob = softmax_row(scores[h, qb])
            mass = 0.0
            for kb in selection_order(scores[h, qb], qb, keep_diagonal):
                keep[h, qb, kb] = 1
                mass += prob[kb]
                if mass >= p:
                    break
    return keep


def expand_variable_blocks(keep_var, row_offsets, col_offsets, unit=64):
    """keep_var [Hq][nr][nc] over a grid with edges on multiples of ``unit`` -> the
    uniform keep matrix [Hq][nt][nt] over unit-sized tiles (nt = ceil(T / unit))."""
    T = int(row_offsets[-1])
    nt = -(-T // unit)
    starts = np.arange(nt) * unit
    r = np.searchsorted(np.asarray(row_offsets), starts, side="right") - 1
    c = np.searchsorted(np.asarray(col_offsets), starts, side="right") - 1
    return keep_var[:, r][:, :, c].astype(np.uint8)
