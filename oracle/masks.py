"""Per-element mask predicates (oracle; test infrastructure only).

Source: "LongCA-bench: 长上下文注意力基准测试" (xllm-io blog), section 三
"注意力掩码模式". The page names the masks and their typical use but gives no
formulas; the predicates below are the plainest readings consistent with the names
and with the workload descriptions (question + answers, bidirectional prefix,
1024-token causal blocks with a final block that sees everything, 128 global tokens
plus a window; for the two document-level heterogeneous masks, the prefix and the
causal blocks of the non-document versions applied inside every packed document; the two
dynamic masks of section 三 "动态掩码", Uniform Block and Variable Block, as block-sparse
keep matrices over a uniform grid and over a grid of variable block sizes). i is the query position, j the key position, both 0-based in one
packed sequence of length T; h is the query head (only the block-sparse mask depends
on it). ``visible`` is True where query i may attend to key j.
"""
from __future__ import annotations

import numpy as np


def _doc_of(cu: np.ndarray, x: np.ndarray) -> np.ndarray:
    # document index d with cu[d] <= x < cu[d+1]
    return np.searchsorted(cu, x, side="right") - 1


def visible(spec, i, j, h=None, keep=None, T=None):
    """Boolean array visible(i, j) (broadcast over i and j; h is a scalar head index).

    spec : masked_long_context_tiled_amd.inputs.MaskSpec (only its fields are read)
    keep : uint8 [Hq][nqb][nkb] keep matrix, block-sparse only (for variable_block:
           [Hq][n_row_blocks][n_col_blocks] over the spec's grid)
    T    : sequence length, needed by CAUSAL BLOCKWISE (its final block is the last
           ``final_block_len`` positions)
    """
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    k = spec.kind
    if k == "full":
        # every query sees every key
        return np.ones(np.broadcast(i, j).shape, dtype=bool)
    if k == "causal":
        # a query sees itself and the past
        return j <= i
    if k in ("full_document", "causal_document"):
        # sequence packing: a query sees only keys of its own document
        cu = np.asarray(spec.cu_seqlens, dtype=np.int64)
        same = _doc_of(cu, i) == _doc_of(cu, j)
        return same & (j <= i) if k == "causal_document" else same
    if k == "full_sliding_window":
        # keys within distance w-1 on either side
        return np.abs(i - j) < spec.window
    if k == "causal_sliding_window":
        # the w most recent keys, the query itself included
        return ((i - j) >= 0) & ((i - j) < spec.window)
    if k == "shared_question":
        # question causal within itself; each answer sees the whole question and
        # itself causally, never another answer
        Qn, A = spec.question_len, spec.answer_len
        ai = np.where(i >= Qn, (i - Qn) // A, -1)
        aj = np.where(j >= Qn, (j - Qn) // A, -1)
        return (j <= i) & ((j < Qn) | (ai == aj))
    if k == "prefix_lm_causal":
        # the prefix is bidirectional, the rest causal
        return (j < spec.prefix_len) | (j <= i)
    if k == "causal_blockwise":
        # causal within fixed blocks; the final block is causal over everything
        F = T - spec.final_block_len
        b = spec.block_len
        return (j <= i) & ((i >= F) | ((i // b) == (j // b)))
    if k == "global_sliding":
        # global tokens see and are seen by all; the rest see a window
        G = spec.global_len
        return (i < G) | (j < G) | (np.abs(i - j) < spec.window)
    if k == "prefix_lm_document":
        # per document: its first prefix_len positions bidirectional, the rest causal;
        # nothing across documents
        cu = np.asarray(spec.cu_seqlens, dtype=np.int64)
        dj = _doc_of(cu, j)
        same = _doc_of(cu, i) == dj
        return same & (((j - cu[dj]) < spec.prefix_len) | (j <= i))
    if k == "block_causal_document":
        # per document: blocks of block_len positions (counted from the document start)
        # see themselves fully and the earlier blocks of their document
        cu = np.asarray(spec.cu_seqlens, dtype=np.int64)
        di, dj = _doc_of(cu, i), _doc_of(cu, j)
        b = spec.block_len
        return (di == dj) & (((i - cu[di]) // b) >= ((j - cu[dj]) // b))
    if k == "block_sparse":
        # a (query block, key block) pair is visible iff kept for this head
        b = spec.sparse_block
        return keep[h][i // b, j // b].astype(bool)
    if k == "variable_block":
        # block-sparse over a grid of variable block sizes: row block r covers
        # [row_offsets[r], row_offsets[r+1]), column block c [col_offsets[c], col_offsets[c+1])
        rb = np.searchsorted(np.asarray(spec.row_offsets, dtype=np.int64), i, side="right") - 1
        cb = np.searchsorted(np.asarray(spec.col_offsets, dtype=np.int64), j, side="right") - 1
        return keep[h][rb, cb].astype(bool)
    raise ValueError(f"unknown mask kind {k!r}")


def mask_block(spec, T, rows, cols, h=0, keep=None):
    """Materialised boolean mask M[rows][cols] (rows, cols: 1-D index arrays or ranges)."""
    r = np.asarray(rows, dtype=np.int64)[:, None]
    c = np.asarray(cols, dtype=np.int64)[None, :]
    m = visible(spec, r, c, h=h, keep=keep, T=T)
    return np.broadcast_to(m, (r.shape[0], c.shape[1]))


def row_visible_counts(spec, T, h=0, keep=None, chunk=2048):
    """Number of visible keys of every query row (int64 [T])."""
    out = np.empty(T, dtype=np.int64)
    cols = np.arange(T)
    for r0 in range(0, T, chunk):
        rows = np.arange(r0, min(T, r0 + chunk))
        out[r0:r0 + len(rows)] = mask_block(spec, T, rows, cols, h, keep).sum(axis=1)
    return out


def visible_count(spec, T, h=0, keep=None, chunk=2048):
    """U = number of visible (query, key) pairs for head h: the sum of the mask."""
    return int(row_visible_counts(spec, T, h, keep, chunk).sum())
