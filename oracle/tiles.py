"""Tile classes and tile / block lists by brute force (oracle; test infrastructure only).

The benchmark pages ("LongCA-bench: 长上下文注意力基准测试", xllm-io blog, section 三
"稀疏注意力内核" and "动态掩码") describe block-sparse attention over uniform 64x64 or
128x128 blocks; skipping work on masked blocks is what those kernels exploit. Here the
same idea is checked at any tile shape:

  class(tile) = EMPTY   if no cell of the tile is visible
              = FULL    if every in-range cell of the tile is visible
              = PARTIAL otherwise

computed directly from the materialised mask. CSR lists every non-empty key tile of
each query-tile row in ascending order; CSC every non-empty query tile of each key
tile column. For a block-sparse keep matrix the lists are its non-zeros per row / per
column, ascending.
"""
from __future__ import annotations

import numpy as np

from .masks import mask_block

EMPTY, PARTIAL, FULL = 0, 1, 2


def tile_classes(spec, T, BM, BN, h=0, keep=None, rows_per_pass=None):
    """uint8 [ceil(T/BM)][ceil(T/BN)] class map from the materialised mask.

    The mask is materialised a few query tiles at a time (``rows_per_pass`` rows, a
    multiple of BM, by default enough for about 2^24 cells) and every tile is read in
    full: any visible cell makes it non-EMPTY, every in-range cell visible makes it FULL.
    Cells past T (the ragged last key tile) count as neither."""
    nqt = -(-T // BM)
    nkt = -(-T // BN)
    cls = np.empty((nqt, nkt), dtype=np.uint8)
    cols = np.arange(T)
    if rows_per_pass is None:
        rows_per_pass = max(BM, (1 << 24) // max(1, nkt * BN) // BM * BM)
    in_range = np.zeros(nkt * BN, dtype=bool)
    in_range[:T] = True
    for r0 in range(0, nqt * BM, rows_per_pass):
        r1 = min(T, r0 + rows_per_pass)
        rows = np.arange(r0, r1)
        vis = np.zeros((len(rows), nkt * BN), dtype=bool)
        vis[:, :T] = mask_block(spec, T, rows, cols, h, keep)
        nq = -(-len(rows) // BM)
        pad = nq * BM - len(rows)          # rows past T: neither visible nor required
        if pad:
            vis = np.concatenate([vis, np.zeros((pad, nkt * BN), dtype=bool)])
        row_in = np.zeros(nq * BM, dtype=bool)
        row_in[:len(rows)] = True
        cell_in = row_in[:, None] & in_range[None, :]
        shape = (nq, BM, nkt, BN)
        any_vis = vis.reshape(shape).any(axis=(1, 3))
        all_vis = (vis | ~cell_in).reshape(shape).all(axis=(1, 3))
        q0 = r0 // BM
        cls[q0:q0 + nq] = np.where(all_vis, FULL, np.where(any_vis, PARTIAL, EMPTY))
    return cls


def tile_csr(cls):
    """(row_ptr int32 [nqt+1], cols int32 [nnz], full uint8 [nnz]) from a class map."""
    ptr = [0]
    cols, full = [], []
    for r in range(cls.shape[0]):
        nz = np.nonzero(cls[r] != EMPTY)[0]
        cols.extend(nz.tolist())
        full.extend((cls[r, nz] == FULL).astype(np.uint8).tolist())
        ptr.append(len(cols))
    return (np.asarray(ptr, dtype=np.int32), np.asarray(cols, dtype=np.int32),
            np.asarray(full, dtype=np.uint8))


def tile_csc(cls):
    """(col_ptr int32 [nkt+1], rows int32 [nnz], full uint8 [nnz]) from a class map."""
    return tile_csr(np.ascontiguousarray(cls.T))


def keep_csr(keep_2d):
    """(row_ptr, cols) of a 2-D keep matrix, ascending."""
    ptr = [0]
    cols = []
    for r in range(keep_2d.shape[0]):
        nz = np.nonzero(keep_2d[r])[0]
        cols.extend(nz.tolist())
        ptr.append(len(cols))
    return np.asarray(ptr, dtype=np.int32), np.asarray(cols, dtype=np.int32)


def keep_csc(keep_2d):
    """(col_ptr, rows) of a 2-D keep matrix, ascending."""
    return keep_csr(np.ascontiguousarray(keep_2d.T))


def launch_order(ptr):
    """Launch order of a list set: list indices by descending length (ptr[i+1] - ptr[i]),
    equal lengths by ascending index."""
    lens = np.diff(np.asarray(ptr, dtype=np.int64))
    return np.asarray(sorted(range(len(lens)), key=lambda i: (-int(lens[i]), i)), dtype=np.int32)
