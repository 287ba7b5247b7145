"""Pins for the oracle's tile classes and tile / block lists (CPU only).

Closed forms: under CAUSAL a tile [r0, r1) x [c0, c1) is EMPTY iff c0 > r1 - 1, FULL
iff c1 - 1 <= r0, else PARTIAL; under FULL every tile is FULL (ragged edge tiles
included); under a document mask a tile is FULL iff its rows and columns lie in one
document and EMPTY iff no row shares a document with a column. Lists are checked
against hand-written examples.
"""
import numpy as np
import pytest

from masked_long_context_tiled_amd.inputs import MaskSpec, document_cu_seqlens
from oracle.tiles import EMPTY, FULL, PARTIAL, keep_csc, keep_csr, launch_order, tile_classes, tile_csc, tile_csr


@pytest.mark.parametrize("T,BM,BN", [(256, 32, 64), (200, 32, 64), (512, 128, 128), (300, 64, 32), (100, 16, 16)])
@pytest.mark.parametrize("passes", [None, 1, 3])
def test_causal_closed_form(T, BM, BN, passes):
    # passes: query tiles materialised per pass (None = the default), so pass boundaries
    # fall inside and at the end of the ragged last tile
    cls = tile_classes(MaskSpec("causal"), T, BM, BN, rows_per_pass=None if passes is None else passes * BM)
    assert cls.shape == (-(-T // BM), -(-T // BN))
    for qt in range(cls.shape[0]):
        r0, r1 = qt * BM, min(T, (qt + 1) * BM)
        for kt in range(cls.shape[1]):
            c0, c1 = kt * BN, min(T, (kt + 1) * BN)
            want = EMPTY if c0 > r1 - 1 else (FULL if c1 - 1 <= r0 else PARTIAL)
            assert cls[qt, kt] == want, (qt, kt)


def test_full_all_full_including_ragged_edges():
    cls = tile_classes(MaskSpec("full"), 130, 32, 64)
    assert (cls == FULL).all()


def test_document_closed_form():
    T, BM, BN = 400, 32, 64
    cu = document_cu_seqlens(2, T, 40, 150)
    doc = np.searchsorted(np.asarray(cu), np.arange(T), side="right") - 1
    cls = tile_classes(MaskSpec("full_document", cu_seqlens=cu), T, BM, BN)
    for qt in range(cls.shape[0]):
        rd = set(doc[qt * BM:min(T, (qt + 1) * BM)].tolist())
        for kt in range(cls.shape[1]):
            cd = set(doc[kt * BN:min(T, (kt + 1) * BN)].tolist())
            if len(rd) == 1 and rd == cd:
                want = FULL
            elif rd & cd:
                want = PARTIAL
            else:
                want = EMPTY
            assert cls[qt, kt] == want


def test_lists_hand_example():
    cls = np.array([[2, 0, 1],
                    [0, 0, 0],
                    [1, 2, 2]], dtype=np.uint8)
    ptr, cols, full = tile_csr(cls)
    assert ptr.tolist() == [0, 2, 2, 5]
    assert cols.tolist() == [0, 2, 0, 1, 2]
    assert full.tolist() == [1, 0, 0, 1, 1]
    ptr, rows, full = tile_csc(cls)
    assert ptr.tolist() == [0, 2, 3, 5]
    assert rows.tolist() == [0, 2, 2, 0, 2]
    assert full.tolist() == [1, 0, 1, 0, 1]


def test_keep_lists_hand_example():
    keep = np.array([[1, 0, 1, 0],
                     [0, 1, 0, 0],
                     [1, 1, 1, 1]], dtype=np.uint8)
    ptr, cols = keep_csr(keep)
    assert ptr.tolist() == [0, 2, 3, 7] and cols.tolist() == [0, 2, 1, 0, 1, 2, 3]
    ptr, rows = keep_csc(keep)
    assert ptr.tolist() == [0, 2, 4, 6, 7] and rows.tolist() == [0, 2, 1, 2, 0, 2, 2]


def test_launch_order_hand_example():
    # lengths 2, 0, 3, 2, 3 -> the two 3s (ascending index), the two 2s, then the 0
    assert launch_order([0, 2, 2, 5, 7, 10]).tolist() == [2, 4, 0, 3, 1]
    assert launch_order([0]).tolist() == []


def test_sliding_window_closed_form_multi_pass():
    # FULL SLIDING WINDOW |i - j| < w: tile EMPTY iff its nearest cells are >= w apart,
    # FULL iff its farthest in-range cells are < w apart
    T, BM, BN, w = 333, 16, 32, 40
    cls = tile_classes(MaskSpec("full_sliding_window", window=w), T, BM, BN, rows_per_pass=2 * BM)
    for qt in range(cls.shape[0]):
        r0, r1 = qt * BM, min(T, (qt + 1) * BM) - 1
        for kt in range(cls.shape[1]):
            c0, c1 = kt * BN, min(T, (kt + 1) * BN) - 1
            near = max(0, c0 - r1, r0 - c1)
            far = max(abs(c1 - r0), abs(r1 - c0))
            want = EMPTY if near >= w else (FULL if far < w else PARTIAL)
            assert cls[qt, kt] == want, (qt, kt)
