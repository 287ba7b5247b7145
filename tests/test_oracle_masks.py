"""Pins for the oracle's mask predicates and its visible-pair count U.

* hand-drawn 12x12 fixtures (tests/golden/masks_T12.txt), one per mask kind;
* per-row visible counts from interval arithmetic written here, independent of the
  predicate code, at the workload parameters;
* closed forms of U (FULL T^2, CAUSAL T(T+1)/2, sliding windows, documents, shared
  question, prefix LM, causal blockwise);
* the reductions between masks (window >= T, empty/whole prefix, one answer, one
  final block, no global tokens, block-sparse at full density).
"""
import numpy as np
import pytest

from masked_long_context_tiled_amd.inputs import MaskSpec, document_cu_seqlens, workloads
from oracle.masks import mask_block, row_visible_counts, visible_count

from conftest import load_golden_masks


def _dense(spec, T, keep=None, h=0):
    return mask_block(spec, T, np.arange(T), np.arange(T), h, keep).astype(np.uint8)


@pytest.mark.parametrize("case", load_golden_masks(), ids=lambda c: c[0].kind)
def test_golden_mask_T12(case):
    spec, keep, want = case
    got = _dense(spec, 12, keep)
    assert np.array_equal(got, want), f"\n{got}\n!=\n{want}"


def test_golden_covers_every_kind():
    from masked_long_context_tiled_amd.inputs import MASK_KINDS
    kinds = {c[0].kind for c in load_golden_masks()}
    assert kinds == set(MASK_KINDS)


# --- per-row counts from interval arithmetic --------------------------------------

def _row_counts_intervals(spec, T):
    """Visible keys per query row, from the row's key intervals (written independently)."""
    out = np.zeros(T, dtype=np.int64)
    for i in range(T):
        k = spec.kind
        if k == "full":
            n = T
        elif k == "causal":
            n = i + 1
        elif k in ("full_document", "causal_document"):
            cu = spec.cu_seqlens
            d = max(x for x in range(len(cu) - 1) if cu[x] <= i)
            n = (cu[d + 1] - cu[d]) if k == "full_document" else (i - cu[d] + 1)
        elif k == "full_sliding_window":
            n = min(T, i + spec.window) - max(0, i - spec.window + 1)
        elif k == "causal_sliding_window":
            n = i - max(0, i - spec.window + 1) + 1
        elif k == "shared_question":
            Qn, A = spec.question_len, spec.answer_len
            n = i + 1 if i < Qn else Qn + (i - (Qn + ((i - Qn) // A) * A) + 1)
        elif k == "prefix_lm_causal":
            n = max(spec.prefix_len, i + 1)
        elif k == "causal_blockwise":
            F = T - spec.final_block_len
            n = i + 1 if i >= F else i - (i // spec.block_len) * spec.block_len + 1
        elif k == "global_sliding":
            G, w = spec.global_len, spec.window
            if i < G:
                n = T
            else:
                lo, hi = max(G, i - w + 1), min(T, i + w)   # window part beyond the globals
                n = G + max(0, hi - lo)
        elif k == "prefix_lm_document":
            cu = spec.cu_seqlens
            d = max(x for x in range(len(cu) - 1) if cu[x] <= i)
            Pd = min(spec.prefix_len, cu[d + 1] - cu[d])     # this document's prefix
            n = max(Pd, i - cu[d] + 1)
        elif k == "block_causal_document":
            cu = spec.cu_seqlens
            d = max(x for x in range(len(cu) - 1) if cu[x] <= i)
            b = spec.block_len
            end_of_block = cu[d] + ((i - cu[d]) // b + 1) * b
            n = min(cu[d + 1], end_of_block) - cu[d]
        else:
            raise AssertionError(k)
        out[i] = n
    return out


@pytest.mark.parametrize("name", [
    "full_document_32k", "causal_document_32k", "full_sliding_window_32k",
    "causal_sliding_window_32k", "shared_question_16k", "prefix_lm_causal_16k",
    "causal_blockwise_16k", "global_sliding_16k", "causal_8k_gqa", "full_8k_gqa",
    "prefix_lm_document_32k", "block_causal_document_32k"])
def test_row_counts_at_workload_params(name):
    wl = workloads(0)[name]
    spec, T = wl.mask, wl.T
    got = row_visible_counts(spec, T)
    want = _row_counts_intervals(spec, T)
    assert np.array_equal(got, want)
    # no configured mask leaves a query row without a visible key
    assert want.min() >= 1


# --- closed forms of U ----------------------------------------------------------

def test_U_closed_forms():
    T = 4096
    assert visible_count(MaskSpec("full"), T) == T * T
    assert visible_count(MaskSpec("causal"), T) == T * (T + 1) // 2
    w = 700
    assert visible_count(MaskSpec("causal_sliding_window", window=w), T) == w * (w + 1) // 2 + (T - w) * w
    assert visible_count(MaskSpec("full_sliding_window", window=w), T) == T * (2 * w - 1) - w * (w - 1)
    cu = document_cu_seqlens(3, T, 100, 900)
    L = np.diff(cu)
    assert visible_count(MaskSpec("full_document", cu_seqlens=cu), T) == int((L * L).sum())
    assert visible_count(MaskSpec("causal_document", cu_seqlens=cu), T) == int((L * (L + 1) // 2).sum())
    Qn, A, n = 512, 896, 4
    assert visible_count(MaskSpec("shared_question", question_len=Qn, answer_len=A, n_answers=n), T) \
        == Qn * (Qn + 1) // 2 + n * (A * Qn + A * (A + 1) // 2)
    P = 1024
    assert visible_count(MaskSpec("prefix_lm_causal", prefix_len=P), T) == P * P + (T * (T + 1) - P * (P + 1)) // 2
    b, Fl = 256, 512
    F = T - Fl
    assert visible_count(MaskSpec("causal_blockwise", block_len=b, final_block_len=Fl), T) \
        == (F // b) * b * (b + 1) // 2 + (T * (T + 1) - F * (F + 1)) // 2


def test_U_closed_forms_document_heterogeneous():
    T = 4096
    cu = document_cu_seqlens(5, T, 100, 900)
    L = np.diff(cu).astype(np.int64)
    P = 300
    Pd = np.minimum(P, L)
    # per document: the prefix block Pd x Pd, then row t >= Pd sees t + 1 keys
    want = int((Pd * Pd + (L * (L + 1) - Pd * (Pd + 1)) // 2).sum())
    assert visible_count(MaskSpec("prefix_lm_document", prefix_len=P, cu_seqlens=cu), T) == want
    b = 64
    # per document: block k (length m_k) sees the m_k keys of itself plus all earlier ones
    tot = 0
    for n in L:
        starts = np.arange(0, n, b)
        m = np.minimum(b, n - starts)
        tot += int((m * (starts + m)).sum())
    assert visible_count(MaskSpec("block_causal_document", block_len=b, cu_seqlens=cu), T) == tot


def test_U_headline_causal_8k():
    # CAUSAL at T = 8192: T(T+1)/2 pairs per head
    assert visible_count(MaskSpec("causal"), 8192) == 33_558_528


# --- reductions between masks ------------------------------------------------------

def test_reductions():
    T = 96
    full, causal = _dense(MaskSpec("full"), T), _dense(MaskSpec("causal"), T)
    assert np.array_equal(_dense(MaskSpec("full_sliding_window", window=T), T), full)
    assert np.array_equal(_dense(MaskSpec("causal_sliding_window", window=T), T), causal)
    assert np.array_equal(_dense(MaskSpec("prefix_lm_causal", prefix_len=0), T), causal)
    assert np.array_equal(_dense(MaskSpec("prefix_lm_causal", prefix_len=T), T), full)
    assert np.array_equal(_dense(MaskSpec("shared_question", question_len=32, answer_len=64, n_answers=1), T), causal)
    assert np.array_equal(_dense(MaskSpec("causal_blockwise", block_len=16, final_block_len=T), T), causal)
    assert np.array_equal(_dense(MaskSpec("full_document", cu_seqlens=(0, T)), T), full)
    assert np.array_equal(_dense(MaskSpec("causal_document", cu_seqlens=(0, T)), T), causal)
    cu = (0, 20, 57, T)
    fd, cd = _dense(MaskSpec("full_document", cu_seqlens=cu), T), _dense(MaskSpec("causal_document", cu_seqlens=cu), T)
    assert np.array_equal(_dense(MaskSpec("prefix_lm_document", prefix_len=0, cu_seqlens=cu), T), cd)
    assert np.array_equal(_dense(MaskSpec("prefix_lm_document", prefix_len=T, cu_seqlens=cu), T), fd)
    assert np.array_equal(_dense(MaskSpec("prefix_lm_document", prefix_len=7, cu_seqlens=(0, T)), T),
                          _dense(MaskSpec("prefix_lm_causal", prefix_len=7), T))
    assert np.array_equal(_dense(MaskSpec("block_causal_document", block_len=1, cu_seqlens=cu), T), cd)
    assert np.array_equal(_dense(MaskSpec("block_causal_document", block_len=T, cu_seqlens=cu), T), fd)
    w = 9
    assert np.array_equal(_dense(MaskSpec("global_sliding", global_len=0, window=w), T),
                          _dense(MaskSpec("full_sliding_window", window=w), T))
    keep = np.ones((1, 6, 6), dtype=np.uint8)
    assert np.array_equal(_dense(MaskSpec("block_sparse", sparse_block=16), T, keep), full)
