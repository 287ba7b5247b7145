"""C-ABI tests that need no GPU: the library loads and exports every function of
include/attn.h, argument validation returns the documented status before any launch,
and the host column-interval descriptor equals the oracle's per-element predicate
bit for bit."""
import ctypes

import numpy as np
import pytest

from masked_long_context_tiled_amd import attn
from masked_long_context_tiled_amd.inputs import MASK_KINDS, MaskSpec, document_cu_seqlens, workloads
from oracle.masks import mask_block


def test_library_exports_every_header_function():
    names = attn.header_functions()
    assert len(names) >= 12
    L = attn.lib()
    for n in names:
        assert hasattr(L, n), n
    # the binding wraps every declared function
    assert set(names) == set(attn._SIGS)


def test_status_strings():
    assert attn.status_string(0) == "ATTN_OK"
    assert attn.status_string(3) == "ATTN_ERR_WORKSPACE"
    assert attn.status_string(99) == "ATTN_ERR_UNKNOWN"


def _status(fn, *args):
    return fn(*args)


def test_problem_validation():
    L = attn.lib()
    n = ctypes.c_size_t()
    ok = attn.problem(1024, 8, 2, "causal")
    assert L.attn_tile_index_size(ctypes.byref(ok), ctypes.byref(n)) == attn.ATTN_OK and n.value > 0
    cases = [
        (attn.problem(1024, 6, 4, "causal"), attn.ATTN_ERR_INVALID_ARG),      # Hq % Hk != 0
        (attn.problem(1024, 6, 2, "causal"), attn.ATTN_ERR_UNSUPPORTED),      # G = 3
        (attn.problem(1024, 8, 2, "causal", head_dim=64), attn.ATTN_ERR_UNSUPPORTED),
        (attn.problem(0, 8, 2, "causal"), attn.ATTN_ERR_INVALID_ARG),
        (attn.problem(1024, 8, 2, 13), attn.ATTN_ERR_INVALID_ARG),            # unknown kind
        (attn.problem(1024, 8, 2, "block_sparse", 32), attn.ATTN_ERR_UNSUPPORTED),
        (attn.problem(1024, 512, 1, "causal"), attn.ATTN_ERR_UNSUPPORTED),    # G > 256
    ]
    for p, want in cases:
        assert L.attn_tile_index_size(ctypes.byref(p), ctypes.byref(n)) == want
    assert L.attn_tile_index_size(None, ctypes.byref(n)) == attn.ATTN_ERR_INVALID_ARG


def test_entry_points_reject_before_launch():
    """Every error path returns before touching the GPU (this host has none)."""
    L = attn.lib()
    p = attn.problem(1024, 8, 2, "causal")
    need = attn.tile_index_size(p)
    fake = 0x1000   # never dereferenced: validation fails first
    # null input pointer
    assert L.attn_fwd(ctypes.byref(p), None, fake, fake, fake, None, fake, fake, fake, need, None, 0, None) == attn.ATTN_ERR_INVALID_ARG
    # missing descriptor for an interval mask
    assert L.attn_fwd(ctypes.byref(p), fake, fake, fake, fake, None, fake, None, fake, need, None, 0, None) == attn.ATTN_ERR_INVALID_ARG
    # index buffer too small
    assert L.attn_fwd(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, fake, need - 1, None, 0, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_tile_index_build(ctypes.byref(p), fake, fake, need - 1, None) == attn.ATTN_ERR_WORKSPACE
    # backward workspace missing / too small
    ws = attn.bwd_workspace_size(p)
    assert ws >= 8 * 1024 * 4 + 16
    args = [fake] * 4 + [None] + [fake] * 6   # q k v o | o_lo | lse dout dq dk dv desc
    assert L.attn_bwd(ctypes.byref(p), *args, fake, need, None, 0, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_bwd(ctypes.byref(p), *args, fake, need, fake, ws - 1, None) == attn.ATTN_ERR_WORKSPACE
    # block index on a dense problem, tile index on a sparse problem
    assert L.attn_block_index_build(ctypes.byref(p), fake, fake, need, None) == attn.ATTN_ERR_INVALID_ARG
    sp = attn.problem(1024, 8, 2, "block_sparse", 64)
    assert L.attn_tile_index_build(ctypes.byref(sp), fake, fake, attn.tile_index_size(sp), None) == attn.ATTN_ERR_INVALID_ARG
    assert L.attn_query_tile_shape(ctypes.byref(sp), *([ctypes.byref(ctypes.c_int32())] * 4)) == attn.ATTN_ERR_INVALID_ARG
    assert L.attn_bwd_preprocess(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, ws - 1, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_bwd_preprocess(ctypes.byref(p), None, fake, fake, fake, None, fake, fake, ws, None) == attn.ATTN_ERR_INVALID_ARG
    assert L.attn_bwd_main(ctypes.byref(p), *([fake] * 9), fake, need, fake, ws - 1, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_cast_bf16(None, fake, 10, None) == attn.ATTN_ERR_INVALID_ARG
    assert L.attn_cast_bf16(None, None, 0, None) == attn.ATTN_OK


def test_mask_param_validation():
    bad = [
        (MaskSpec("full_sliding_window", window=0), 64),
        (MaskSpec("global_sliding", global_len=4, window=0), 64),
        (MaskSpec("full_document", cu_seqlens=(0, 10, 10, 64)), 64),     # empty document
        (MaskSpec("full_document", cu_seqlens=(0, 10, 60)), 64),         # does not end at T
        (MaskSpec("causal_document", cu_seqlens=(1, 64)), 64),           # does not start at 0
        (MaskSpec("shared_question", question_len=16, answer_len=16, n_answers=2), 64),
        (MaskSpec("prefix_lm_causal", prefix_len=65), 64),
        (MaskSpec("causal_blockwise", block_len=0, final_block_len=8), 64),
        (MaskSpec("causal_blockwise", block_len=8, final_block_len=65), 64),
        (MaskSpec("block_sparse", sparse_block=64), 64),                 # no descriptor
        (MaskSpec("prefix_lm_document", prefix_len=-1, cu_seqlens=(0, 64)), 64),
        (MaskSpec("block_causal_document", block_len=0, cu_seqlens=(0, 64)), 64),
        (MaskSpec("block_causal_document", block_len=4, cu_seqlens=(0, 70)), 64),  # does not end at T
    ]
    for spec, T in bad:
        with pytest.raises(attn.AttnError) as ei:
            attn.mask_desc_build(spec, T)
        assert ei.value.status == attn.ATTN_ERR_INVALID_ARG, spec
    p, _ = attn.mask_params(MaskSpec("causal"))
    assert attn.lib().attn_mask_desc_build(ctypes.byref(p), 16, None) == attn.ATTN_ERR_INVALID_ARG


def test_tile_shapes_and_layout():
    for G, bm in ((1, 256), (4, 64), (8, 32), (16, 16)):
        p = attn.problem(8192, 64, 64 // G, "causal")
        assert attn.query_tile_shape(p) == (bm, 64, bm, 128)
        lay = attn.tile_index_layout(p)
        assert lay["nqt_f"] == 8192 // bm and lay["nkt_f"] == 128 and lay["nkt_b"] == 64
        offs = sorted(lay[k] for k in ("fwd_cls", "fwd_ptr", "fwd_ent", "fwd_order",
                                        "bwd_cls", "bwd_ptr", "bwd_ent", "bwd_order"))
        assert all(o % 256 == 0 for o in offs) and len(set(offs)) == 8
        assert lay["total_bytes"] == attn.tile_index_size(p)
    sp = attn.problem(65536, 64, 8, "block_sparse", 64)
    lay = attn.tile_index_layout(sp)
    assert lay["nqt_f"] == 64 * 1024 and lay["nqt_b"] == 8 * 1024


# --- descriptor == predicate ---------------------------------------------------------

def _desc_dense(desc, rows):
    r = np.asarray(rows)[:, None]
    a0, b0, a1, b1 = (desc[:, i][None, :] for i in range(4))
    return ((r >= a0) & (r < b0)) | ((r >= a1) & (r < b1))


def _small_specs(T):
    return [
        MaskSpec("full"), MaskSpec("causal"),
        MaskSpec("full_document", cu_seqlens=document_cu_seqlens(1, T, 20, 200)),
        MaskSpec("causal_document", cu_seqlens=document_cu_seqlens(2, T, 20, 200)),
        MaskSpec("full_sliding_window", window=37), MaskSpec("full_sliding_window", window=1),
        MaskSpec("full_sliding_window", window=5 * T),
        MaskSpec("causal_sliding_window", window=53), MaskSpec("causal_sliding_window", window=1),
        MaskSpec("shared_question", question_len=100, answer_len=(T - 100) // 4, n_answers=4),
        MaskSpec("shared_question", question_len=0, answer_len=T, n_answers=1),
        MaskSpec("prefix_lm_causal", prefix_len=77), MaskSpec("prefix_lm_causal", prefix_len=0),
        MaskSpec("prefix_lm_causal", prefix_len=T),
        MaskSpec("causal_blockwise", block_len=64, final_block_len=128),
        MaskSpec("causal_blockwise", block_len=50, final_block_len=100),   # final block not block-aligned
        MaskSpec("causal_blockwise", block_len=64, final_block_len=0),
        MaskSpec("causal_blockwise", block_len=64, final_block_len=T),
        MaskSpec("global_sliding", global_len=16, window=40), MaskSpec("global_sliding", global_len=0, window=40),
        MaskSpec("global_sliding", global_len=60, window=30), MaskSpec("global_sliding", global_len=T, window=3),
        MaskSpec("prefix_lm_document", prefix_len=30, cu_seqlens=document_cu_seqlens(6, T, 20, 200)),
        MaskSpec("prefix_lm_document", prefix_len=0, cu_seqlens=document_cu_seqlens(7, T, 20, 200)),
        MaskSpec("prefix_lm_document", prefix_len=10 * T, cu_seqlens=document_cu_seqlens(8, T, 20, 200)),
        MaskSpec("block_causal_document", block_len=16, cu_seqlens=document_cu_seqlens(9, T, 20, 200)),
        MaskSpec("block_causal_document", block_len=1, cu_seqlens=document_cu_seqlens(10, T, 20, 200)),
        MaskSpec("block_causal_document", block_len=7 * T, cu_seqlens=document_cu_seqlens(11, T, 20, 200)),
    ]


@pytest.mark.parametrize("T", [500, 1024])
def test_desc_equals_predicate_small(T):
    rows = np.arange(T)
    for spec in _small_specs(T):
        desc = attn.mask_desc_build(spec, T)
        a0, b0, a1, b1 = desc.T
        assert np.all((0 <= a0) & (a0 <= b0) & (b0 <= a1) & (a1 <= b1) & (b1 <= T)) or \
            np.all(((a1 == 0) & (b1 == 0)) | (b0 <= a1)), spec
        got = _desc_dense(desc, rows)
        want = mask_block(spec, T, rows, np.arange(T))
        assert np.array_equal(got, want), spec


def test_every_interval_kind_covered():
    kinds = {s.kind for s in _small_specs(512)}
    assert kinds == set(MASK_KINDS) - {"block_sparse"}


@pytest.mark.parametrize("name", [n for n, w in workloads(0).items()
                                  if w.mask.kind != "block_sparse" and w.T <= 32768])
def test_desc_equals_predicate_workloads(name):
    wl = workloads(0)[name]
    desc = attn.mask_desc_build(wl.mask, wl.T)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.integers(0, wl.T, 200), [0, 1, wl.T - 1],
                                     np.arange(0, wl.T, max(1, wl.T // 64))]))
    got = _desc_dense(desc, rows)
    want = mask_block(wl.mask, wl.T, rows, np.arange(wl.T))
    assert np.array_equal(got, want)


def test_block_select_noalloc_rejects_beyond_static_array():
    # 64 query heads at T = 64K with b = 64 need 37.7 MB of block means, more than the 32 MiB
    # static array: rejected before any device call (no GPU needed)
    prob = attn.problem(65536, 64, 8, "block_sparse", 64)
    assert attn.block_select_workspace_size(prob) > (32 << 20)
    params = attn.block_select_params("topk", topk=4)
    fake = ctypes.c_void_p(256)
    L = attn.lib()
    assert L.attn_block_select_noalloc(ctypes.byref(prob), ctypes.byref(params), fake, fake, fake, fake,
                                       None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_block_select_noalloc(ctypes.byref(prob), None, fake, fake, fake, fake,
                                       None) == attn.ATTN_ERR_INVALID_ARG


def test_device_descriptor_validation_without_launch():
    L = attn.lib()
    p, keep = attn.mask_params(MaskSpec("causal_document", cu_seqlens=(0, 10, 20)))
    fake = ctypes.c_void_p(256)
    # a DOCUMENT kind without the device copy of cu_seqlens, and a null output: rejected first
    assert L.attn_mask_desc_build_device(ctypes.byref(p), 20, None, fake, None) == attn.ATTN_ERR_INVALID_ARG
    assert L.attn_mask_desc_build_device(ctypes.byref(p), 20, fake, None, None) == attn.ATTN_ERR_INVALID_ARG
    # cu_seqlens not ending at T (validated on the host copy)
    assert L.attn_mask_desc_build_device(ctypes.byref(p), 21, fake, fake, None) == attn.ATTN_ERR_INVALID_ARG


def _split_count(T, Hq, Hk):
    """Pieces per dense dK/dV key tile the library chose, read off attn_bwd_workspace_size:
    D [Hq][T] fp32, 256 bytes of bounds, fp16 Q and dO [T][Hq][128], fp16 K and V [T][Hk][128]
    (each part 256-byte aligned), then with S > 1 pieces their fp32 partial dK and dV."""
    a256 = lambda n: (n + 255) // 256 * 256
    base = a256(Hq * T * 4) + 256 + 2 * a256(T * Hq * 128 * 2) + 2 * a256(T * Hk * 128 * 2)
    extra = attn.bwd_workspace_size(attn.problem(T, Hq, Hk, "causal")) - base
    if extra == 0:
        return 1
    per_piece = 2 * T * Hk * 128 * 4
    S = extra // per_piece
    assert extra == a256(S * per_piece), (extra, per_piece)
    return S


@pytest.mark.parametrize("T, Hq, Hk, S", [
    (8192, 64, 8, 1),     # 8 KV heads x 64 key tiles of 128 = 512 work items: no split
    (4096, 64, 8, 2),     # 256 -> 2 pieces
    (2048, 64, 8, 4),     # 128 -> 4
    (1024, 64, 8, 8),     # 64 -> 8 (the cap)
    (512, 4, 1, 8),       # 4 -> capped at 8
    (1024, 64, 64, 1),    # MHA: 64 x 8 = 512
    (1024, 32, 32, 2),
    (1000, 32, 16, 4),    # ragged: 8 key tiles of which the last is short
])
def test_dense_dkdv_split_count(T, Hq, Hk, S):
    """Short sequences cut each dense key tile's query list into S pieces, the smallest power
    of two up to 8 giving at least 512 dK/dV work items; the workspace grows by their
    partial sums."""
    assert _split_count(T, Hq, Hk) == S
