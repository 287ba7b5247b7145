"""Host-side tests (no GPU) of the block selector's argument checks and of the
Variable Block expansion, which runs on the host: its output must equal the oracle's
expansion, and the expanded uniform mask must equal the variable-block predicate."""
import ctypes

import numpy as np
import pytest

from masked_long_context_tiled_amd import attn
from masked_long_context_tiled_amd.inputs import MaskSpec, variable_block_grid, variable_block_keep
from oracle.masks import mask_block
from oracle.select import expand_variable_blocks

FAKE = 0x1000   # never dereferenced: validation fails first


def _select(prob, params, ws_bytes=None, **null):
    L = attn.lib()
    ws = attn.block_select_workspace_size(prob) if ws_bytes is None else ws_bytes
    ptrs = {n: (None if null.get(n) else FAKE) for n in ("q", "k", "scores", "keep", "ws")}
    return L.attn_block_select(ctypes.byref(prob), ctypes.byref(params), ptrs["q"], ptrs["k"], ptrs["scores"],
                               ptrs["keep"], ptrs["ws"], ws, None)


def test_block_select_rejects_before_launch():
    sp = attn.problem(1000, 8, 2, "block_sparse", 64)
    ok = attn.block_select_params("topk", topk=4)
    ws = attn.block_select_workspace_size(sp)
    nb = -(-1000 // 64)
    assert ws >= (8 + 2) * nb * 128 * 4
    dense = attn.problem(1000, 8, 2, "causal")
    assert _select(dense, ok, ws_bytes=ws) == attn.ATTN_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert attn.lib().attn_block_select_workspace_size(ctypes.byref(dense), ctypes.byref(n)) == attn.ATTN_ERR_INVALID_ARG
    for bad in (attn.block_select_params("topk", topk=0), attn.block_select_params("topp", topp=0.0),
                attn.block_select_params("topp", topp=1.5), attn.attn_block_select_params(7, 1, 0.5, 1)):
        assert _select(sp, bad) == attn.ATTN_ERR_INVALID_ARG
    for name in ("q", "k", "scores", "keep", "ws"):
        assert _select(sp, ok, **{name: True}) == attn.ATTN_ERR_INVALID_ARG, name
    assert _select(sp, ok, ws_bytes=ws - 1) == attn.ATTN_ERR_WORKSPACE
    big = attn.problem(64 * 4097, 1, 1, "block_sparse", 64)       # 4097 blocks per row
    assert _select(big, ok, ws_bytes=1 << 40) == attn.ATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("T,seed", [(1000, 0), (4096, 1), (64, 2), (130, 3)])
def test_variable_block_expand_equals_oracle(T, seed):
    Hq = 3
    ro = variable_block_grid(seed, T)
    co = variable_block_grid(seed + 100, T)
    keep = variable_block_keep(seed, Hq, ro, co)
    got = attn.variable_block_expand(T, Hq, ro, co, keep)
    assert np.array_equal(got, expand_variable_blocks(keep, ro, co))
    if T <= 1000:
        spec = MaskSpec("variable_block", row_offsets=ro, col_offsets=co)
        uni = MaskSpec("block_sparse", sparse_block=64)
        for h in range(Hq):
            assert np.array_equal(mask_block(spec, T, range(T), range(T), h, keep),
                                  mask_block(uni, T, range(T), range(T), h, got))


def test_variable_block_expand_rejects_bad_edges():
    keep = np.ones((1, 2, 2), dtype=np.uint8)
    for ro in [(0, 100, 200), (0, 128, 190), (64, 128, 200), (0, 128, 128), (0, 192, 128)]:
        with pytest.raises(attn.AttnError) as ei:
            attn.variable_block_expand(200, 1, ro, (0, 64, 200), keep)
        assert ei.value.status == attn.ATTN_ERR_INVALID_ARG, ro
    assert attn.lib().attn_variable_block_expand(200, 1, None, 1, None, 1, None, None) == attn.ATTN_ERR_INVALID_ARG
