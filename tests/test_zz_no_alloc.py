"""attn_block_select_noalloc (the workspace-free variant of attn_block_select, for callers
that cannot allocate device memory) against attn_block_select: bit-identical scores and
keep matrices on two calls in a row through the C ABI, the second on a smaller problem
(the static array keeps the first call's contents, which must not leak into the second),
and the size limit rejected before any launch."""
import numpy as np
import pytest

from masked_long_context_tiled_amd import attn
from masked_long_context_tiled_amd.inputs import attention_inputs

from gpu_helpers import note, to_dev_bf16

pytestmark = pytest.mark.gpu


def _select_both(T, Hq, Hk, b, params, seed):
    import torch
    prob = attn.problem(T, Hq, Hk, "block_sparse", b)
    nb = -(-T // b)
    x = attention_inputs(seed, T, Hq, Hk, with_do=False)
    q, k = to_dev_bf16(x["q"], torch), to_dev_bf16(x["k"], torch)
    stream = torch.cuda.current_stream().cuda_stream
    out = []
    for noalloc in (False, True):
        scores = torch.full((Hq, nb, nb), float("nan"), dtype=torch.float32, device="cuda")
        keep = torch.full((Hq, nb, nb), 7, dtype=torch.uint8, device="cuda")
        if noalloc:
            attn.block_select_noalloc(prob, params, q.data_ptr(), k.data_ptr(), scores.data_ptr(),
                                      keep.data_ptr(), stream)
        else:
            nws = attn.block_select_workspace_size(prob)
            ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
            attn.block_select(prob, params, q.data_ptr(), k.data_ptr(), scores.data_ptr(), keep.data_ptr(),
                              ws.data_ptr(), nws, stream)
        torch.cuda.synchronize()
        out.append((scores.cpu().numpy(), keep.cpu().numpy()))
    return out


@pytest.mark.parametrize("mode", ["topk", "topp"])
def test_noalloc_matches_workspace_entry_point(mode):
    # first a large problem (fills most of the static array), then a smaller one
    for T, Hq, Hk, b, seed in ((24576, 64, 8, 64, 41), (3000, 16, 2, 128, 42)):
        nb = -(-T // b)
        params = attn.block_select_params(mode, topk=max(1, nb // 2), topp=0.6, keep_diagonal=True)
        note(f"no-alloc block select {mode}: T={T} Hq={Hq} Hk={Hk} b={b}")
        (s_ws, k_ws), (s_na, k_na) = _select_both(T, Hq, Hk, b, params, seed)
        assert np.array_equal(s_ws.view(np.uint32), s_na.view(np.uint32)), "scores differ"
        assert np.array_equal(k_ws, k_na), "keep matrices differ"
        assert set(np.unique(k_na).tolist()) <= {0, 1}


def test_noalloc_rejects_problems_beyond_the_static_array():
    import ctypes
    prob = attn.problem(65536, 64, 8, "block_sparse", 64)          # 37.7 MB of block means
    assert attn.block_select_workspace_size(prob) > (32 << 20)
    params = attn.block_select_params("topk", topk=4)
    fake = ctypes.c_void_p(256)                                     # never dereferenced: rejected first
    st = attn.lib().attn_block_select_noalloc(ctypes.byref(prob), ctypes.byref(params), fake, fake, fake, fake,
                                              None)
    assert st == attn.ATTN_ERR_WORKSPACE
