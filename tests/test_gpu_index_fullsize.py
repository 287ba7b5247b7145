"""Bit-exact tile index and block index at the workloads' full sizes.

Dense masks: the library builds the index on the GPU from its descriptor; its class
maps, CSR / CSC lists and launch orders are hashed and compared with the digests that
tests/golden/make_index_digests.py wrote from the oracle (oracle.tiles, brute force over
the materialised mask). These sizes take the index kernels' multi-chunk paths: lists of
more than 64 candidate tiles (ballot compaction over several chunks), more than 1024
lists (several elements per thread in the row-pointer scan) and more than 1024 items to
order (multi-chunk ranking; 4096 query tiles at 128K).

Block-sparse at 64K: the block index of the workloads' keep matrices (65,536 CSR lists at
b = 64) against the oracle's lists of the same keep matrix, compared array for array.
"""
import hashlib
import json
import os

import numpy as np
import pytest

from masked_long_context_tiled_amd import attn
from masked_long_context_tiled_amd.inputs import keep_for, workloads
from oracle.select import expand_variable_blocks
from oracle.tiles import keep_csc, keep_csr

from conftest import GOLDEN
from gpu_helpers import note

pytestmark = pytest.mark.gpu

with open(os.path.join(GOLDEN, "index_digests.json")) as _f:
    DIGESTS = json.load(_f)


def _digest(a, dtype):
    return hashlib.sha256(np.ascontiguousarray(a, dtype=dtype).tobytes()).hexdigest()


def _compare(tag, want, cls, ptr, ent, order):
    got = {"shape": list(cls.shape), "cls": _digest(cls, "u1"), "ptr": _digest(ptr, "<i4"),
           "idx": _digest(ent >> 1, "<i4"), "full": _digest(ent & 1, "u1"), "order": _digest(order, "<i4"),
           "nnz": int(ptr[-1]), "n_full": int((cls == 2).sum()), "n_partial": int((cls == 1).sum())}
    bad = [k for k in want if got[k] != want[k]]
    assert not bad, f"{tag}: sections differ from the oracle: {bad} (got {[got[k] for k in bad]})"


@pytest.mark.parametrize("name", sorted(DIGESTS))
def test_tile_index_full_size(name):
    import torch
    rec = DIGESTS[name]
    wl = workloads(0)[name]
    assert (wl.T, wl.Hq, wl.Hk) == (rec["T"], rec["Hq"], rec["Hk"])
    note(f"tile index full size {name}: T={wl.T} Hq={wl.Hq} Hk={wl.Hk}")
    ma = attn.MaskedAttention(wl.T, wl.Hq, wl.Hk, wl.mask)
    assert list(attn.query_tile_shape(ma.prob)) == rec["tiles"]
    torch.cuda.synchronize()
    sec = ma.index_sections()
    _compare(f"{name} forward", rec["fwd"], sec["fwd_cls"], sec["fwd_ptr"], sec["fwd_ent"], sec["fwd_order"])
    _compare(f"{name} backward", rec["bwd"], sec["bwd_cls"], sec["bwd_ptr"], sec["bwd_ent"], sec["bwd_order"])
    note(f"  fwd nnz {rec['fwd']['nnz']} of {np.prod(rec['fwd']['shape'])}, "
         f"bwd nnz {rec['bwd']['nnz']} of {np.prod(rec['bwd']['shape'])}: equal")


@pytest.mark.parametrize("name", ["block_sparse_64k_b128", "block_sparse_64k_b64", "variable_block_64k"])
def test_block_index_full_size(name):
    import torch
    wl = workloads(0)[name]
    keep = keep_for(wl, 0)
    ma = attn.MaskedAttention(wl.T, wl.Hq, wl.Hk, wl.mask, keep=keep)
    if wl.mask.kind == "variable_block":
        # the library runs the uniform 64-block mask the grid expands to: the oracle's expansion
        keep = expand_variable_blocks(keep, wl.mask.row_offsets, wl.mask.col_offsets)
    note(f"block index full size {name}: keep {keep.shape}")
    torch.cuda.synchronize()
    sec = ma.index_sections()
    Hq, nb = keep.shape[0], keep.shape[1]
    G = wl.Hq // wl.Hk
    ptr, cols = keep_csr(keep.reshape(Hq * nb, nb))
    assert np.array_equal(sec["fwd_ptr"], ptr), "CSR row pointers"
    assert np.array_equal(sec["fwd_ent"], cols), "CSR entries"
    # CSC over (g, kb): entries (h - g*G) * nb + qb of the group's heads, ascending
    want_ptr, want_ent = [np.zeros(1, dtype=np.int64)], []
    base = 0
    for g in range(wl.Hk):
        p, r = keep_csc(keep[g * G:(g + 1) * G].reshape(G * nb, nb))
        want_ptr.append(base + p[1:].astype(np.int64))
        want_ent.append(r)
        base += int(p[-1])
    assert np.array_equal(sec["bwd_ptr"], np.concatenate(want_ptr)), "CSC column pointers"
    assert np.array_equal(sec["bwd_ent"], np.concatenate(want_ent)), "CSC entries"
    note(f"  {Hq * nb} CSR lists, {wl.Hk * nb} CSC lists, nnz {int(ptr[-1])}: equal")
