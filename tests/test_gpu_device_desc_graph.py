"""The device-built column-interval descriptor and HIP-graph replay of a whole step.

* attn_mask_desc_build_device writes, bit for bit, the descriptor of the host builder
  (itself checked against the oracle's per-element predicate on the CPU) for every interval
  mask kind at a ragged T and at the workloads' full sizes.
* One step (device descriptor, tile index, forward, backward preprocess, dK/dV, dQ)
  captured into a HIP graph and replayed several times, with eager library work and
  synchronisations between the replays, gives after every replay exactly the outputs of the
  same step launched eagerly (every kernel is deterministic)."""
import numpy as np
import pytest

from masked_long_context_tiled_amd import attn
from masked_long_context_tiled_amd.inputs import MaskSpec, attention_inputs, document_cu_seqlens, workloads

from gpu_helpers import note, to_dev_bf16

pytestmark = pytest.mark.gpu


def _specs(T):
    return [
        MaskSpec("full"), MaskSpec("causal"),
        MaskSpec("full_document", cu_seqlens=document_cu_seqlens(3, T, 64, 400)),
        MaskSpec("causal_document", cu_seqlens=document_cu_seqlens(4, T, 64, 400)),
        MaskSpec("full_sliding_window", window=130), MaskSpec("causal_sliding_window", window=130),
        MaskSpec("shared_question", question_len=T - 4 * 220, answer_len=220, n_answers=4),
        MaskSpec("prefix_lm_causal", prefix_len=250),
        MaskSpec("causal_blockwise", block_len=64, final_block_len=T - 12 * 64),
        MaskSpec("global_sliding", global_len=8, window=128),
        MaskSpec("prefix_lm_document", prefix_len=70, cu_seqlens=document_cu_seqlens(5, T, 64, 400)),
        MaskSpec("block_causal_document", block_len=48, cu_seqlens=document_cu_seqlens(6, T, 64, 400)),
    ]


def _device_desc(spec, T):
    import torch
    cu = torch.tensor(spec.cu_seqlens, dtype=torch.int32, device="cuda") if spec.cu_seqlens else None
    out = torch.full((T, 4), -7, dtype=torch.int32, device="cuda")
    attn.mask_desc_build_device(spec, T, 0 if cu is None else cu.data_ptr(), out.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("idx", range(12))
def test_device_descriptor_equals_host(idx):
    T = 1000
    spec = _specs(T)[idx]
    note(f"device descriptor {spec.kind} T={T}")
    assert np.array_equal(_device_desc(spec, T), attn.mask_desc_build(spec, T))


def test_device_descriptor_full_size():
    for name, wl in workloads(0).items():
        if wl.mask.kind in ("block_sparse", "variable_block") or wl.T < 8192:
            continue
        note(f"device descriptor {name} T={wl.T}")
        assert np.array_equal(_device_desc(wl.mask, wl.T), attn.mask_desc_build(wl.mask, wl.T)), name


@pytest.mark.parametrize("kind", ["causal", "causal_document"])
def test_graph_replay_of_a_step(kind):
    import torch
    T, Hq, Hk = 1000, 8, 2
    spec = MaskSpec("causal") if kind == "causal" else \
        MaskSpec("causal_document", cu_seqlens=document_cu_seqlens(40, T, 64, 400))
    note(f"graph replay {kind} T={T}")
    x = attention_inputs(41, T, Hq, Hk)
    q, k, v, do = (to_dev_bf16(x[n], torch) for n in ("q", "k", "v", "do"))
    prob = attn.problem(T, Hq, Hk, spec.kind)
    nidx = attn.tile_index_size(prob)
    nws = attn.bwd_workspace_size(prob)
    cu = torch.tensor(spec.cu_seqlens, dtype=torch.int32, device="cuda") if spec.cu_seqlens else None
    bufs = {"desc": torch.empty((T, 4), dtype=torch.int32, device="cuda"),
            "index": torch.empty(nidx, dtype=torch.uint8, device="cuda"),
            "ws": torch.empty(nws, dtype=torch.uint8, device="cuda"),
            "o": torch.empty((T, Hq, 128), dtype=torch.bfloat16, device="cuda"),
            "o_lo": torch.empty((T, Hq, 128), dtype=torch.bfloat16, device="cuda"),
            "lse": torch.empty((Hq, T), dtype=torch.float32, device="cuda"),
            "dq": torch.empty((T, Hq, 128), dtype=torch.float32, device="cuda"),
            "dk": torch.empty((T, Hk, 128), dtype=torch.float32, device="cuda"),
            "dv": torch.empty((T, Hk, 128), dtype=torch.float32, device="cuda")}
    b = {n: t.data_ptr() for n, t in bufs.items()}

    def step():
        sp = torch.cuda.current_stream().cuda_stream
        attn.mask_desc_build_device(spec, T, 0 if cu is None else cu.data_ptr(), b["desc"], sp)
        attn.tile_index_build(prob, b["desc"], b["index"], nidx, sp)
        attn.fwd(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), b["o"], b["o_lo"], b["lse"], b["desc"],
                 b["index"], nidx, 0, 0, sp)
        attn.bwd(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), b["o"], b["o_lo"], b["lse"], do.data_ptr(),
                 b["dq"], b["dk"], b["dv"], b["desc"], b["index"], nidx, b["ws"], nws, sp)

    L = attn.tile_index_layout(prob)
    nf, nbk = L["nqt_f"] * L["nkt_f"], L["nqt_b"] * L["nkt_b"]

    def snapshot():
        # outputs, descriptor and the defined sections of the index (its alignment gaps and
        # the unused tails of the entry arrays are never written)
        torch.cuda.synchronize()
        out = {n: bufs[n].clone() for n in ("desc", "o", "o_lo", "lse", "dq", "dk", "dv")}
        raw = bufs["index"]
        i32 = lambda off, n: raw[off:off + 4 * n].view(torch.int32).clone()
        out["fwd_cls"] = raw[L["fwd_cls"]:L["fwd_cls"] + nf].clone()
        out["bwd_cls"] = raw[L["bwd_cls"]:L["bwd_cls"] + nbk].clone()
        out["fwd_ptr"] = i32(L["fwd_ptr"], L["nqt_f"] + 1)
        out["bwd_ptr"] = i32(L["bwd_ptr"], L["nkt_b"] + 1)
        out["fwd_ent"] = i32(L["fwd_ent"], int(out["fwd_ptr"][-1]))
        out["bwd_ent"] = i32(L["bwd_ent"], int(out["bwd_ptr"][-1]))
        out["fwd_order"] = i32(L["fwd_order"], L["nqt_f"])
        out["bwd_order"] = i32(L["bwd_order"], L["nkt_b"])
        return out

    def clobber():
        for n, t in bufs.items():
            t.zero_() if t.dtype != torch.int32 else t.fill_(-1)

    step()
    want = snapshot()
    graph = torch.cuda.CUDAGraph()
    clobber()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        clobber()
        graph.replay()
        got = snapshot()
        for n in want:
            assert torch.equal(got[n], want[n]), f"replay {rep}: {n} differs from the eager step"
        step()                                  # eager library work between the replays
        torch.cuda.synchronize()
