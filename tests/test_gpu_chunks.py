"""GPU parity of the context-parallel building block: a sequence split into chunks, every
(query chunk, key chunk) pair run as its own problem with attn_mask_desc_build_chunk, the
partial forwards merged with attn_lse_merge in ring order, and the backward shares of
every pair (given the merged O, O_lo, LSE) summed. The result must match the fp64 oracle
of the whole sequence to the same bounds as the plain path."""
import numpy as np
import pytest

from masked_long_context_tiled_amd import attn
from masked_long_context_tiled_amd.inputs import MaskSpec, attention_inputs, document_cu_seqlens
from oracle.attention import attention_backward

from gpu_helpers import LSE_TOL, TOL, assert_close, bf16_dev_to_f64, note, oracle_inputs, to_dev_bf16

pytestmark = pytest.mark.gpu


def _specs(T):
    return [
        MaskSpec("causal"),
        MaskSpec("causal_document", cu_seqlens=document_cu_seqlens(3, T, 64, 400)),
        MaskSpec("shared_question", question_len=T - 3 * 300, answer_len=300, n_answers=3),
        MaskSpec("global_sliding", global_len=8, window=160),
        MaskSpec("block_causal_document", block_len=48, cu_seqlens=document_cu_seqlens(6, T, 64, 400)),
    ]


@pytest.mark.parametrize("idx", range(5))
def test_ring_chunks_match_whole_sequence(idx):
    import torch
    T, n, Hq, Hk = 1536, 512, 8, 2
    nc = T // n
    spec = _specs(T)[idx]
    note(f"ring chunks T={T} n={n} Hq={Hq} Hk={Hk} mask={spec.kind}")
    x = attention_inputs(40 + idx, T, Hq, Hk)
    q, k, v, do = (to_dev_bf16(x[m], torch) for m in ("q", "k", "v", "do"))
    stream = torch.cuda.current_stream().cuda_stream
    merge_prob = attn.problem(n, Hq, Hk, spec.kind)

    def pair(qi, ki):
        d = attn.mask_desc_build_chunk(spec, T, qi * n, ki * n, n)
        return attn.MaskedAttention(n, Hq, Hk, spec, desc=d)

    # forward: each query chunk visits the key chunks in ring order, starting at its own
    acc = {}
    for qi in range(nc):
        qs = slice(qi * n, (qi + 1) * n)
        for step in range(nc):
            ki = (qi + step) % nc
            ks = slice(ki * n, (ki + 1) * n)
            o, lse, o_lo = pair(qi, ki).forward(q[qs], k[ks], v[ks])
            if step == 0:
                acc[qi] = (o.clone(), o_lo.clone(), lse.clone())
            else:
                ao, alo, al = acc[qi]
                attn.lse_merge(merge_prob, ao.data_ptr(), alo.data_ptr(), al.data_ptr(), o.data_ptr(),
                               o_lo.data_ptr(), lse.data_ptr(), stream)
    # backward: shares of every pair with the merged rows
    dq = torch.zeros((T, Hq, 128), dtype=torch.float32, device=q.device)
    dk = torch.zeros((T, Hk, 128), dtype=torch.float32, device=q.device)
    dv = torch.zeros((T, Hk, 128), dtype=torch.float32, device=q.device)
    for qi in range(nc):
        qs = slice(qi * n, (qi + 1) * n)
        ao, alo, al = acc[qi]
        for ki in range(nc):
            ks = slice(ki * n, (ki + 1) * n)
            a, b, c = pair(qi, ki).backward(q[qs], k[ks], v[ks], ao, al, do[qs], o_lo=alo)
            dq[qs] += a
            dk[ks] += b
            dv[ks] += c
    torch.cuda.synchronize()

    ref = attention_backward(*(oracle_inputs(x)[m] for m in ("q", "k", "v", "do")), spec)
    o_all = np.concatenate([bf16_dev_to_f64(acc[i][0]) for i in range(nc)])
    lse_all = np.concatenate([acc[i][2].cpu().numpy() for i in range(nc)], axis=1)
    errs = [assert_close("O", o_all, ref["o"], TOL), assert_close("LSE", lse_all, ref["lse"], LSE_TOL),
            assert_close("dQ", dq.cpu().numpy(), ref["dq"], TOL), assert_close("dK", dk.cpu().numpy(), ref["dk"], TOL),
            assert_close("dV", dv.cpu().numpy(), ref["dv"], TOL)]
    note("  max errors " + " ".join(f"{e:.2e}" for e in errs))


def test_lse_merge_empty_partial_keeps_accumulator():
    import torch
    T, Hq = 100, 4
    prob = attn.problem(T, Hq, 1, "causal")
    g = torch.Generator(device="cuda").manual_seed(1)
    o = torch.randn(T, Hq, 128, generator=g, device="cuda").to(torch.bfloat16)
    lse = torch.randn(Hq, T, generator=g, device="cuda")
    o0, lse0 = o.clone(), lse.clone()
    empty_o = torch.zeros_like(o)
    empty_lse = torch.full_like(lse, float("-inf"))
    note("lse merge with an empty partial")
    attn.lse_merge(prob, o.data_ptr(), 0, lse.data_ptr(), empty_o.data_ptr(), 0, empty_lse.data_ptr(),
                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, lse0)


@pytest.mark.parametrize("G", [4, 16])
def test_chunk_pair_with_fully_masked_rows(G):
    """One CAUSAL chunk pair whose key chunk starts after some of its queries: those rows
    see no key (O = 0, LSE = -inf, zero gradients), the rest see a ragged causal block; the
    backward uses the pair's own O and LSE. Checked against the fp64 chunk oracle."""
    import torch
    from oracle.chunks import chunk_backward, chunk_forward
    T, n, q0, k0, Hk = 1300, 500, 100, 390, 1
    Hq = G * Hk
    spec = MaskSpec("causal")
    note(f"chunk pair with empty rows G={G} T={T} n={n} q0={q0} k0={k0}")
    x = attention_inputs(60 + G, T, Hq, Hk)
    xo = oracle_inputs(x)
    qs, ks = slice(q0, q0 + n), slice(k0, k0 + n)
    q, k, v, do = (to_dev_bf16(np.ascontiguousarray(x[m][sl]), torch)
                   for m, sl in (("q", qs), ("k", ks), ("v", ks), ("do", qs)))
    ma = attn.MaskedAttention(n, Hq, Hk, spec, desc=attn.mask_desc_build_chunk(spec, T, q0, k0, n))
    o, lse, o_lo = ma.forward(q, k, v)
    dq, dk, dv = ma.backward(q, k, v, o, lse, do, o_lo=o_lo)
    torch.cuda.synchronize()
    ro, rl = chunk_forward(xo["q"][qs], xo["k"][ks], xo["v"][ks], spec, T, q0, k0)
    rdq, rdk, rdv = chunk_backward(xo["q"][qs], xo["k"][ks], xo["v"][ks], xo["do"][qs], ro, rl, spec, T, q0, k0)
    lse_h = lse.cpu().numpy()
    empty = np.isneginf(rl)
    assert empty.any() and not empty.all()
    assert np.array_equal(np.isneginf(lse_h), empty)
    errs = [assert_close("O", bf16_dev_to_f64(o), ro, TOL), assert_close("LSE", lse_h, rl, LSE_TOL),
            assert_close("dQ", dq.cpu().numpy(), rdq, TOL), assert_close("dK", dk.cpu().numpy(), rdk, TOL),
            assert_close("dV", dv.cpu().numpy(), rdv, TOL)]
    rows = np.nonzero(empty[0])[0]
    assert (bf16_dev_to_f64(o)[rows] == 0).all() and (dq.cpu().numpy()[rows] == 0).all()
    note("  max errors " + " ".join(f"{e:.2e}" for e in errs))
