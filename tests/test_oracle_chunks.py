"""Pins of the context-parallel oracle (oracle/chunks.py) against the whole-sequence oracle,
and of the library's chunk-pair descriptor against the per-element predicate."""
import numpy as np
import pytest

from masked_long_context_tiled_amd import attn
from masked_long_context_tiled_amd.inputs import MASK_KINDS, MaskSpec, attention_inputs, bf16_bits_to_f64, \
    document_cu_seqlens
from oracle.attention import attention_backward, attention_forward
from oracle.chunks import chunk_backward, chunk_forward, lse_merge
from oracle.masks import mask_block


def _specs(T):
    return [
        MaskSpec("causal"),
        MaskSpec("full"),
        MaskSpec("causal_document", cu_seqlens=document_cu_seqlens(2, T, 20, 90)),
        MaskSpec("full_sliding_window", window=37),
        MaskSpec("shared_question", question_len=T - 3 * 40, answer_len=40, n_answers=3),
        MaskSpec("global_sliding", global_len=5, window=21),
        MaskSpec("prefix_lm_document", prefix_len=13, cu_seqlens=document_cu_seqlens(4, T, 20, 90)),
        MaskSpec("block_causal_document", block_len=9, cu_seqlens=document_cu_seqlens(5, T, 20, 90)),
    ]


def _inputs(T, Hq=4, Hk=2, seed=3):
    x = attention_inputs(seed, T, Hq, Hk, d=16)
    return {n: bf16_bits_to_f64(a) for n, a in x.items()}


@pytest.mark.parametrize("idx", range(8))
def test_merged_chunks_equal_whole_sequence(idx):
    T, n = 240, 60
    spec = _specs(T)[idx]
    x = _inputs(T)
    o_ref, lse_ref = attention_forward(x["q"], x["k"], x["v"], spec)
    for qc in range(0, T, n):
        order = list(range(0, T, n))[::-1] if idx % 2 else list(range(0, T, n))   # merge order is free
        acc = None
        for kc in order:
            part = chunk_forward(x["q"][qc:qc + n], x["k"][kc:kc + n], x["v"][kc:kc + n], spec, T, qc, kc)
            acc = part if acc is None else lse_merge(acc[0], acc[1], part[0], part[1])
        np.testing.assert_allclose(acc[0], o_ref[qc:qc + n], rtol=0, atol=1e-12)
        np.testing.assert_allclose(acc[1], lse_ref[:, qc:qc + n], rtol=0, atol=1e-12)


@pytest.mark.parametrize("idx", [0, 2, 4, 5, 7])
def test_chunk_backward_shares_sum_to_whole(idx):
    T, n = 180, 60
    spec = _specs(T)[idx]
    x = _inputs(T)
    ref = attention_backward(x["q"], x["k"], x["v"], x["do"], spec)
    dq = np.zeros_like(ref["dq"])
    dk = np.zeros_like(ref["dk"])
    dv = np.zeros_like(ref["dv"])
    for qc in range(0, T, n):
        for kc in range(0, T, n):
            a, b, c = chunk_backward(x["q"][qc:qc + n], x["k"][kc:kc + n], x["v"][kc:kc + n], x["do"][qc:qc + n],
                                     ref["o"][qc:qc + n], ref["lse"][:, qc:qc + n], spec, T, qc, kc)
            dq[qc:qc + n] += a
            dk[kc:kc + n] += b
            dv[kc:kc + n] += c
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(got, ref[name], rtol=0, atol=1e-11, err_msg=name)


def test_whole_sequence_chunk_is_plain_attention():
    T = 96
    x = _inputs(T)
    spec = MaskSpec("causal")
    o, lse = chunk_forward(x["q"], x["k"], x["v"], spec, T, 0, 0)
    o_ref, lse_ref = attention_forward(x["q"], x["k"], x["v"], spec)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13)


def test_merge_identities():
    rng = np.random.default_rng(0)
    n, Hq, d = 7, 3, 5
    o1, o2 = rng.standard_normal((n, Hq, d)), rng.standard_normal((n, Hq, d))
    l1, l2 = rng.standard_normal((Hq, n)), rng.standard_normal((Hq, n))
    empty = np.full((Hq, n), -np.inf)
    zero = np.zeros((n, Hq, d))
    # an empty partial changes nothing; merging is symmetric
    o, l = lse_merge(o1, l1, zero, empty)
    np.testing.assert_array_equal(o, o1)
    np.testing.assert_array_equal(l, l1)
    oa, la = lse_merge(o1, l1, o2, l2)
    ob, lb = lse_merge(o2, l2, o1, l1)
    np.testing.assert_allclose(oa, ob, atol=1e-15)
    np.testing.assert_allclose(la, lb, atol=1e-15)
    # two equal partials: same O, LSE + ln 2
    o, l = lse_merge(o1, l1, o1, l1)
    np.testing.assert_allclose(o, o1, atol=1e-15)
    np.testing.assert_allclose(l, l1 + np.log(2.0), atol=1e-15)
    # both empty: O = 0, LSE = -inf
    o, l = lse_merge(zero, empty, zero, empty)
    assert np.all(o == 0) and np.all(np.isneginf(l))


@pytest.mark.parametrize("T,n", [(300, 100), (257, 64)])
def test_chunk_descriptor_equals_predicate(T, n):
    for spec in _specs(T):
        for q0 in range(0, T - n + 1, 61):
            for k0 in range(0, T - n + 1, 53):
                desc = attn.mask_desc_build_chunk(spec, T, q0, k0, n)
                r = np.arange(n)[:, None]
                a0, b0, a1, b1 = (desc[:, i][None, :] for i in range(4))
                got = ((r >= a0) & (r < b0)) | ((r >= a1) & (r < b1))
                want = mask_block(spec, T, np.arange(q0, q0 + n), np.arange(k0, k0 + n))
                assert np.array_equal(got, want), (spec.kind, q0, k0)
                assert np.all((desc >= 0) & (desc <= n))


def test_chunk_descriptor_validation():
    spec = MaskSpec("causal")
    for args in ((100, -1, 0, 10), (100, 0, 95, 10), (100, 95, 0, 10), (100, 0, 0, 0)):
        with pytest.raises(attn.AttnError) as ei:
            attn.mask_desc_build_chunk(spec, *args)
        assert ei.value.status == attn.ATTN_ERR_INVALID_ARG
    # the whole sequence as one chunk is the ordinary descriptor
    assert np.array_equal(attn.mask_desc_build_chunk(spec, 77, 0, 0, 77), attn.mask_desc_build(spec, 77))
