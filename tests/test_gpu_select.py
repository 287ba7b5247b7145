"""GPU parity of the dynamic block-sparse path: the TopK / TopP block selector
(attn_block_select) against the fp64 oracle of oracle/select.py, the selected keep
matrix driving the block-sparse forward and backward, and the Variable Block mask
(expanded on the host) against the oracle's variable-block predicate.

The selection is an integer decision taken on fp32 scores: the kernel's keep matrix must
equal the oracle's selection applied to the kernel's own scores (TopK exactly; TopP up
to prefixes whose mass is within fp32 rounding of p), and the scores must match the
oracle's fp64 block scores."""
import numpy as np
import pytest

from masked_long_context_tiled_amd import attn
from masked_long_context_tiled_amd.inputs import (MaskSpec, attention_inputs, variable_block_grid,
                                                  variable_block_keep)
from oracle.attention import attention_backward
from oracle.select import block_means, block_scores, select_topk, select_topp, selection_order, softmax_row

from gpu_helpers import TOL, LSE_TOL, assert_close, note, oracle_inputs, run_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu

SCORE_TOL = 1e-5   # score gap below which the oracle's fp64 TopK may differ from fp32
MASS_TOL = 1e-5


def _run_select(x, T, Hq, Hk, b, params, scale=0.0):
    import torch
    prob = attn.problem(T, Hq, Hk, "block_sparse", b, scale)
    nb = -(-T // b)
    q, k = to_dev_bf16(x["q"], torch), to_dev_bf16(x["k"], torch)
    scores = torch.empty((Hq, nb, nb), dtype=torch.float32, device="cuda")
    keep = torch.full((Hq, nb, nb), 7, dtype=torch.uint8, device="cuda")
    nws = attn.block_select_workspace_size(prob)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    attn.block_select(prob, params, q.data_ptr(), k.data_ptr(), scores.data_ptr(), keep.data_ptr(),
                      ws.data_ptr(), nws, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return scores.cpu().numpy().astype(np.float64), keep.cpu().numpy(), keep


def _gamma(n):
    u = 2.0 ** -24
    return n * u / (1 - n * u)


def _check_scores(x, b, s_gpu, scale=None):
    """Scores against the fp64 oracle, within the fp32 rounding-error bound of the
    kernel's arithmetic: block sums of b terms (error <= gamma_b * sum |x|), then a
    128-term dot product (gamma_128 * sum |qbar kbar|), then the scale."""
    xo = oracle_inputs(x)
    sc = (1.0 / np.sqrt(128)) if scale is None else scale
    ref = block_scores(xo["q"], xo["k"], b, sc)
    qm, km = block_means(xo["q"], b), block_means(xo["k"], b)
    qa, ka = block_means(np.abs(xo["q"]), b), block_means(np.abs(xo["k"]), b)
    G = qm.shape[0] // km.shape[0]
    for h in range(qm.shape[0]):
        g = h // G
        bound = sc * (_gamma(b + 1) * (qa[h] @ np.abs(km[g]).T + np.abs(qm[h]) @ ka[g].T)
                      + _gamma(128) * (np.abs(qm[h]) @ np.abs(km[g]).T)) + 2.0 ** -23 * np.abs(ref[h])
        err = np.abs(ref[h] - s_gpu[h])
        assert (err <= bound + 1e-30).all(), f"block scores head {h}: max |err| = {err.max():.2e}"
    return ref


CASES = [(1000, 8, 2, 64), (3000, 16, 2, 128), (19200, 2, 1, 64)]


@pytest.mark.parametrize("T,Hq,Hk,b", CASES)
@pytest.mark.parametrize("diag", [True, False])
def test_topk_selection(T, Hq, Hk, b, diag):
    nb = -(-T // b)
    k = max(1, nb // 3)
    note(f"block select topk T={T} Hq={Hq} Hk={Hk} b={b} k={k} diag={diag}")
    x = attention_inputs(7, T, Hq, Hk, with_do=False)
    s, keep, _ = _run_select(x, T, Hq, Hk, b, attn.block_select_params("topk", topk=k, keep_diagonal=diag))
    ref = _check_scores(x, b, s)
    assert np.array_equal(keep, select_topk(s, k, diag))
    # against the fp64 scores too, wherever the k-th and (k+1)-th scores are apart
    want = select_topk(ref, k, diag)
    for h in range(Hq):
        for qb in range(nb):
            order = selection_order(ref[h, qb], qb, diag)
            if k < nb and abs(ref[h, qb, order[k - 1]] - ref[h, qb, order[k]]) <= 2 * SCORE_TOL:
                continue
            assert np.array_equal(keep[h, qb], want[h, qb]), (h, qb)


@pytest.mark.parametrize("T,Hq,Hk,b", CASES)
@pytest.mark.parametrize("p", [0.3, 0.9])
def test_topp_selection(T, Hq, Hk, b, p):
    nb = -(-T // b)
    note(f"block select topp T={T} Hq={Hq} Hk={Hk} b={b} p={p}")
    x = attention_inputs(8, T, Hq, Hk, with_do=False)
    # a large scale spreads the block scores (block means of N(0, 1) rows are small), so
    # the softmax over blocks is far from uniform and TopP keeps varying numbers of blocks
    scale = 30.0
    s, keep, _ = _run_select(x, T, Hq, Hk, b, attn.block_select_params("topp", topp=p, keep_diagonal=True), scale)
    _check_scores(x, b, s, scale)
    want = select_topp(s, p, True)
    assert set(np.unique(keep)) <= {0, 1}
    for h in range(Hq):
        for qb in range(nb):
            prob = softmax_row(s[h, qb])
            order = selection_order(s[h, qb], qb, True)
            n = int(keep[h, qb].sum())
            assert n >= 1 and set(np.flatnonzero(keep[h, qb])) == set(order[:n]), (h, qb)
            cum = np.cumsum(prob[order])
            assert cum[n - 1] >= p - MASS_TOL and (n == 1 or cum[n - 2] < p + MASS_TOL), (h, qb)
            if np.all(np.abs(cum - p) > MASS_TOL):
                assert np.array_equal(keep[h, qb], want[h, qb]), (h, qb)


@pytest.mark.parametrize("b", [64, 128])
@pytest.mark.parametrize("mode", ["topk", "topp"])
def test_selected_keep_drives_sparse_attention(b, mode):
    import torch
    T, Hq, Hk = 1000, 8, 2
    note(f"selected block-sparse attention b={b} mode={mode}")
    x = attention_inputs(9, T, Hq, Hk)
    nb = -(-T // b)
    params = attn.block_select_params(mode, topk=max(1, nb // 2), topp=0.7, keep_diagonal=True)
    _, keep_np, keep_dev = _run_select(x, T, Hq, Hk, b, params)
    # the oracle selects its own blocks from fp64 scores (no near ties at this seed)
    xo = oracle_inputs(x)
    ref_s = block_scores(xo["q"], xo["k"], b)
    keep_or = select_topk(ref_s, nb // 2, True) if mode == "topk" else select_topp(ref_s, 0.7, True)
    assert np.array_equal(keep_np, keep_or)
    spec = MaskSpec("block_sparse", sparse_block=b)
    out = run_gpu(T, Hq, Hk, spec, keep=keep_dev, inputs=x)
    ref = attention_backward(*(xo[m] for m in ("q", "k", "v", "do")), spec, keep=keep_or)
    for name in ("o", "dq", "dk", "dv"):
        assert_close(name, out[name], ref[name], TOL)
    assert_close("lse", out["lse"], ref["lse"], LSE_TOL)


@pytest.mark.parametrize("T,seed", [(1000, 0), (1536, 1)])
def test_variable_block_attention(T, seed):
    Hq, Hk = 8, 2
    ro = variable_block_grid(seed, T)
    co = variable_block_grid(seed + 50, T)
    keep_var = variable_block_keep(seed, Hq, ro, co)
    note(f"variable block attention T={T} seed={seed} row blocks={len(ro) - 1} col blocks={len(co) - 1}")
    x = attention_inputs(20 + seed, T, Hq, Hk)
    spec = MaskSpec("variable_block", row_offsets=ro, col_offsets=co)
    out = run_gpu(T, Hq, Hk, spec, keep=keep_var, inputs=x)
    ref = attention_backward(*(oracle_inputs(x)[m] for m in ("q", "k", "v", "do")), spec, keep=keep_var)
    for name in ("o", "dq", "dk", "dv"):
        assert_close(name, out[name], ref[name], TOL)
    assert_close("lse", out["lse"], ref["lse"], LSE_TOL)
