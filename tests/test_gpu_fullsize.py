"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The whole forward and backward run on the GPU at full size; the fp64 oracle then checks
  * O, LSE and dQ on sampled rows (every row of the oracle is exact on its own), and
  * dK, dV on key-column slabs whose visible rows are few enough to compute in full,
  * elsewhere the gradient identities that hold at any size: sum_j dK_j = 0 per KV
    head and sum_j dV_j = sum of dO over the group's rows that see a key.
Bounds as in the small cases: max |err| <= 2e-2 on O, dQ, dK, dV; LSE within 1e-3.
"""
import numpy as np
import pytest

from masked_long_context_tiled_amd import attn
from masked_long_context_tiled_amd.inputs import attention_inputs, bf16_bits_to_f64, keep_for, workloads
from oracle.attention import attention_backward
from oracle.masks import mask_block

from gpu_helpers import LSE_TOL, TOL, assert_close, bf16_dev_to_f64, check_selection, note, to_dev_bf16

pytestmark = pytest.mark.gpu


def _run(name, seed=0, edit_keep=None):
    """Full-size forward + backward of a workload; edit_keep(keep) may change a copy of a
    block-sparse or variable-block keep matrix first."""
    import torch
    wl = workloads(seed)[name]
    note(f"full size {name}: T={wl.T} Hq={wl.Hq} Hk={wl.Hk} mask={wl.mask.kind}: inputs")
    x = attention_inputs(seed, wl.T, wl.Hq, wl.Hk)
    keep = keep_for(wl, seed)
    if edit_keep is not None:
        keep = edit_keep(keep.copy())
    q, k, v, do = (to_dev_bf16(x[n], torch) for n in ("q", "k", "v", "do"))
    note(f"full size {name}: GPU forward + backward")
    ma = attn.MaskedAttention(wl.T, wl.Hq, wl.Hk, wl.mask, keep=keep)
    o, lse, o_lo = ma.forward(q, k, v)
    dq, dk, dv = ma.backward(q, k, v, o, lse, do, o_lo=o_lo)
    torch.cuda.synchronize()
    return wl, x, keep, {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _group_arrays(x, wl, heads):
    """fp64 inputs restricted to query heads `heads` (all in one KV group) and their KV head."""
    G = wl.Hq // wl.Hk
    g = heads[0] // G
    assert all(h // G == g for h in heads)
    sub = lambda a, hs: bf16_bits_to_f64(np.ascontiguousarray(a[:, hs]))
    return sub(x["q"], heads), sub(x["k"], [g]), sub(x["v"], [g]), sub(x["do"], heads), g


def _check_rows(wl, x, keep, out, heads, rows):
    G = wl.Hq // wl.Hk
    groups = sorted({h // G for h in heads})
    if len(groups) > 1:                       # one oracle call per KV group
        for g in groups:
            _check_rows(wl, x, keep, out, [h for h in heads if h // G == g], rows)
        return
    import torch
    q, k, v, do, g = _group_arrays(x, wl, heads)
    kp = None if keep is None else keep[heads]
    ref = attention_backward(q, k, v, do, wl.mask, rows=rows, keep=kp)
    r_t = torch.as_tensor(rows, device=out["dq"].device)
    h_t = torch.as_tensor(heads, device=out["dq"].device)
    o = bf16_dev_to_f64(out["o"][r_t][:, h_t].contiguous())
    lse = out["lse"][h_t][:, r_t].cpu().numpy()
    dq = out["dq"][r_t][:, h_t].cpu().numpy()
    e = (assert_close("O", o, ref["o"], TOL), assert_close("LSE", lse, ref["lse"], LSE_TOL),
         assert_close("dQ", dq, ref["dq"], TOL))
    note(f"  rows {len(rows)} heads {heads}: O {e[0]:.2e} LSE {e[1]:.2e} dQ {e[2]:.2e}")


def _check_key_slab(wl, x, keep, out, g, cols):
    """dK, dV of KV head g on key columns `cols`, from every row that sees one of them."""
    G = wl.Hq // wl.Hk
    heads = list(range(g * G, (g + 1) * G))
    q, k, v, do, _ = _group_arrays(x, wl, heads)
    kp = None if keep is None else keep[heads]
    seen = np.zeros(wl.T, dtype=bool)
    for hi in range(G):
        for r0 in range(0, wl.T, 4096):
            rr = np.arange(r0, min(wl.T, r0 + 4096))
            seen[rr] |= mask_block(wl.mask, wl.T, rr, cols, hi, kp).any(axis=1)
    rows = np.nonzero(seen)[0]
    ref = attention_backward(q, k, v, do, wl.mask, rows=rows, key_cols=cols, keep=kp)
    dk = out["dk"][cols.min():cols.max() + 1, g].cpu().numpy()[cols - cols.min()]
    dv = out["dv"][cols.min():cols.max() + 1, g].cpu().numpy()[cols - cols.min()]
    e = (assert_close("dK", dk, ref["dk"][:, 0], TOL), assert_close("dV", dv, ref["dv"][:, 0], TOL))
    note(f"  key slab [{cols.min()}, {cols.max()}] of KV head {g} ({len(rows)} rows): dK {e[0]:.2e} dV {e[1]:.2e}")


def _check_sums(wl, x, out, rows_visible=None):
    """sum_j dK_j = 0 and sum_j dV_j = sum over rows with a visible key of dO, per KV head."""
    import torch
    G = wl.Hq // wl.Hk
    dk_sum = out["dk"].double().sum(0).cpu().numpy()               # [Hk][d]
    dv_sum = out["dv"].double().sum(0).cpu().numpy()
    do = torch.from_numpy(np.ascontiguousarray(x["do"]).view(np.int16)).view(torch.bfloat16)
    finite = torch.isfinite(out["lse"]).cpu()                       # [Hq][T]
    want = np.zeros((wl.Hk, 128))
    for h in range(wl.Hq):
        want[h // G] += (do[:, h].double() * finite[h][:, None]).sum(0).numpy()
    # each sum adds T * G terms of size ~1 whose P and dS carry independent fp16 rounding
    # (relative 2^-12): the error grows like the square root of the number of terms. The
    # bound catches gross errors only (a missing key tile of a dense mask, a scale error);
    # a dropped or doubled block of one head moves a sum by far less than the bound at 64K,
    # which is what the element-wise key slabs are for
    tol = 5e-2 * np.sqrt(wl.T * G / 512.0)
    e1 = assert_close("sum dK", dk_sum, 0.0 * dk_sum, tol)
    e2 = assert_close("sum dV", dv_sum, want, tol)
    note(f"  gradient sums: |sum dK| {e1:.2e}  |sum dV - sum dO| {e2:.2e}  (bound {tol:.2e})")


def _sample_rows(T, n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, T // 2, T - 1], rng.integers(0, T, n)]))


@pytest.mark.parametrize("name", ["causal_8k_gqa", "full_8k_gqa", "causal_8k_mha", "full_8k_mha"])
def test_8k(name):
    wl, x, keep, out = _run(name)
    G = wl.Hq // wl.Hk
    _check_rows(wl, x, keep, out, heads=[0, 1], rows=_sample_rows(wl.T, 48, 1))
    _check_rows(wl, x, keep, out, heads=[wl.Hq - G], rows=_sample_rows(wl.T, 48, 2))
    last = wl.Hk - 1
    _check_key_slab(wl, x, keep, out, last, np.arange(wl.T - 96, wl.T))
    if wl.mask.kind == "causal" and G == 8:
        _check_key_slab(wl, x, keep, out, 3, np.arange(6144, 6208))
    _check_sums(wl, x, out)


@pytest.mark.parametrize("name", ["full_document_32k", "causal_document_32k", "full_sliding_window_32k",
                                  "causal_sliding_window_32k", "shared_question_16k", "prefix_lm_causal_16k",
                                  "causal_blockwise_16k", "global_sliding_16k", "prefix_lm_document_32k",
                                  "block_causal_document_32k"])
def test_workload_masks(name):
    wl, x, keep, out = _run(name)
    _check_rows(wl, x, keep, out, heads=[8, 15], rows=_sample_rows(wl.T, 24, 3))
    kind = wl.mask.kind
    if kind in ("causal_document", "full_document", "prefix_lm_document", "block_causal_document"):
        cu = np.asarray(wl.mask.cu_seqlens)
        d = int(np.argmin(np.diff(cu)))                        # the shortest document
        _check_key_slab(wl, x, keep, out, 5, np.arange(cu[d], min(cu[d + 1], cu[d] + 64)))
    elif kind in ("causal_sliding_window", "shared_question", "prefix_lm_causal", "causal_blockwise"):
        _check_key_slab(wl, x, keep, out, 2, np.arange(wl.T - 64, wl.T))
    _check_sums(wl, x, out)


@pytest.mark.timeout(900)
def test_causal_128k():
    wl, x, keep, out = _run("causal_128k")
    _check_rows(wl, x, keep, out, heads=[0, 5], rows=_sample_rows(wl.T, 12, 4))
    _check_key_slab(wl, x, keep, out, 7, np.arange(wl.T - 48, wl.T))
    _check_sums(wl, x, out)


def _sparse_slab_edit(g, nb, qbs, G=8):
    """Keep-matrix edit: key block nb - 1 is kept, in KV group g, only by the (head offset,
    query block) pairs in qbs, so every row that sees it can be computed by the oracle."""
    def edit(keep):
        keep[g * G:(g + 1) * G, :, nb - 1] = 0
        for hi, qb in qbs:
            keep[g * G + hi, qb, nb - 1] = 1
        return keep
    return edit


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["block_sparse_64k_b128", "block_sparse_64k_b64"])
def test_block_sparse_64k(name):
    wl = workloads(0)[name]
    b = wl.mask.sparse_block
    nb = wl.T // b
    edit = _sparse_slab_edit(7, nb, [(0, nb - 1), (0, 5), (3, nb // 2), (3, nb // 2 + 1), (6, 0)])
    wl, x, keep, out = _run(name, edit_keep=edit)
    _check_rows(wl, x, keep, out, heads=[16, 17], rows=_sample_rows(wl.T, 12, 5))
    _check_key_slab(wl, x, keep, out, 7, np.arange(wl.T - b, wl.T))
    _check_sums(wl, x, out)


@pytest.mark.timeout(600)
def test_variable_block_64k():
    wl = workloads(0)["variable_block_64k"]
    ro, co = np.asarray(wl.mask.row_offsets), np.asarray(wl.mask.col_offsets)
    nr, nc = len(ro) - 1, len(co) - 1
    # the last column block kept, in KV group 6, by three (head, row block) pairs only
    edit = _sparse_slab_edit(6, nc, [(1, nr - 1), (2, 7), (7, nr // 3)])
    wl, x, keep, out = _run("variable_block_64k", edit_keep=edit)
    _check_rows(wl, x, keep, out, heads=[16, 17], rows=_sample_rows(wl.T, 12, 6))
    _check_key_slab(wl, x, keep, out, 6, np.arange(co[-2], co[-1]))
    _check_sums(wl, x, out)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["topk_sparse_64k_b128", "topp_sparse_64k_b128"])
def test_dynamic_sparse_64k(name):
    """Selection on the GPU at full size, then the block-sparse path on the selected blocks.
    The oracle selects the checked heads' blocks itself from fp64 block scores; the GPU's
    selection must agree with it there."""
    import torch
    from oracle.select import block_scores

    wl = workloads(0)[name]
    b = wl.mask.sparse_block
    nb = -(-wl.T // b)
    mode, val = wl.select
    note(f"full size {name}: T={wl.T} Hq={wl.Hq} Hk={wl.Hk} b={b} select={wl.select}: inputs")
    x = attention_inputs(0, wl.T, wl.Hq, wl.Hk)
    q, k, v, do = (to_dev_bf16(x[n], torch) for n in ("q", "k", "v", "do"))
    prob = attn.problem(wl.T, wl.Hq, wl.Hk, "block_sparse", b)
    scores = torch.empty((wl.Hq, nb, nb), dtype=torch.float32, device="cuda")
    keep_dev = torch.empty((wl.Hq, nb, nb), dtype=torch.uint8, device="cuda")
    nws = attn.block_select_workspace_size(prob)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    params = attn.block_select_params(mode, topk=int(val) if mode == "topk" else 0,
                                      topp=float(val) if mode == "topp" else 0.0, keep_diagonal=True)
    note(f"full size {name}: GPU selection, forward + backward")
    attn.block_select(prob, params, q.data_ptr(), k.data_ptr(), scores.data_ptr(), keep_dev.data_ptr(),
                      ws.data_ptr(), nws, torch.cuda.current_stream().cuda_stream)
    ma = attn.MaskedAttention(wl.T, wl.Hq, wl.Hk, wl.mask, keep=keep_dev)
    o, lse, o_lo = ma.forward(q, k, v)
    dq, dk, dv = ma.backward(q, k, v, o, lse, do, o_lo=o_lo)
    torch.cuda.synchronize()
    out = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}

    heads = [16, 17]
    qh, kh, _, _, g = _group_arrays(x, wl, heads)
    ref_s = block_scores(qh, kh, b)
    gpu_s = scores.cpu().numpy().astype(np.float64)
    err = float(np.abs(gpu_s[heads] - ref_s).max())
    assert err <= 1e-5, f"block scores: max |err| = {err:.2e}"
    gpu_keep = keep_dev.cpu().numpy()
    # the selection rule on the GPU's own scores for the first two KV groups (8192 rows);
    # the fp64 selection on heads 16, 17 wherever no near-tie decides
    sub = list(range(16)) + heads
    compared, skipped = check_selection(gpu_keep[sub], gpu_s[sub], mode, val, True,
                                        ref_s=ref_s, heads=[16, 17])
    note(f"  scores max |err| {err:.2e}; rows equal to the fp64 selection {compared}, "
         f"near-ties {skipped}")
    # attention with the GPU's keep matrix (an integer input of the attention problem)
    _check_rows(wl, x, gpu_keep, out, heads=heads, rows=_sample_rows(wl.T, 16, 7))
    _check_sums(wl, x, out)


def _host_f64(t):
    """bf16 device tensor (any shape) -> float64 numpy array."""
    import torch
    return bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


@pytest.mark.timeout(900)
def test_causal_512k():
    """CAUSAL GQA 64:8 at T = 524288, the top of the pages' 1K-512K range. Q, dO, O hold
    2^32 elements each and dQ is 16 GiB, so the last rows sit past every 32-bit element
    offset. Inputs are drawn on the device (attention_inputs_device); the oracle receives
    the rows it checks, copied back. Checked: O, LSE, dQ on sampled rows (the last row
    included) of heads in the first and last KV groups, dK / dV of the last 48 keys of KV
    head 7 from every row that sees them, and the two gradient sums."""
    import torch
    from masked_long_context_tiled_amd.inputs import MaskSpec, attention_inputs_device
    T, Hq, Hk, G = 524288, 64, 8, 8
    spec = MaskSpec("causal")
    note(f"512K causal: T={T} Hq={Hq} Hk={Hk}: inputs on the device")
    xd = attention_inputs_device(5, T, Hq, Hk, "cuda")
    ma = attn.MaskedAttention(T, Hq, Hk, spec)
    note("512K causal: GPU forward")
    o, lse, o_lo = ma.forward(xd["q"], xd["k"], xd["v"])
    note("512K causal: GPU backward")
    dq, dk, dv = ma.backward(xd["q"], xd["k"], xd["v"], o, lse, xd["do"], o_lo=o_lo)
    torch.cuda.synchronize()
    note("512K causal: oracle on sampled rows")

    def group_inputs(heads, rows):
        g = heads[0] // G
        h_t = torch.as_tensor(heads, device="cuda")
        r_t = torch.as_tensor(rows, device="cuda")
        q = np.zeros((T, len(heads), 128))
        do = np.zeros((T, len(heads), 128))
        q[rows] = _host_f64(xd["q"][r_t][:, h_t])
        do[rows] = _host_f64(xd["do"][r_t][:, h_t])
        k = _host_f64(xd["k"][:, g:g + 1])
        v = _host_f64(xd["v"][:, g:g + 1])
        return q, k, v, do, g, h_t, r_t

    for heads, seed in (([0, 5], 8), ([63], 9)):
        rows = _sample_rows(T, 10, seed)
        q, k, v, do, g, h_t, r_t = group_inputs(heads, rows)
        ref = attention_backward(q, k, v, do, spec, rows=rows)
        e = (assert_close("O", _host_f64(o[r_t][:, h_t]), ref["o"], TOL),
             assert_close("LSE", lse[h_t][:, r_t].cpu().numpy(), ref["lse"], LSE_TOL),
             assert_close("dQ", dq[r_t][:, h_t].cpu().numpy(), ref["dq"], TOL))
        note(f"  rows {len(rows)} (last {rows[-1]}) heads {heads}: O {e[0]:.2e} LSE {e[1]:.2e} dQ {e[2]:.2e}")

    cols = np.arange(T - 48, T)
    rows = cols.copy()                        # CAUSAL: key j is seen by rows i >= j
    heads = list(range(7 * G, 8 * G))
    q, k, v, do, g, h_t, r_t = group_inputs(heads, rows)
    ref = attention_backward(q, k, v, do, spec, rows=rows, key_cols=cols)
    e = (assert_close("dK", dk[T - 48:, 7].cpu().numpy(), ref["dk"][:, 0], TOL),
         assert_close("dV", dv[T - 48:, 7].cpu().numpy(), ref["dv"][:, 0], TOL))
    note(f"  key slab [{T - 48}, {T - 1}] of KV head 7: dK {e[0]:.2e} dV {e[1]:.2e}")

    # sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i over the group (every CAUSAL row sees a key)
    dk_sum = torch.zeros((Hk, 128), dtype=torch.float64, device="cuda")
    dv_sum = torch.zeros_like(dk_sum)
    want = torch.zeros_like(dk_sum)
    for r0 in range(0, T, 32768):
        dk_sum += dk[r0:r0 + 32768].double().sum(0)
        dv_sum += dv[r0:r0 + 32768].double().sum(0)
        want += xd["do"][r0:r0 + 32768].double().sum(0).view(Hk, G, 128).sum(1)
    tol = 5e-2 * np.sqrt(T * G / 512.0)
    e1 = assert_close("sum dK", dk_sum.cpu().numpy(), np.zeros((Hk, 128)), tol)
    e2 = assert_close("sum dV", dv_sum.cpu().numpy(), want.cpu().numpy(), tol)
    note(f"  gradient sums: |sum dK| {e1:.2e}  |sum dV - sum dO| {e2:.2e}  (bound {tol:.2e})")
