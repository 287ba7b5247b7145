"""Helpers shared by the GPU tests: upload seeded inputs, run the library, run the oracle."""
import json
import os
import sys

import numpy as np

from masked_long_context_tiled_amd import attn
from masked_long_context_tiled_amd.inputs import attention_inputs, bf16_bits_to_f64

TOL = 2e-2          # max-abs bound on O, dQ, dK, dV against the fp64 oracle
LSE_TOL = 1e-3


def note(msg):
    """Name the case on stdout before each GPU step (flushed)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_dev_to_f64(t):
    import torch
    return bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def run_gpu(T, Hq, Hk, spec, keep=None, seed=0, backward=True, inputs=None, scale=0.0):
    """Run forward (and backward) through the C ABI; return numpy results and the inputs.
    scale <= 0 selects the library's default 1 / sqrt(128)."""
    import torch
    x = inputs if inputs is not None else attention_inputs(seed, T, Hq, Hk)
    q, k, v = (to_dev_bf16(x[n], torch) for n in ("q", "k", "v"))
    ma = attn.MaskedAttention(T, Hq, Hk, spec, keep=keep, scale=scale)
    o, lse, o_lo = ma.forward(q, k, v)
    out = {"ma": ma}
    if backward:
        do = to_dev_bf16(x["do"], torch)
        dq, dk, dv = ma.backward(q, k, v, o, lse, do, o_lo=o_lo)
        torch.cuda.synchronize()
        out.update(dq=dq.cpu().numpy(), dk=dk.cpu().numpy(), dv=dv.cpu().numpy())
    torch.cuda.synchronize()
    out.update(o=bf16_dev_to_f64(o), lse=lse.cpu().numpy(), inputs=x)
    return out


def oracle_inputs(x):
    return {n: bf16_bits_to_f64(x[n]) for n in x}


def max_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nanmax(d)) if d.size else 0.0


def record_margin(name, err, tol):
    """Append (test, quantity, max error, bound) to the JSON-lines file named by the
    environment variable MLCT_PARITY_LOG, if set: the measured parity margins."""
    path = os.environ.get("MLCT_PARITY_LOG")
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    with open(path, "a") as f:
        f.write(json.dumps({"test": test, "q": name, "err": err, "tol": tol}) + "\n")


def assert_close(name, got, want, tol):
    err = max_err(got, want)
    record_margin(name, err, tol)
    assert np.isfinite(err) and err <= tol, f"{name}: max |err| = {err:.3e} > {tol:.1e}"
    return err


# --- block selection rules (TopK / TopP) ------------------------------------------------

SCORE_TOL = 1e-5   # score gap below which fp32 and fp64 selections may differ
MASS_TOL = 1e-5    # TopP prefix mass within which fp32 and fp64 cuts may differ


def check_selection(keep, s_gpu, mode, val, diag, ref_s=None, heads=None):
    """The GPU keep matrix [Hq][nb][nb] must be exactly the selection rule applied to the
    GPU's own fp32 scores s_gpu (TopK: the first k of the order; TopP: the shortest prefix
    whose mass reaches p, up to prefixes within MASS_TOL of p). Where fp64 scores ref_s
    (for the query heads ``heads``) are given, the keep must equal the oracle's fp64
    selection except at near-ties: TopK rows whose k-th and (k+1)-th fp64 scores lie within
    2 SCORE_TOL; TopP rows whose fp64 prefix mass at the cut lies within MASS_TOL of p or
    whose kept and dropped blocks are within 2 SCORE_TOL of each other in fp64.
    Returns the number of rows compared with the fp64 selection and the number skipped."""
    from oracle.select import select_topk, select_topp, selection_order, softmax_row
    Hq, nb, _ = keep.shape
    assert set(np.unique(keep).tolist()) <= {0, 1}
    if mode == "topk":
        assert np.array_equal(keep, select_topk(s_gpu, int(val), diag)), "TopK rule on the GPU's scores"
    else:
        p = float(val)
        want = select_topp(s_gpu, p, diag)
        for h in range(Hq):
            for qb in range(nb):
                order = selection_order(s_gpu[h, qb], qb, diag)
                n = int(keep[h, qb].sum())
                assert n >= 1 and set(np.flatnonzero(keep[h, qb])) == set(order[:n]), (h, qb)
                cum = np.cumsum(softmax_row(s_gpu[h, qb])[order])
                assert cum[n - 1] >= p - MASS_TOL and (n == 1 or cum[n - 2] < p + MASS_TOL), (h, qb)
                if np.all(np.abs(cum - p) > MASS_TOL):
                    assert np.array_equal(keep[h, qb], want[h, qb]), (h, qb)
    if ref_s is None:
        return 0, 0
    heads = list(range(Hq)) if heads is None else list(heads)
    want = select_topk(ref_s, int(val), diag) if mode == "topk" else select_topp(ref_s, float(val), diag)
    compared = skipped = 0
    for hi, h in enumerate(heads):
        for qb in range(nb):
            if np.array_equal(keep[h, qb], want[hi, qb]):
                compared += 1
                continue
            row = ref_s[hi, qb]
            order = selection_order(row, qb, diag)
            kept = np.flatnonzero(keep[h, qb])
            dropped = np.flatnonzero(keep[h, qb] == 0)
            if diag:
                kept = kept[kept != qb]
            near_tie = (kept.size and dropped.size
                        and row[kept].min() >= row[dropped].max() - 2 * SCORE_TOL)
            if mode == "topk":
                k = int(val)
                ok = k < nb and abs(row[order[k - 1]] - row[order[k]]) <= 2 * SCORE_TOL and near_tie
            else:
                n = int(keep[h, qb].sum())
                cum = np.cumsum(softmax_row(row)[order])
                near_p = abs(cum[n - 1] - float(val)) <= MASS_TOL or (n >= 2 and abs(cum[n - 2] - float(val)) <= MASS_TOL)
                ok = near_p or near_tie
            assert ok, f"head {h} query block {qb}: differs from the fp64 selection away from a near-tie"
            skipped += 1
    return compared, skipped
