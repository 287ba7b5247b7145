"""Helpers shared by the GPU tests: upload seeded inputs, run the library, run the oracle."""
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


def run_gpu(T, Hq, Hk, spec, keep=None, seed=0, backward=True, inputs=None):
    """Run forward (and backward) through the C ABI; return numpy results and the inputs."""
    import torch
    x = inputs if inputs is not None else attention_inputs(seed, T, Hq, Hk)
    q, k, v = (to_dev_bf16(x[n], torch) for n in ("q", "k", "v"))
    ma = attn.MaskedAttention(T, Hq, Hk, spec, keep=keep)
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


def assert_close(name, got, want, tol):
    err = max_err(got, want)
    assert np.isfinite(err) and err <= tol, f"{name}: max |err| = {err:.3e} > {tol:.1e}"
    return err
