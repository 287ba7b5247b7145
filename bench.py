#!/usr/bin/env python3
"""Throughput of the masked attention hot path on one MI355X (gfx950).

One step = one pass of the whole path over one batch of synthetic inputs that are
already resident in HBM (the document boundaries of the DOCUMENT masks included):
  column-interval descriptor (built on the device) -> tile index (classifier + lists)
  -> attn_fwd -> attn_bwd_preprocess (D = rowsum(dO*O), operand bounds)
  -> attn_bwd_dkdv (dK, dV) -> attn_bwd_dq (dQ).
The step's launches are captured once into a HIP graph and the timed steps replay it
(--no-graph: the same launches issued one by one in every step).
Block-sparse workloads replace the first two steps by the block index of a keep matrix
uploaded once; dynamic block-sparse workloads select that keep matrix from Q and K
(attn_block_select, TopK / TopP) in every step; the variable-block workload expands its
grid to the uniform 64-block keep matrix once, on the host, before timing.
The default workload is CAUSAL at T = 8192, 64 query heads sharing 8 KV heads, head
dim 128, bf16 inputs N(0,1) from a seed.

Effective FLOPs count only visible (query, key) pairs U (from the descriptor, or from
the keep matrix for block-sparse masks): forward 4*d*Hq*U, backward 10*d*Hq*U.
`value` is the effective TFLOP/s of whole steps (fwd + bwd work / step wall time).
Per-kernel times come from HIP events on the stream the kernels run on.

Prints one JSON line on stdout. Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from masked_long_context_tiled_amd import attn  # noqa: E402
from masked_long_context_tiled_amd.inputs import MaskSpec, attention_inputs, keep_for, workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
METRIC = "effective attn TFLOPs fwd/bwd, 8K GQA 64:8 hd128 bf16 per mask; % MFMA peak"
KERNEL_SOURCES = ["fwd.hip", "bwd.hip", "index.hip", "common.h", "host.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """Hash of the kernel sources with comments and whitespace removed, so that committed
    counter results stay valid across edits that change no code."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "masked_long_context_tiled_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def visible_pairs(spec, T, desc, keep) -> int:
    """U: visible pairs per head (mean over heads for block-sparse)."""
    if spec.kind == "block_sparse":
        b = spec.sparse_block
        nb = keep.shape[1]
        sizes = np.minimum(b, T - np.arange(nb) * b).astype(np.int64)
        per_head = np.einsum("hqk,q,k->h", keep.astype(np.int64), sizes, sizes)
        return int(per_head.sum()) // keep.shape[0], int(per_head.sum())
    d = desc.astype(np.int64)
    U = int(((d[:, 1] - d[:, 0]) + (d[:, 3] - d[:, 2])).sum())
    return U, None


def traffic_for(workload: str, kernel: str):
    """HBM bytes per launch from committed counter runs, if they match the current kernels."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, x, keep, heads: int):
    """Time the fp64 CPU oracle (forward + backward) on a bounded sample: `heads` query
    heads of the same KV group, every row. Reported as effective TFLOP/s."""
    from oracle.attention import attention_backward   # test infrastructure, timed here only
    from oracle.masks import visible_count
    from masked_long_context_tiled_amd.inputs import bf16_bits_to_f64
    try:
        from threadpoolctl import threadpool_info
        cores = max(i.get("num_threads", 1) for i in threadpool_info()) if threadpool_info() else os.cpu_count()
    except Exception:
        cores = os.cpu_count()
    hs = list(range(min(heads, wl.Hq)))
    q = bf16_bits_to_f64(x["q"][:, hs])
    do = bf16_bits_to_f64(x["do"][:, hs])
    G = wl.Hq // wl.Hk
    g = hs[0] // G
    k = bf16_bits_to_f64(x["k"][:, g:g + 1])
    v = bf16_bits_to_f64(x["v"][:, g:g + 1])
    t0 = time.perf_counter()
    if wl.select is not None:
        # dynamic block-sparse: the oracle selects the sample heads' blocks itself
        from oracle.select import block_scores, select_topk, select_topp
        s = block_scores(q, k, wl.mask.sparse_block)
        mode, val = wl.select
        sub_keep = select_topk(s, int(val), True) if mode == "topk" else select_topp(s, float(val), True)
    else:
        sub_keep = None if keep is None else keep[hs]
    attention_backward(q, k, v, do, wl.mask, keep=sub_keep)
    dt = time.perf_counter() - t0
    U = sum(visible_count(wl.mask, wl.T, h, sub_keep) for h in range(len(hs)))
    flops = 14.0 * wl.d * U
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(hs)} query heads x all {wl.T} rows of {wl.name}, fwd+bwd fp64, {dt:.1f} s",
            "seconds": round(dt, 2)}


def sweep(args, torch, dev):
    """Forward + backward at T = 1K, 2K, ... --sweep-max for one mask at GQA 64:8, head dim
    128: effective TFLOP/s and the peak device memory of each length (inputs, outputs,
    tile index and workspace, as allocated by PyTorch's caching allocator). Inputs are
    N(0,1) bf16 drawn on the device from a seeded generator."""
    Hq, Hk, d = 64, 8, 128
    spec = MaskSpec(args.sweep_mask)
    points = []
    T = 1024
    while T <= args.sweep_max:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed + T)
        rnd = lambda *shape: torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        q, k, v, do = rnd(T, Hq, d), rnd(T, Hk, d), rnd(T, Hk, d), rnd(T, Hq, d)
        prob = attn.problem(T, Hq, Hk, spec.kind)
        idx_bytes = attn.tile_index_size(prob)
        ws_bytes = attn.bwd_workspace_size(prob)
        index = torch.empty(idx_bytes, dtype=torch.uint8, device=dev)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        o = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
        o_lo = torch.empty_like(o)
        lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
        dq = torch.empty((T, Hq, d), dtype=torch.float32, device=dev)
        dk = torch.empty((T, Hk, d), dtype=torch.float32, device=dev)
        dv = torch.empty((T, Hk, d), dtype=torch.float32, device=dev)
        desc_host = attn.mask_desc_build(spec, T)
        desc_dev = torch.from_numpy(desc_host).to(dev)
        U, _ = visible_pairs(spec, T, desc_host, None)
        fwd_flops = 4.0 * d * Hq * U
        bwd_flops = 2.5 * fwd_flops
        stream = torch.cuda.current_stream(dev)
        sp = stream.cuda_stream
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

        def run():
            attn.tile_index_build(prob, desc_dev.data_ptr(), index.data_ptr(), idx_bytes, sp)
            ev[0].record(stream)
            attn.fwd(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), o_lo.data_ptr(),
                     lse.data_ptr(), desc_dev.data_ptr(), index.data_ptr(), idx_bytes, 0, 0, sp)
            ev[1].record(stream)
            attn.bwd(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), o_lo.data_ptr(),
                     lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                     desc_dev.data_ptr(), index.data_ptr(), idx_bytes, ws.data_ptr(), ws_bytes, sp)
            ev[2].record(stream)
            ev[2].synchronize()
            return ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])

        run()   # warm-up
        reps = 3 if T <= 65536 else 1
        tf, tb = zip(*[run() for _ in range(reps)])
        t_f, t_b = float(np.median(tf)), float(np.median(tb))
        peak = torch.cuda.max_memory_allocated(dev) - base
        pt = {"T": T, "fwd_ms": round(t_f, 3), "bwd_ms": round(t_b, 3),
              "fwd_tflops": round(fwd_flops / (t_f * 1e-3) / 1e12, 1),
              "bwd_tflops": round(bwd_flops / (t_b * 1e-3) / 1e12, 1),
              "peak_device_bytes": int(peak), "index_bytes": int(idx_bytes), "bwd_workspace_bytes": int(ws_bytes)}
        points.append(pt)
        log(f"sweep T={T}: fwd {pt['fwd_ms']} ms ({pt['fwd_tflops']} TF/s) bwd {pt['bwd_ms']} ms "
            f"({pt['bwd_tflops']} TF/s) peak {peak / 2**30:.2f} GiB")
        del q, k, v, do, index, ws, o, o_lo, lse, dq, dk, dv, desc_dev
        T *= 2
    print(json.dumps({"sweep": {"mask": spec.kind, "Hq": Hq, "Hk": Hk, "head_dim": d, "dtype": "bf16",
                                "data": "synthetic", "seed": args.seed}, "points": points}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="causal_8k_gqa", choices=sorted(workloads(0)))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-heads", type=int, default=2, help="query heads in the oracle timing sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch each step's kernels one by one instead of replaying a captured HIP graph")
    ap.add_argument("--out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--sweep", action="store_true",
                    help="sequence-length sweep (1K .. --sweep-max, powers of two) of one mask at GQA 64:8: "
                         "forward / backward TFLOP/s and peak device memory per length; prints one JSON line")
    ap.add_argument("--sweep-mask", default="causal", choices=["causal", "full"])
    ap.add_argument("--sweep-max", type=int, default=524288)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run attn_cast_bf16 over 2^28 floats 5 times (reads 1 GiB, writes 512 MiB "
                         "per launch): the known-size kernel that scales the HBM byte counters")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="only time torch.matmul (the ROCm BLAS library) on bf16 square matrices of 8192 and "
                         "16384: the dense-GEMM rate this GPU reaches, as context for the attention kernels' "
                         "fractions of the published MFMA peak; prints one JSON line")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the attention path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the per-GPU share of a sharded run is the 1-GPU workload).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    attn.lib()   # fail loudly if the HIP library is missing

    if args.sweep:
        sweep(args, torch, dev)
        return

    if args.gemm_reference:
        res = []
        for n in (8192, 16384):
            g = torch.Generator(device=dev).manual_seed(args.seed)
            a_ = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
            b_ = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
            for _ in range(3):
                c_ = a_ @ b_
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 20
            e0.record()
            for _ in range(reps):
                c_ = a_ @ b_
            e1.record()
            e1.synchronize()
            ms = e0.elapsed_time(e1) / reps
            res.append({"n": n, "ms": round(ms, 4), "tflops": round(2 * n ** 3 / ms / 1e9, 1),
                        "frac_peak": round(2 * n ** 3 / ms / 1e9 / PEAK_BF16_TFLOPS, 4)})
            del a_, b_, c_
        print(json.dumps({"gemm_reference": {"op": "torch.matmul bf16 (n x n) @ (n x n)", "points": res,
                                             "peak_tflops": PEAK_BF16_TFLOPS}}))
        return

    if args.copy_calibration:
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty(n, dtype=torch.bfloat16, device=dev)
        for _ in range(5):
            attn.cast_bf16(src.data_ptr(), dst.data_ptr(), n, torch.cuda.current_stream(dev).cuda_stream)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"kernel": "cast_kernel", "launches": 5,
                                               "read_bytes": 4 * n, "write_bytes": 2 * n}}))
        return

    wl = workloads(args.seed)[args.workload]
    T, Hq, Hk, d, spec = wl.T, wl.Hq, wl.Hk, wl.d, wl.mask
    log(f"workload {wl.name}: T={T} Hq={Hq} Hk={Hk} mask={spec.kind}")
    x = attention_inputs(args.seed, T, Hq, Hk)
    keep = keep_for(wl, args.seed)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = up(x["q"]), up(x["k"]), up(x["v"]), up(x["do"])
    keep_oracle = keep
    if spec.kind == "variable_block":
        keep = attn.variable_block_expand(T, Hq, spec.row_offsets, spec.col_offsets, keep)
        spec = MaskSpec("block_sparse", sparse_block=64)
    dynamic = wl.select is not None
    sparse = spec.kind == "block_sparse"
    prob = attn.problem(T, Hq, Hk, spec.kind, spec.sparse_block if sparse else 0)
    idx_bytes = attn.tile_index_size(prob)
    index = torch.empty(idx_bytes, dtype=torch.uint8, device=dev)
    desc_dev = torch.empty((T, 4), dtype=torch.int32, device=dev)
    if dynamic:
        nb = -(-T // spec.sparse_block)
        keep_dev = torch.empty((Hq, nb, nb), dtype=torch.uint8, device=dev)
        scores = torch.empty((Hq, nb, nb), dtype=torch.float32, device=dev)
        sel_bytes = attn.block_select_workspace_size(prob)
        sel_ws = torch.empty(sel_bytes, dtype=torch.uint8, device=dev)
        mode, val = wl.select
        sel_params = attn.block_select_params(mode, topk=int(val) if mode == "topk" else 0,
                                              topp=float(val) if mode == "topp" else 0.0, keep_diagonal=True)
    else:
        keep_dev = torch.from_numpy(keep).to(dev) if sparse else None
    o = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
    o_lo = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    dq = torch.empty((T, Hq, d), dtype=torch.float32, device=dev)
    dk = torch.empty((T, Hk, d), dtype=torch.float32, device=dev)
    dv = torch.empty((T, Hk, d), dtype=torch.float32, device=dev)
    ws_bytes = attn.bwd_workspace_size(prob)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    cu_dev = None
    if not sparse and spec.cu_seqlens:
        # the document boundaries are an input of the problem, resident like Q, K, V
        cu_dev = torch.tensor(spec.cu_seqlens, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
    times = {"select": [], "index": [], "fwd": [], "bwd_pre": [], "bwd_dkdv": [], "bwd_dq": []}

    def step(record: bool):
        cur = torch.cuda.current_stream(dev)   # the capture stream inside a graph
        sp = cur.cuda_stream

        def mark(i):
            if record:
                ev[i].record(cur)

        if sparse:
            mark(6)
            if dynamic:
                attn.block_select(prob, sel_params, q.data_ptr(), k.data_ptr(), scores.data_ptr(),
                                  keep_dev.data_ptr(), sel_ws.data_ptr(), sel_bytes, sp)
            mark(0)
            attn.block_index_build(prob, keep_dev.data_ptr(), index.data_ptr(), idx_bytes, sp)
        else:
            mark(6)
            mark(0)
            attn.mask_desc_build_device(spec, T, 0 if cu_dev is None else cu_dev.data_ptr(),
                                        desc_dev.data_ptr(), sp)                                # a1 (device)
            attn.tile_index_build(prob, desc_dev.data_ptr(), index.data_ptr(), idx_bytes, sp)   # a2
        mark(1)
        attn.fwd(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), o_lo.data_ptr(), lse.data_ptr(),
                 0 if sparse else desc_dev.data_ptr(), index.data_ptr(), idx_bytes, 0, 0, sp)       # a3
        mark(2)
        attn.bwd_preprocess(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), o_lo.data_ptr(),
                            do.data_ptr(), ws.data_ptr(), ws_bytes, sp)                                     # a4
        mark(3)
        attn.bwd_dkdv(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), do.data_ptr(),
                      dk.data_ptr(), dv.data_ptr(), 0 if sparse else desc_dev.data_ptr(),
                      index.data_ptr(), idx_bytes, ws.data_ptr(), ws_bytes, sp)                     # a5 (dK, dV)
        mark(4)
        attn.bwd_dq(prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), do.data_ptr(),
                    dq.data_ptr(), 0 if sparse else desc_dev.data_ptr(),
                    index.data_ptr(), idx_bytes, ws.data_ptr(), ws_bytes, sp)                       # a5 (dQ)
        mark(5)
        if record:
            ev[5].synchronize()
            times["select"].append(ev[6].elapsed_time(ev[0]))
            times["index"].append(ev[0].elapsed_time(ev[1]))
            times["fwd"].append(ev[1].elapsed_time(ev[2]))
            times["bwd_pre"].append(ev[2].elapsed_time(ev[3]))
            times["bwd_dkdv"].append(ev[3].elapsed_time(ev[4]))
            times["bwd_dq"].append(ev[4].elapsed_time(ev[5]))

    log(f"warmup {args.warmup} steps")
    for _ in range(max(1, args.warmup)):
        step(False)
    torch.cuda.synchronize()

    desc_host = None if sparse else attn.mask_desc_build(spec, T)
    if dynamic:
        keep = keep_dev.cpu().numpy()   # the selection is the same in every step (fixed inputs)
    U, U_all = visible_pairs(spec, T, desc_host, keep)
    # block-sparse U differs per head: use the exact total over heads
    fwd_flops = 4.0 * d * (U_all if U_all is not None else Hq * U)
    bwd_flops = 2.5 * fwd_flops

    # one step's launches captured into a HIP graph, replayed by the timed steps (the same
    # kernels on the same buffers; --no-graph launches them one by one instead)
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(False)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    log(f"timing {args.steps} steps ({'graph replays' if graph is not None else 'eager launches'})")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step(False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps

    # per-kernel event times over a second pass of the same steps
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    med = {k: float(np.median(v)) for k, v in times.items()}
    mean = {k: float(np.mean(v)) for k, v in times.items()}
    t_bwd = med["bwd_pre"] + med["bwd_dkdv"] + med["bwd_dq"]
    fwd_tf = fwd_flops / (med["fwd"] * 1e-3) / 1e12
    bwd_tf = bwd_flops / (t_bwd * 1e-3) / 1e12
    # dominant kernel: bwd_kernel (attn_bwd_dkdv), algorithmic work = the S, dP, dV and dK
    # products over the visible pairs = 8 * d * Hq * U
    dkdv_flops = 0.8 * bwd_flops
    dkdv_tf = dkdv_flops / (mean["bwd_dkdv"] * 1e-3) / 1e12
    value = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms | select {med['select']:.3f} index {med['index']:.3f} fwd {med['fwd']:.3f} "
        f"bwd_pre {med['bwd_pre']:.3f} dkdv {med['bwd_dkdv']:.3f} dq {med['bwd_dq']:.3f} ms | "
        f"fwd {fwd_tf:.1f} TF/s bwd {bwd_tf:.1f} TF/s")

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "mask": spec.kind, "T": T, "Hq": Hq, "Hk": Hk, "head_dim": d,
                   "global_batch": 1, "seq_len": T, "parallelism": "none", "seed": args.seed,
                   "launch": "hip graph" if graph is not None else "eager",
                   **({"select": list(wl.select)} if dynamic else {}),
                   **({"sparse_block": spec.sparse_block} if sparse else {})},
        "visible_pairs_per_head": U,
        "fwd": {"ms": round(med["fwd"], 4), "tflops": round(fwd_tf, 2),
                "frac_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4)},
        "bwd": {"ms": round(t_bwd, 4), "tflops": round(bwd_tf, 2),
                "frac_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
                "preprocess_ms": round(med["bwd_pre"], 4), "dkdv_ms": round(med["bwd_dkdv"], 4),
                "dq_ms": round(med["bwd_dq"], 4)},
        "index_build_ms": round(med["index"], 4),
        **({"select_ms": round(med["select"], 4)} if dynamic else {}),
        "roofline": {"kernel": "bwd_kernel (attn_bwd_dkdv)", "bound": "mfma",
                     "achieved": round(dkdv_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dkdv_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for(wl.name, "bwd_kernel"),
                     # not measured in this run: HBM bytes per launch from the committed
                     # rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of this workload, valid only
                     # while the kernel sources hash the same (null otherwise)
                     "traffic_source": (f"profiles/traffic_bwd_kernel_{wl.name}.json (rocprofv3 --pmc, "
                                        f"kernel hash {kernel_hash()})"
                                        if traffic_for(wl.name, "bwd_kernel") is not None else None),
                     "avg_launch_ms": round(mean["bwd_dkdv"], 4),
                     "flops_per_launch": dkdv_flops},
        "kernel_hash": kernel_hash(),
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_heads} heads")
        rec["cpu_baseline"] = cpu_baseline(wl, x, keep_oracle, args.cpu_heads)
    else:
        rec["cpu_baseline"] = None
    line = json.dumps(rec)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
