"""Write tests/golden/index_digests.json from the oracle alone.

For every dense workload at its full size, the oracle's tile classes (oracle.tiles:
brute force over the materialised mask), the CSR / CSC lists of the non-empty tiles and
their launch orders are reduced to SHA-256 digests of their canonical bytes, next to a
few counts that make a mismatch readable. The GPU test builds the same index through the
library and compares digests, so the full-size tile index is checked bit for bit without
rebuilding 10^10-cell masks where the GPU tests run.

Tile shapes are those of the kernels: forward tiles of 256 / G query positions x 64 keys,
backward tiles of 256 / G query positions x 128 keys (G = Hq / Hk); the test also checks
that the library reports these shapes.

Run: python tests/golden/make_index_digests.py   (a few minutes on 8 cores)
"""
import hashlib
import json
import os
import sys
from multiprocessing import Pool

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from masked_long_context_tiled_amd.inputs import workloads  # noqa: E402
from oracle.tiles import FULL, PARTIAL, launch_order, tile_classes, tile_csc, tile_csr  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "index_digests.json")

DENSE = ["causal_8k_gqa", "full_8k_gqa", "causal_8k_mha", "full_8k_mha",
         "full_document_32k", "causal_document_32k", "full_sliding_window_32k",
         "causal_sliding_window_32k", "shared_question_16k", "prefix_lm_causal_16k",
         "causal_blockwise_16k", "global_sliding_16k", "prefix_lm_document_32k",
         "block_causal_document_32k", "causal_128k"]


def digest(a, dtype):
    return hashlib.sha256(np.ascontiguousarray(a, dtype=dtype).tobytes()).hexdigest()


def map_digests(cls, lists):
    ptr, idx, full = lists
    return {"shape": list(cls.shape), "n_full": int((cls == FULL).sum()),
            "n_partial": int((cls == PARTIAL).sum()), "nnz": int(ptr[-1]),
            "cls": digest(cls, "u1"), "ptr": digest(ptr, "<i4"), "idx": digest(idx, "<i4"),
            "full": digest(full, "u1"), "order": digest(launch_order(ptr), "<i4")}


def one(name):
    wl = workloads(0)[name]
    G = wl.Hq // wl.Hk
    fbm, fbn, bbm, bbn = 256 // G, 64, 256 // G, 128
    fwd = tile_classes(wl.mask, wl.T, fbm, fbn)
    bwd = tile_classes(wl.mask, wl.T, bbm, bbn)
    rec = {"T": wl.T, "Hq": wl.Hq, "Hk": wl.Hk, "tiles": [fbm, fbn, bbm, bbn],
           "fwd": map_digests(fwd, tile_csr(fwd)), "bwd": map_digests(bwd, tile_csc(bwd))}
    print(f"{name}: fwd {rec['fwd']['shape']} nnz {rec['fwd']['nnz']}, "
          f"bwd {rec['bwd']['shape']} nnz {rec['bwd']['nnz']}", flush=True)
    return name, rec


if __name__ == "__main__":
    with Pool(int(os.environ.get("JOBS", "4"))) as pool:
        recs = dict(pool.map(one, DENSE))
    with open(OUT, "w") as f:
        json.dump({n: recs[n] for n in DENSE}, f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", OUT)
