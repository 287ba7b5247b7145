import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from masked_long_context_tiled_amd.inputs import MaskSpec  # noqa: E402

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: larger CPU cases")


def load_golden_masks(path=None):
    """Parse tests/golden/masks_T12.txt -> list of (MaskSpec, keep or None, uint8 [12][12])."""
    path = path or os.path.join(GOLDEN, "masks_T12.txt")
    out = []
    cur = None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("=="):
                parts = line[2:].split()
                kind, kv = parts[0], dict(p.split("=") for p in parts[1:])
                keep = None
                args = {}
                for key, val in kv.items():
                    if key == "cu_seqlens":
                        args[key] = tuple(int(x) for x in val.split(","))
                    elif key == "keep":
                        keep = np.array([[int(c) for c in r] for r in val.split("/")],
                                        dtype=np.uint8)[None]
                    else:
                        args[key] = int(val)
                cur = [MaskSpec(kind, **args), keep, []]
                out.append(cur)
            else:
                cur[2].append([int(c) for c in line])
    return [(s, k, np.array(m, dtype=np.uint8)) for s, k, m in out]
