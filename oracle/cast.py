"""fp32 -> bf16 conversion by round to nearest, ties to even (oracle; test infrastructure only).

The pages run attention in bf16 ("LongCA-bench: 长上下文注意力基准测试", xllm-io blog,
section 四 "实验设置"); gradients computed in fp32 are handed to bf16 consumers by the
IEEE 754 conversion to the narrower format, which rounds to nearest with ties to even.
bf16 keeps the sign, the 8-bit exponent and the top 7 fraction bits of fp32, so on the
bit pattern b (uint32) of a finite value the conversion is

    drop the low 16 bits, rounding up iff they exceed 0x8000, or equal 0x8000 while the
    kept pattern is odd

(a round-up that carries into the exponent is exact: the largest finite values round to
infinity). Infinities keep their sign; a NaN stays a NaN (its payload is not fixed here).
Subnormal inputs round the same way, since both formats share the exponent field.
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_rne(x):
    """float32 array -> uint16 bf16 patterns; NaN inputs give 0x7FC0 with the input's sign
    (callers compare NaN-ness only)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    hi = b >> 16
    lo = b & 0xFFFF
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    out = (hi + up.astype(np.uint64)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    out[nan] = (0x7FC0 | (hi[nan] & 0x8000)).astype(np.uint16)
    return out
