"""Pins for the oracle's fp32 -> bf16 round-to-nearest-even (CPU only): hand-worked values
(ties to even in both directions, the carry into the exponent, overflow to infinity,
subnormals) and PyTorch's CPU conversion (a library routine) on every class of bit
pattern."""
import numpy as np
import torch

from oracle.cast import f32_to_bf16_rne


def _f(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


def test_hand_values():
    cases = {
        0x3F800000: 0x3F80,   # 1.0
        0x3F808000: 0x3F80,   # 1 + 2^-8: tie, kept pattern even -> down
        0x3F818000: 0x3F82,   # 1 + 3 * 2^-8: tie, kept pattern odd -> up
        0x3F808001: 0x3F81,   # just above the tie -> up
        0x3F807FFF: 0x3F80,   # just below the tie -> down
        0xBF818000: 0xBF82,   # negative ties round the magnitude the same way
        0x3FFFFFFF: 0x4000,   # carry into the exponent: 1.99999988 -> 2.0
        0x7F7FFFFF: 0x7F80,   # largest finite fp32 -> +inf
        0x7F7F7FFF: 0x7F7F,   # largest value that stays finite
        0x7F800000: 0x7F80,   # +inf
        0xFF800000: 0xFF80,   # -inf
        0x00000000: 0x0000,
        0x80000000: 0x8000,   # -0
        0x00008000: 0x0000,   # smallest subnormal tie at an even pattern -> 0
        0x00018000: 0x0002,   # subnormal tie at an odd pattern -> up
        0x007FFFFF: 0x0080,   # largest subnormal -> smallest normal
    }
    got = f32_to_bf16_rne(_f(list(cases)))
    assert got.tolist() == list(cases.values())


def test_nan_stays_nan():
    x = _f([0x7FC00000, 0x7F800001, 0xFFFFFFFF, 0x7FBFFFFF])
    got = f32_to_bf16_rne(x)
    e = (got >> 7) & 0xFF
    assert np.all(e == 0xFF) and np.all((got & 0x7F) != 0)


def test_against_torch_every_class():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    bits[:65536] = (0x3F80 << 16) | np.arange(65536, dtype=np.uint32)   # every low half at 1.x
    bits[65536:131072] = np.arange(65536, dtype=np.uint32)               # subnormals near 0
    x = bits.view(np.float32)
    fin = ~np.isnan(x)
    want = torch.from_numpy(x[fin].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_rne(x[fin]), want)
