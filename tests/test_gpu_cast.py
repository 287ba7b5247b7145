"""attn_cast_bf16 (the optional fp32 -> bf16 cast of the gradients) against the oracle's
round to nearest even, bit for bit: random bit patterns of every class (normals,
subnormals, zeros, infinities, NaNs), every low half-word at one exponent (all ties and
near-ties), the overflow to infinity, and lengths that are not a multiple of the grid's
stride. A NaN must stay a NaN (its payload is not part of the contract)."""
import numpy as np
import pytest

from masked_long_context_tiled_amd import attn
from oracle.cast import f32_to_bf16_rne

from gpu_helpers import note

pytestmark = pytest.mark.gpu


def _bits(n, seed):
    rng = np.random.default_rng(seed)
    b = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
    m = min(n, 65536)
    b[:m] = (0x3F80 << 16) | np.arange(m, dtype=np.uint32)
    extra = np.array([0x7F7FFFFF, 0x7F7F7FFF, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFF800001,
                      0x00000001, 0x80008000, 0x00018000, 0x007FFFFF, 0x00000000, 0x80000000],
                     dtype=np.uint32)
    if n >= 65536 + len(extra):
        b[65536:65536 + len(extra)] = extra
    return b


@pytest.mark.parametrize("n", [1, 1000, 524_288 + 37, 3_000_001])
def test_cast_bit_exact(n):
    import torch
    note(f"cast n={n}")
    bits = _bits(n, n)
    x = torch.from_numpy(bits.view(np.float32).copy()).cuda()
    out = torch.full((n,), 0x1234, dtype=torch.int16, device="cuda")
    attn.cast_bf16(x.data_ptr(), out.data_ptr(), n, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    want = f32_to_bf16_rne(bits.view(np.float32))
    nan = np.isnan(bits.view(np.float32))
    got_nan = (((got >> 7) & 0xFF) == 0xFF) & ((got & 0x7F) != 0)
    assert np.array_equal(got_nan, nan), "NaN in, NaN out (and nothing else a NaN)"
    bad = np.flatnonzero((got != want) & ~nan)
    assert bad.size == 0, f"{bad.size} values differ, first input 0x{bits[bad[0]]:08x}: got 0x{got[bad[0]]:04x} want 0x{want[bad[0]]:04x}"
