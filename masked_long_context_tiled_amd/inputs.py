"""Seeded synthetic inputs shared by the CPU oracle tests, the GPU tests and the bench.

This module holds no attention arithmetic. It only:
  * names the mask kinds and carries their parameters (``MaskSpec``),
  * draws the random tensors (Q, K, V, dO) and rounds them to bf16 bit patterns,
  * draws the random structure the workloads need (document lengths for the
    packed-sequence masks, the keep matrix of a uniform block-sparse mask, the grid
    and keep matrix of a variable-block mask),
  * lists the workload configurations by name.

Both sides consume the same bits: the oracle upcasts the bf16 patterns to fp64,
the GPU path uploads them as bf16.

Source for the mask names and the problem shape: "LongCA-bench: 长上下文注意力基准测试"
(xllm-io paper-review blog), section 三 "注意力掩码模式" (the 12 static masks and the
two dynamic block masks) and section 四 "实验设置" (bf16, head dim 128, GQA 64:8 and
MHA 64:64, sequence length 1K-512K).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

# Mask kinds, in the order of the C enum ``attn_mask_kind``.
MASK_KINDS = (
    "full",
    "causal",
    "full_document",
    "causal_document",
    "full_sliding_window",
    "causal_sliding_window",
    "shared_question",
    "prefix_lm_causal",
    "causal_blockwise",
    "global_sliding",
    "block_sparse",
    "prefix_lm_document",
    "block_causal_document",
)

# Variable Block: block-sparse over a grid of variable block sizes. The library runs it as
# the uniform 64-block mask its grid expands to, so it has no kind of its own in the C enum.
VARIABLE_BLOCK = "variable_block"


@dataclass(frozen=True)
class MaskSpec:
    """A mask kind and its parameters (positions are 0-based, in one packed sequence).

    window          sliding window width w (FULL/CAUSAL SLIDING WINDOW, GLOBAL SLIDING)
    prefix_len      bidirectional prefix length (PREFIX LM CAUSAL; per document for
                    PREFIX LM DOCUMENT)
    question_len    shared question length (SHARED QUESTION)
    answer_len      length of each answer (SHARED QUESTION)
    n_answers       number of answers (SHARED QUESTION)
    block_len       causal block length (CAUSAL BLOCKWISE); block length within each
                    document (BLOCK CAUSAL DOCUMENT)
    final_block_len length of the final block that sees everything before it (CAUSAL BLOCKWISE)
    global_len      number of global tokens at the start (GLOBAL SLIDING)
    cu_seqlens      document boundaries, cu_seqlens[0] = 0, cu_seqlens[-1] = T (the four
                    DOCUMENT masks)
    sparse_block    block edge b of a uniform block-sparse mask (64 or 128)
    row_offsets     variable-block grid: row block r is [row_offsets[r], row_offsets[r+1])
    col_offsets     and column block c is [col_offsets[c], col_offsets[c+1]) (0 ... T)
    """

    kind: str
    window: int = 0
    prefix_len: int = 0
    question_len: int = 0
    answer_len: int = 0
    n_answers: int = 0
    block_len: int = 0
    final_block_len: int = 0
    global_len: int = 0
    cu_seqlens: Tuple[int, ...] = field(default_factory=tuple)
    sparse_block: int = 0
    row_offsets: Tuple[int, ...] = field(default_factory=tuple)
    col_offsets: Tuple[int, ...] = field(default_factory=tuple)

    def __post_init__(self):
        if self.kind not in MASK_KINDS and self.kind != VARIABLE_BLOCK:
            raise ValueError(f"unknown mask kind {self.kind!r}")

    @property
    def kind_id(self) -> int:
        return MASK_KINDS.index(self.kind)

    def with_(self, **kw) -> "MaskSpec":
        return replace(self, **kw)


# ---------------------------------------------------------------------------
# bf16 bit patterns
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (round to nearest, ties to even); return uint16 bits.

    For finite inputs the 32-bit sum below cannot overflow (the largest, 0xFF7FFFFF + 0x8000,
    stays below 2^32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------------------
# Random tensors
# ---------------------------------------------------------------------------

def attention_inputs(seed: int, T: int, Hq: int, Hk: int, d: int = 128,
                     with_do: bool = True) -> dict:
    """Q [T][Hq][d], K/V [T][Hk][d], dO [T][Hq][d] as bf16 bit patterns (uint16).

    Drawn i.i.d. N(0,1) in float32 from ``numpy.random.default_rng(seed)`` in the
    order Q, K, V, dO, then rounded to bf16.
    """
    rng = np.random.default_rng(seed)
    out = {}
    out["q"] = f32_to_bf16_bits(rng.standard_normal((T, Hq, d), dtype=np.float32))
    out["k"] = f32_to_bf16_bits(rng.standard_normal((T, Hk, d), dtype=np.float32))
    out["v"] = f32_to_bf16_bits(rng.standard_normal((T, Hk, d), dtype=np.float32))
    if with_do:
        out["do"] = f32_to_bf16_bits(rng.standard_normal((T, Hq, d), dtype=np.float32))
    return out


def attention_inputs_device(seed: int, T: int, Hq: int, Hk: int, device, d: int = 128,
                            chunk: int = 16384) -> dict:
    """Q [T][Hq][d], K/V [T][Hk][d], dO [T][Hq][d] as bf16 tensors drawn on ``device``.

    For lengths whose inputs are too large to draw on the host (512K: Q and dO hold 2^32
    values each): i.i.d. N(0,1) float32 from one ``torch.Generator`` on the device seeded
    with ``seed``, drawn in the order Q, K, V, dO and, within each tensor, in blocks of
    ``chunk`` positions, each block rounded to bf16 (round to nearest even) as it is drawn.
    The same arguments give the same bits on the same software stack; a test copies the
    rows it checks back to the host for the oracle.
    """
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = {}
    for name, H in (("q", Hq), ("k", Hk), ("v", Hk), ("do", Hq)):
        t = torch.empty((T, H, d), dtype=torch.bfloat16, device=device)
        for r0 in range(0, T, chunk):
            r1 = min(T, r0 + chunk)
            t[r0:r1] = torch.randn((r1 - r0, H, d), generator=gen, device=device,
                                   dtype=torch.float32).to(torch.bfloat16)
        out[name] = t
    return out


def document_cu_seqlens(seed: int, total: int, lo: int = 512, hi: int = 8192) -> Tuple[int, ...]:
    """Packed-sequence document boundaries.

    Lengths are integers uniform on [lo, hi] (inclusive), drawn one after another
    from ``default_rng(seed)`` until they cover ``total``; the last one is cut so the
    lengths sum to exactly ``total``.
    """
    rng = np.random.default_rng(seed)
    cu = [0]
    while cu[-1] < total:
        n = int(rng.integers(lo, hi + 1))
        cu.append(min(total, cu[-1] + n))
    return tuple(cu)


def block_sparse_keep(seed: int, Hq: int, nqb: int, nkb: int) -> np.ndarray:
    """Keep matrix uint8 [Hq][nqb][nkb] of a uniform block-sparse mask at 50% density.

    For every (query head, query block) exactly floor(nkb/2) key blocks are kept
    (at least one): the diagonal block r (when r < nkb) is always kept, the rest are
    the smallest of i.i.d. uniform keys drawn from ``default_rng(seed)``.
    """
    rng = np.random.default_rng(seed)
    keys = rng.random((Hq, nqb, nkb))
    r = np.arange(min(nqb, nkb))
    keys[:, r, r] = -1.0
    n_keep = max(1, nkb // 2)
    order = np.argsort(keys, axis=2, kind="stable")[:, :, :n_keep]
    keep = np.zeros((Hq, nqb, nkb), dtype=np.uint8)
    np.put_along_axis(keep, order, 1, axis=2)
    return keep


def variable_block_grid(seed: int, T: int, unit: int = 64, max_units: int = 8) -> Tuple[int, ...]:
    """Block edges 0 = o_0 < o_1 < ... < o_n = T of a variable-block grid.

    Block sizes are unit * m with m uniform on 1 .. max_units, drawn one after another
    from ``default_rng(seed)`` until they cover T; the last block is cut at T.
    """
    rng = np.random.default_rng(seed)
    off = [0]
    while off[-1] < T:
        off.append(min(T, off[-1] + unit * int(rng.integers(1, max_units + 1))))
    return tuple(off)


def variable_block_keep(seed: int, Hq: int, row_offsets, col_offsets) -> np.ndarray:
    """Keep matrix uint8 [Hq][n_row_blocks][n_col_blocks] of a variable-block mask.

    For every (query head, row block) the column blocks are visited in a random order
    (``default_rng(seed)``, one permutation per row) and kept until they cover at least
    half of the T keys, so every row block sees about 50 % of the keys and at least one
    block.
    """
    rng = np.random.default_rng(seed)
    nr, nc = len(row_offsets) - 1, len(col_offsets) - 1
    size = np.diff(np.asarray(col_offsets, dtype=np.int64))
    T = int(col_offsets[-1])
    keep = np.zeros((Hq, nr, nc), dtype=np.uint8)
    for h in range(Hq):
        for r in range(nr):
            covered = 0
            for c in rng.permutation(nc):
                if covered * 2 >= T:
                    break
                keep[h, r, c] = 1
                covered += int(size[c])
    return keep


# ---------------------------------------------------------------------------
# Workload configurations (mask shapes of the benchmark pages' workloads)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    Hq: int
    Hk: int
    mask: MaskSpec
    d: int = 128
    # dynamic block-sparse: the keep matrix is selected from Q and K in every step,
    # ("topk", k) or ("topp", p), the diagonal block always kept
    select: Optional[Tuple[str, float]] = None


def workloads(seed: int = 0) -> dict:
    """Named workloads. Document boundaries depend on ``seed``."""
    cu32 = document_cu_seqlens(seed, 32768)
    w = {}
    w["tiny_causal"] = Workload("tiny_causal", 512, 4, 1, MaskSpec("causal"))
    for hk in (8, 64):
        tag = "gqa" if hk == 8 else "mha"
        w[f"full_8k_{tag}"] = Workload(f"full_8k_{tag}", 8192, 64, hk, MaskSpec("full"))
        w[f"causal_8k_{tag}"] = Workload(f"causal_8k_{tag}", 8192, 64, hk, MaskSpec("causal"))
    w["full_document_32k"] = Workload("full_document_32k", 32768, 64, 8,
                                      MaskSpec("full_document", cu_seqlens=cu32))
    w["causal_document_32k"] = Workload("causal_document_32k", 32768, 64, 8,
                                        MaskSpec("causal_document", cu_seqlens=cu32))
    w["full_sliding_window_32k"] = Workload("full_sliding_window_32k", 32768, 64, 8,
                                            MaskSpec("full_sliding_window", window=4096))
    w["causal_sliding_window_32k"] = Workload("causal_sliding_window_32k", 32768, 64, 8,
                                              MaskSpec("causal_sliding_window", window=4096))
    w["shared_question_16k"] = Workload(
        "shared_question_16k", 16384, 64, 8,
        MaskSpec("shared_question", question_len=2048, answer_len=3584, n_answers=4))
    w["prefix_lm_causal_16k"] = Workload("prefix_lm_causal_16k", 16384, 64, 8,
                                         MaskSpec("prefix_lm_causal", prefix_len=4096))
    w["causal_blockwise_16k"] = Workload(
        "causal_blockwise_16k", 16384, 64, 8,
        MaskSpec("causal_blockwise", block_len=1024, final_block_len=2048))
    w["global_sliding_16k"] = Workload("global_sliding_16k", 16384, 64, 8,
                                       MaskSpec("global_sliding", global_len=128, window=2048))
    w["prefix_lm_document_32k"] = Workload("prefix_lm_document_32k", 32768, 64, 8,
                                           MaskSpec("prefix_lm_document", prefix_len=1024,
                                                    cu_seqlens=cu32))
    w["block_causal_document_32k"] = Workload("block_causal_document_32k", 32768, 64, 8,
                                              MaskSpec("block_causal_document", block_len=256,
                                                       cu_seqlens=cu32))
    w["causal_128k"] = Workload("causal_128k", 131072, 64, 8, MaskSpec("causal"))
    for b in (128, 64):
        w[f"block_sparse_64k_b{b}"] = Workload(f"block_sparse_64k_b{b}", 65536, 64, 8,
                                               MaskSpec("block_sparse", sparse_block=b))
    w["topk_sparse_64k_b128"] = Workload("topk_sparse_64k_b128", 65536, 64, 8,
                                         MaskSpec("block_sparse", sparse_block=128), select=("topk", 256))
    w["topp_sparse_64k_b128"] = Workload("topp_sparse_64k_b128", 65536, 64, 8,
                                         MaskSpec("block_sparse", sparse_block=128), select=("topp", 0.5))
    w["variable_block_64k"] = Workload(
        "variable_block_64k", 65536, 64, 8,
        MaskSpec(VARIABLE_BLOCK, row_offsets=variable_block_grid(seed, 65536),
                 col_offsets=variable_block_grid(seed + 1, 65536)))
    return w


def keep_for(workload: Workload, seed: int) -> Optional[np.ndarray]:
    """The keep matrix of a block-sparse or variable-block workload (None for other masks
    and for dynamic workloads, whose keep matrix is selected from the inputs)."""
    if workload.select is not None:
        return None
    if workload.mask.kind == VARIABLE_BLOCK:
        return variable_block_keep(seed, workload.Hq, workload.mask.row_offsets, workload.mask.col_offsets)
    if workload.mask.kind != "block_sparse":
        return None
    b = workload.mask.sparse_block
    nb = -(-workload.T // b)
    return block_sparse_keep(seed, workload.Hq, nb, nb)
