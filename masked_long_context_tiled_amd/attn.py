"""ctypes binding of libattn.so (include/attn.h): argument marshalling only.

Every step of the attention path runs in the library's HIP kernels. The functions
below mirror the C entry points one to one (same names without the ``attn_`` prefix)
and take raw device pointers as Python ints; ``MaskedAttention`` is a small helper
that allocates the buffers with PyTorch and passes their pointers through. If the
shared library has not been built this module raises on first use: there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import numpy as np

from .inputs import MASK_KINDS, VARIABLE_BLOCK, MaskSpec

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLCT_ATTN_LIB names another build of the same library (the CPU tests point it at the
# host-only sanitizer build, whose kernel launchers abort); by default the in-tree build.
LIB_PATH = os.environ.get("MLCT_ATTN_LIB") or os.path.join(_HERE, "libattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "attn.h")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(5)


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


class attn_mask_params(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("prefix_len", ctypes.c_int32),
        ("question_len", ctypes.c_int32),
        ("answer_len", ctypes.c_int32),
        ("n_answers", ctypes.c_int32),
        ("block_len", ctypes.c_int32),
        ("final_block_len", ctypes.c_int32),
        ("global_len", ctypes.c_int32),
        ("n_docs", ctypes.c_int32),
        ("cu_seqlens", ctypes.POINTER(ctypes.c_int32)),
    ]


class attn_problem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32),
        ("Hq", ctypes.c_int32),
        ("Hk", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("mask_kind", ctypes.c_int32),
        ("sparse_block", ctypes.c_int32),
    ]


class attn_block_select_params(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("topp", ctypes.c_float),
        ("keep_diagonal", ctypes.c_int32),
    ]


ATTN_SELECT_TOPK, ATTN_SELECT_TOPP = 0, 1


class attn_index_layout(ctypes.Structure):
    _fields_ = [
        ("nqt_f", ctypes.c_int32), ("nkt_f", ctypes.c_int32),
        ("nqt_b", ctypes.c_int32), ("nkt_b", ctypes.c_int32),
        ("fwd_cls", ctypes.c_size_t), ("fwd_ptr", ctypes.c_size_t),
        ("fwd_ent", ctypes.c_size_t), ("fwd_order", ctypes.c_size_t),
        ("bwd_cls", ctypes.c_size_t), ("bwd_ptr", ctypes.c_size_t),
        ("bwd_ent", ctypes.c_size_t), ("bwd_order", ctypes.c_size_t),
        ("total_bytes", ctypes.c_size_t),
    ]


_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_PROB = ctypes.POINTER(attn_problem)
_SIGS = {
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_mask_desc_build": (ctypes.c_int, [ctypes.POINTER(attn_mask_params), ctypes.c_int32, _P]),
    "attn_tile_index_size": (ctypes.c_int, [_PROB, ctypes.POINTER(_SZ)]),
    "attn_query_tile_shape": (ctypes.c_int, [_PROB] + [ctypes.POINTER(ctypes.c_int32)] * 4),
    "attn_tile_index_layout": (ctypes.c_int, [_PROB, ctypes.POINTER(attn_index_layout)]),
    "attn_tile_index_build": (ctypes.c_int, [_PROB, _P, _P, _SZ, _P]),
    "attn_block_index_build": (ctypes.c_int, [_PROB, _P, _P, _SZ, _P]),
    "attn_fwd_workspace_size": (ctypes.c_int, [_PROB, ctypes.POINTER(_SZ)]),
    "attn_bwd_workspace_size": (ctypes.c_int, [_PROB, ctypes.POINTER(_SZ)]),
    "attn_fwd": (ctypes.c_int, [_PROB, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P]),
    "attn_bwd": (ctypes.c_int, [_PROB, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P]),
    "attn_bwd_preprocess": (ctypes.c_int, [_PROB, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "attn_bwd_main": (ctypes.c_int, [_PROB, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P]),
    "attn_bwd_dkdv": (ctypes.c_int, [_PROB, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P]),
    "attn_bwd_dq": (ctypes.c_int, [_PROB, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P]),
    "attn_cast_bf16": (ctypes.c_int, [_P, _P, _SZ, _P]),
    "attn_mask_desc_build_device": (ctypes.c_int, [ctypes.POINTER(attn_mask_params), ctypes.c_int32, _P, _P, _P]),
    "attn_mask_desc_build_chunk": (ctypes.c_int, [ctypes.POINTER(attn_mask_params), ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_int32, _P]),
    "attn_lse_merge": (ctypes.c_int, [_PROB, _P, _P, _P, _P, _P, _P, _P]),
    "attn_block_select_workspace_size": (ctypes.c_int, [_PROB, ctypes.POINTER(_SZ)]),
    "attn_block_select": (ctypes.c_int, [_PROB, ctypes.POINTER(attn_block_select_params), _P, _P, _P, _P, _P,
                                         _SZ, _P]),
    "attn_block_select_noalloc": (ctypes.c_int, [_PROB, ctypes.POINTER(attn_block_select_params), _P, _P, _P, _P,
                                                 _P]),
    "attn_variable_block_expand": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P,
                                                  ctypes.c_int32, _P, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m masked_long_context_tiled_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_functions(path: str = HEADER_PATH):
    """Names of the functions declared in include/attn.h."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def status_string(s: int) -> str:
    return lib().attn_status_string(int(s)).decode()


def _check(s: int, where: str):
    if s != ATTN_OK:
        raise AttnError(s, where)


def kind_id(kind) -> int:
    return MASK_KINDS.index(kind) if isinstance(kind, str) else int(kind)


def problem(T: int, Hq: int, Hk: int, mask_kind, sparse_block: int = 0, scale: float = 0.0,
            head_dim: int = 128) -> attn_problem:
    return attn_problem(int(T), int(Hq), int(Hk), int(head_dim), float(scale), kind_id(mask_kind),
                        int(sparse_block))


def mask_params(spec: MaskSpec):
    """(attn_mask_params, keepalive) for a MaskSpec."""
    cu = np.ascontiguousarray(np.asarray(spec.cu_seqlens, dtype=np.int32))
    p = attn_mask_params(
        spec.kind_id, spec.window, spec.prefix_len, spec.question_len, spec.answer_len,
        spec.n_answers, spec.block_len, spec.final_block_len, spec.global_len,
        max(0, len(cu) - 1),
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if len(cu) else None)
    return p, cu


# --- one-to-one wrappers -------------------------------------------------------------

def mask_desc_build(spec: MaskSpec, T: int) -> np.ndarray:
    """Host column-interval descriptor int32 [T][4]."""
    p, keep = mask_params(spec)
    out = np.empty((T, 4), dtype=np.int32)
    _check(lib().attn_mask_desc_build(ctypes.byref(p), int(T), out.ctypes.data), "attn_mask_desc_build")
    return out


def tile_index_size(prob: attn_problem) -> int:
    n = _SZ()
    _check(lib().attn_tile_index_size(ctypes.byref(prob), ctypes.byref(n)), "attn_tile_index_size")
    return n.value


def query_tile_shape(prob: attn_problem):
    v = [ctypes.c_int32() for _ in range(4)]
    _check(lib().attn_query_tile_shape(ctypes.byref(prob), *[ctypes.byref(x) for x in v]),
           "attn_query_tile_shape")
    return tuple(x.value for x in v)


def tile_index_layout(prob: attn_problem) -> dict:
    lay = attn_index_layout()
    _check(lib().attn_tile_index_layout(ctypes.byref(prob), ctypes.byref(lay)), "attn_tile_index_layout")
    return {name: getattr(lay, name) for name, _ in attn_index_layout._fields_}


def tile_index_build(prob, desc_dev: int, index_dev: int, index_bytes: int, stream: int = 0):
    _check(lib().attn_tile_index_build(ctypes.byref(prob), desc_dev, index_dev, index_bytes, stream),
           "attn_tile_index_build")


def block_index_build(prob, keep_dev: int, index_dev: int, index_bytes: int, stream: int = 0):
    _check(lib().attn_block_index_build(ctypes.byref(prob), keep_dev, index_dev, index_bytes, stream),
           "attn_block_index_build")


def fwd_workspace_size(prob) -> int:
    n = _SZ()
    _check(lib().attn_fwd_workspace_size(ctypes.byref(prob), ctypes.byref(n)), "attn_fwd_workspace_size")
    return n.value


def bwd_workspace_size(prob) -> int:
    n = _SZ()
    _check(lib().attn_bwd_workspace_size(ctypes.byref(prob), ctypes.byref(n)), "attn_bwd_workspace_size")
    return n.value


def fwd(prob, q, k, v, o, o_lo, lse, desc, index, index_bytes, ws, ws_bytes, stream=0):
    _check(lib().attn_fwd(ctypes.byref(prob), q, k, v, o, o_lo, lse, desc, index, index_bytes, ws, ws_bytes,
                          stream), "attn_fwd")


def bwd(prob, q, k, v, o, o_lo, lse, dout, dq, dk, dv, desc, index, index_bytes, ws, ws_bytes, stream=0):
    _check(lib().attn_bwd(ctypes.byref(prob), q, k, v, o, o_lo, lse, dout, dq, dk, dv, desc, index,
                          index_bytes, ws, ws_bytes, stream), "attn_bwd")


def bwd_preprocess(prob, q, k, v, o, o_lo, dout, ws, ws_bytes, stream=0):
    _check(lib().attn_bwd_preprocess(ctypes.byref(prob), q, k, v, o, o_lo, dout, ws, ws_bytes, stream),
           "attn_bwd_preprocess")


def bwd_main(prob, q, k, v, lse, dout, dq, dk, dv, desc, index, index_bytes, ws, ws_bytes, stream=0):
    _check(lib().attn_bwd_main(ctypes.byref(prob), q, k, v, lse, dout, dq, dk, dv, desc, index, index_bytes,
                               ws, ws_bytes, stream), "attn_bwd_main")


def bwd_dkdv(prob, q, k, v, lse, dout, dk, dv, desc, index, index_bytes, ws, ws_bytes, stream=0):
    _check(lib().attn_bwd_dkdv(ctypes.byref(prob), q, k, v, lse, dout, dk, dv, desc, index, index_bytes,
                               ws, ws_bytes, stream), "attn_bwd_dkdv")


def bwd_dq(prob, q, k, v, lse, dout, dq, desc, index, index_bytes, ws, ws_bytes, stream=0):
    _check(lib().attn_bwd_dq(ctypes.byref(prob), q, k, v, lse, dout, dq, desc, index, index_bytes,
                             ws, ws_bytes, stream), "attn_bwd_dq")


def cast_bf16(src: int, dst: int, n: int, stream: int = 0):
    _check(lib().attn_cast_bf16(src, dst, n, stream), "attn_cast_bf16")


def mask_desc_build_device(spec: MaskSpec, T: int, cu_seqlens_dev: int, desc_dev: int, stream: int = 0):
    """attn_mask_desc_build_device: the descriptor of spec written to the device buffer
    desc_dev (int32 [T][4]); cu_seqlens_dev: device copy of spec.cu_seqlens (0 if unused)."""
    p, keep = mask_params(spec)
    _check(lib().attn_mask_desc_build_device(ctypes.byref(p), int(T), cu_seqlens_dev or None, desc_dev, stream),
           "attn_mask_desc_build_device")


def mask_desc_build_chunk(spec: MaskSpec, T: int, q_offset: int, k_offset: int, n: int) -> np.ndarray:
    """Host descriptor int32 [n][4] of the n x n chunk pair at (q_offset, k_offset)."""
    p, keep = mask_params(spec)
    out = np.empty((n, 4), dtype=np.int32)
    _check(lib().attn_mask_desc_build_chunk(ctypes.byref(p), int(T), int(q_offset), int(k_offset), int(n),
                                            out.ctypes.data), "attn_mask_desc_build_chunk")
    return out


def lse_merge(prob, o, o_lo, lse, o_part, o_part_lo, lse_part, stream=0):
    _check(lib().attn_lse_merge(ctypes.byref(prob), o, o_lo, lse, o_part, o_part_lo, lse_part, stream),
           "attn_lse_merge")


def block_select_params(mode: str, topk: int = 0, topp: float = 0.0, keep_diagonal: bool = True):
    m = {"topk": ATTN_SELECT_TOPK, "topp": ATTN_SELECT_TOPP}[mode]
    return attn_block_select_params(m, int(topk), float(topp), 1 if keep_diagonal else 0)


def block_select_workspace_size(prob) -> int:
    n = _SZ(0)
    _check(lib().attn_block_select_workspace_size(ctypes.byref(prob), ctypes.byref(n)),
           "attn_block_select_workspace_size")
    return n.value


def block_select(prob, params, q, k, scores, keep, ws, ws_bytes, stream=0):
    _check(lib().attn_block_select(ctypes.byref(prob), ctypes.byref(params), q, k, scores, keep, ws, ws_bytes,
                                   stream), "attn_block_select")


def block_select_noalloc(prob, params, q, k, scores, keep, stream=0):
    """attn_block_select with the library's static per-GPU workspace (no allocation)."""
    _check(lib().attn_block_select_noalloc(ctypes.byref(prob), ctypes.byref(params), q, k, scores, keep, stream),
           "attn_block_select_noalloc")


def variable_block_expand(T: int, Hq: int, row_offsets, col_offsets, keep_var: np.ndarray) -> np.ndarray:
    """Host uint8 [Hq][nt][nt] (nt = ceil(T / 64)): the uniform 64-block keep matrix of a
    variable-block mask whose edges are multiples of 64."""
    ro = np.ascontiguousarray(row_offsets, dtype=np.int32)
    co = np.ascontiguousarray(col_offsets, dtype=np.int32)
    kv = np.ascontiguousarray(keep_var, dtype=np.uint8)
    if kv.shape != (Hq, len(ro) - 1, len(co) - 1):
        raise ValueError(f"keep_var shape {kv.shape}, expected {(Hq, len(ro) - 1, len(co) - 1)}")
    nt = -(-T // 64)
    out = np.empty((Hq, nt, nt), dtype=np.uint8)
    _check(lib().attn_variable_block_expand(int(T), int(Hq), ro.ctypes.data, len(ro) - 1, co.ctypes.data,
                                            len(co) - 1, kv.ctypes.data, out.ctypes.data),
           "attn_variable_block_expand")
    return out


# --- PyTorch-allocated convenience object ----------------------------------------------

class MaskedAttention:
    """Buffers and index for one (T, Hq, Hk, mask) problem on a CUDA/HIP device.

    PyTorch provides the memory and the stream; every computation is a library call.
    q, k, v, do are bf16 tensors [T][H][128]; outputs are allocated here. ``desc`` may give
    a ready host descriptor int32 [T][4] (e.g. of a chunk pair, from mask_desc_build_chunk)
    instead of the one of ``spec`` over the whole length T. Block-sparse masks take
    ``keep`` (uint8 [Hq][nb][nb], numpy or a device tensor); a variable-block spec takes its
    keep matrix over the spec's grid (numpy) and runs as the 64-block mask it expands to.
    """

    def __init__(self, T: int, Hq: int, Hk: int, spec: MaskSpec, keep=None, device="cuda",
                 scale: float = 0.0, desc=None):
        import torch
        self.torch = torch
        if spec.kind == VARIABLE_BLOCK:
            # runs as the uniform 64-block mask its grid expands to (host expansion)
            if keep is None or isinstance(keep, torch.Tensor):
                raise ValueError("variable_block needs its keep matrix as a host numpy array")
            keep = variable_block_expand(T, Hq, spec.row_offsets, spec.col_offsets, keep)
            spec = MaskSpec("block_sparse", sparse_block=64)
        self.T, self.Hq, self.Hk, self.spec = T, Hq, Hk, spec
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        sparse = spec.kind == "block_sparse"
        self.prob = problem(T, Hq, Hk, spec.kind, spec.sparse_block if sparse else 0, scale)
        self.index_bytes = tile_index_size(self.prob)
        self.index = torch.empty(self.index_bytes, dtype=torch.uint8, device=self.device)
        self.layout = tile_index_layout(self.prob)
        if sparse:
            if keep is None:
                raise ValueError("block_sparse needs a keep matrix")
            keep_t = keep if isinstance(keep, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(keep))
            self.keep = keep_t.to(self.device, torch.uint8).contiguous()
            self.desc = None
            block_index_build(self.prob, self.keep.data_ptr(), self.index.data_ptr(), self.index_bytes,
                              self._stream())
        else:
            d = mask_desc_build(spec, T) if desc is None else np.ascontiguousarray(desc, dtype=np.int32)
            if d.shape != (T, 4):
                raise ValueError(f"descriptor shape {d.shape}, expected ({T}, 4)")
            self.desc = torch.from_numpy(d).to(self.device)
            tile_index_build(self.prob, self.desc.data_ptr(), self.index.data_ptr(), self.index_bytes,
                             self._stream())
        self.bwd_ws_bytes = bwd_workspace_size(self.prob)
        self.bwd_ws = torch.empty(max(1, self.bwd_ws_bytes), dtype=torch.uint8, device=self.device)

    def _stream(self) -> int:
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def _desc_ptr(self) -> int:
        return 0 if self.desc is None else self.desc.data_ptr()

    def forward(self, q, k, v, o=None, lse=None, o_lo=None, with_o_lo=True):
        """Returns (o, lse, o_lo); o_lo (the fp32 residual of O, for an accurate backward)
        is None when with_o_lo is False."""
        torch = self.torch
        for t in (q, k, v):
            if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device != self.device:
                raise ValueError("q, k, v must be contiguous bf16 tensors on the problem's device")
        if o is None:
            o = torch.empty((self.T, self.Hq, 128), dtype=torch.bfloat16, device=self.device)
        if lse is None:
            lse = torch.empty((self.Hq, self.T), dtype=torch.float32, device=self.device)
        if o_lo is None and with_o_lo:
            o_lo = torch.empty((self.T, self.Hq, 128), dtype=torch.bfloat16, device=self.device)
        fwd(self.prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
            0 if o_lo is None else o_lo.data_ptr(), lse.data_ptr(),
            self._desc_ptr(), self.index.data_ptr(), self.index_bytes, 0, 0, self._stream())
        return o, lse, o_lo

    def backward(self, q, k, v, o, lse, do, o_lo=None, dq=None, dk=None, dv=None):
        torch = self.torch
        if dq is None:
            dq = torch.empty((self.T, self.Hq, 128), dtype=torch.float32, device=self.device)
        if dk is None:
            dk = torch.empty((self.T, self.Hk, 128), dtype=torch.float32, device=self.device)
        if dv is None:
            dv = torch.empty((self.T, self.Hk, 128), dtype=torch.float32, device=self.device)
        bwd(self.prob, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
            0 if o_lo is None else o_lo.data_ptr(), lse.data_ptr(), do.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), self._desc_ptr(), self.index.data_ptr(),
            self.index_bytes, self.bwd_ws.data_ptr(), self.bwd_ws_bytes, self._stream())
        return dq, dk, dv

    def index_sections(self):
        """Host copies of the index sections (class maps, lists, orders) for inspection."""
        torch = self.torch
        raw = self.index.cpu().numpy()
        L = self.layout
        out = {}
        if self.spec.kind != "block_sparse":
            nf = L["nqt_f"] * L["nkt_f"]
            nb = L["nqt_b"] * L["nkt_b"]
            out["fwd_cls"] = raw[L["fwd_cls"]:L["fwd_cls"] + nf].reshape(L["nqt_f"], L["nkt_f"])
            out["bwd_cls"] = raw[L["bwd_cls"]:L["bwd_cls"] + nb].reshape(L["nqt_b"], L["nkt_b"])
            out["fwd_order"] = raw[L["fwd_order"]:L["fwd_order"] + 4 * L["nqt_f"]].view(np.int32)
            out["bwd_order"] = raw[L["bwd_order"]:L["bwd_order"] + 4 * L["nkt_b"]].view(np.int32)
            nrow_f, nrow_b = L["nqt_f"], L["nkt_b"]
        else:
            nrow_f, nrow_b = L["nqt_f"], L["nqt_b"]
        fptr = raw[L["fwd_ptr"]:L["fwd_ptr"] + 4 * (nrow_f + 1)].view(np.int32)
        bptr = raw[L["bwd_ptr"]:L["bwd_ptr"] + 4 * (nrow_b + 1)].view(np.int32)
        out["fwd_ptr"], out["bwd_ptr"] = fptr, bptr
        out["fwd_ent"] = raw[L["fwd_ent"]:L["fwd_ent"] + 4 * int(fptr[-1])].view(np.int32)
        out["bwd_ent"] = raw[L["bwd_ent"]:L["bwd_ent"] + 4 * int(bptr[-1])].view(np.int32)
        return out
