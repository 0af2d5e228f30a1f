"""Shared-prefix decode attention on MI355X: Python binding of the hp_attn C ABI.

This module only marshals arguments: it turns torch device tensors into the
plain pointers, sizes and structs that ``include/hp_attn.h`` declares and
calls the HIP library ``libhp_attn.so`` built from ``csrc/``.  Every step of
the computation runs in that library's gfx950 kernels; there is no fallback.
If the library has not been built, every call raises.

Entry points (same names as the C ABI):
  prefix_attn    one prefix node attended by the stacked queries of its sequences
  suffix_decode  per-sequence paged decode over private suffixes
  lse_merge      exact n-way merge of (O, LSE) partials
  cascade_step   a whole decode step over a prefix tree plus paged suffixes
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhp_attn.so")

HP_F32, HP_F16, HP_BF16 = 0, 1, 2
HP_MAX_LEVELS = 4
HP_MAX_NODES = 32
HP_MAX_MERGE = 16
HP_BLOCK_SIZE = 16
STATUS = {0: "HP_OK", 1: "HP_ERR_NULL", 2: "HP_ERR_INVALID_ARG", 3: "HP_ERR_UNSUPPORTED",
          4: "HP_ERR_WORKSPACE", 5: "HP_ERR_HIP"}
EXPORTS = ["hp_prefix_attn_workspace_size", "hp_prefix_attn", "hp_suffix_decode_workspace_size",
           "hp_suffix_decode", "hp_lse_merge", "hp_cascade_workspace_size", "hp_cascade_step",
           "hp_cascade_step_timed", "hp_status_string", "hp_last_hip_error", "hp_version"]

_DTYPE = {torch.float32: HP_F32, torch.float16: HP_F16, torch.bfloat16: HP_BF16}


class HpError(RuntimeError):
    def __init__(self, status: int, where: str, lib=None):
        msg = f"{where}: {STATUS.get(status, status)}"
        if lib is not None:
            msg += f" ({lib.hp_status_string(status).decode()})"
            if status == 5:
                msg += f" hipError={lib.hp_last_hip_error()}"
        super().__init__(msg)
        self.status = status


class Query(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("B", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class PrefixNode(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("stride_tok", ctypes.c_int64),
                ("stride_head", ctypes.c_int64), ("len", ctypes.c_int32),
                ("seq_begin", ctypes.c_int32), ("seq_end", ctypes.c_int32)]


class PrefixTree(ctypes.Structure):
    _fields_ = [("num_levels", ctypes.c_int32),
                ("nodes_per_level", ctypes.c_int32 * HP_MAX_LEVELS),
                ("nodes", ctypes.POINTER(PrefixNode))]


class PagedKV(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("max_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32)]


_lib = None
_lock = threading.Lock()


def lib():
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                                   "(hipcc --offload-arch=gfx950); there is no fallback path")
            L = ctypes.CDLL(LIB_PATH)
            st = ctypes.c_int
            p = ctypes.c_void_p
            L.hp_status_string.restype = ctypes.c_char_p
            L.hp_status_string.argtypes = [st]
            L.hp_last_hip_error.restype = ctypes.c_int32
            L.hp_version.restype = ctypes.c_char_p
            L.hp_prefix_attn_workspace_size.restype = st
            L.hp_prefix_attn_workspace_size.argtypes = [ctypes.POINTER(Query),
                                                        ctypes.POINTER(PrefixNode),
                                                        ctypes.POINTER(ctypes.c_size_t)]
            L.hp_prefix_attn.restype = st
            L.hp_prefix_attn.argtypes = [ctypes.POINTER(Query), ctypes.POINTER(PrefixNode), p, p,
                                         p, ctypes.c_size_t, p]
            L.hp_suffix_decode_workspace_size.restype = st
            L.hp_suffix_decode_workspace_size.argtypes = [ctypes.POINTER(Query),
                                                          ctypes.POINTER(PagedKV),
                                                          ctypes.POINTER(ctypes.c_size_t)]
            L.hp_suffix_decode.restype = st
            L.hp_suffix_decode.argtypes = [ctypes.POINTER(Query), ctypes.POINTER(PagedKV), p, p,
                                           p, ctypes.c_size_t, p]
            L.hp_lse_merge.restype = st
            L.hp_lse_merge.argtypes = [ctypes.c_int32, p, p, p, p, ctypes.c_int64,
                                       ctypes.c_int32, p]
            L.hp_cascade_workspace_size.restype = st
            L.hp_cascade_workspace_size.argtypes = [ctypes.POINTER(Query),
                                                    ctypes.POINTER(PrefixTree),
                                                    ctypes.POINTER(PagedKV),
                                                    ctypes.POINTER(ctypes.c_size_t)]
            L.hp_cascade_step.restype = st
            L.hp_cascade_step.argtypes = [ctypes.POINTER(Query), ctypes.POINTER(PrefixTree),
                                          ctypes.POINTER(PagedKV), p, p, p, ctypes.c_size_t, p]
            L.hp_cascade_step_timed.restype = st
            L.hp_cascade_step_timed.argtypes = [ctypes.POINTER(Query), ctypes.POINTER(PrefixTree),
                                                ctypes.POINTER(PagedKV), p, p, p,
                                                ctypes.c_size_t, p, p, ctypes.c_int32]
            _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise HpError(status, where, lib())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _require_cuda(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) device tensor")


def make_query(q: torch.Tensor, Hkv: int, scale: Optional[float] = None) -> Query:
    _require_cuda(q, "q")
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B][Hq][d] tensor")
    if q.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    return Query(q.data_ptr(), B, Hq, Hkv, d, _DTYPE[q.dtype], scale)


def make_node(k: torch.Tensor, v: torch.Tensor, seq_begin: int, seq_end: int) -> PrefixNode:
    """k, v: device [len][Hkv][d] (last dim contiguous, equal strides)."""
    _require_cuda(k, "k")
    _require_cuda(v, "v")
    if k.dim() != 3 or k.shape != v.shape or k.stride() != v.stride() or k.stride(2) != 1:
        raise ValueError("prefix k and v must be [len][Hkv][d] with equal strides, d contiguous")
    return PrefixNode(k.data_ptr(), v.data_ptr(), k.stride(0), k.stride(1), k.shape[0],
                      seq_begin, seq_end)


def make_tree(levels: Sequence[Sequence[Tuple[torch.Tensor, torch.Tensor, int, int]]]):
    """levels: root first; each a list of (k, v, seq_begin, seq_end).  Returns (tree, keepalive)."""
    if len(levels) > HP_MAX_LEVELS:
        raise ValueError(f"at most {HP_MAX_LEVELS} levels")
    flat = [make_node(k, v, b0, b1) for level in levels for (k, v, b0, b1) in level]
    arr = (PrefixNode * max(1, len(flat)))(*flat)
    counts = (ctypes.c_int32 * HP_MAX_LEVELS)(*([len(l) for l in levels] +
                                                [0] * (HP_MAX_LEVELS - len(levels))))
    tree = PrefixTree(len(levels), counts, ctypes.cast(arr, ctypes.POINTER(PrefixNode)))
    return tree, arr


def make_paged(k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
               seq_lens: torch.Tensor) -> PagedKV:
    for t, nm in ((k_pool, "k_pool"), (v_pool, "v_pool"), (block_table, "block_table"),
                  (seq_lens, "seq_lens")):
        _require_cuda(t, nm)
    if k_pool.dim() != 4 or k_pool.shape != v_pool.shape or not k_pool.is_contiguous() \
            or not v_pool.is_contiguous():
        raise ValueError("pools must be contiguous [num_blocks][block_size][Hkv][d]")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or \
            not block_table.is_contiguous() or block_table.dim() != 2:
        raise ValueError("block_table [B][max_blocks] and seq_lens [B] must be int32")
    return PagedKV(k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(),
                   seq_lens.data_ptr(), block_table.shape[1], k_pool.shape[1], k_pool.shape[0])


def _out(q: torch.Tensor, out, lse, zero: bool):
    B, Hq, d = q.shape
    if out is None:
        out = (torch.zeros if zero else torch.empty)(B, Hq, d, dtype=torch.float32,
                                                     device=q.device)
    if lse is None:
        lse = (torch.zeros if zero else torch.empty)(B, Hq, dtype=torch.float32, device=q.device)
    return out, lse


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def prefix_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_begin: int = 0,
                seq_end: Optional[int] = None, scale: Optional[float] = None, out=None, lse=None,
                stream=None):
    """Rows b in [seq_begin, seq_end) attend k/v ([len][Hkv][d]); returns (out, lse)."""
    L = lib()
    Hkv = k.shape[1]
    qs = make_query(q, Hkv, scale)
    node = make_node(k, v, seq_begin, q.shape[0] if seq_end is None else seq_end)
    out, lse = _out(q, out, lse, zero=True)
    nbytes = ctypes.c_size_t(0)
    _check(L.hp_prefix_attn_workspace_size(ctypes.byref(qs), ctypes.byref(node),
                                           ctypes.byref(nbytes)), "hp_prefix_attn_workspace_size")
    ws = _workspace(nbytes.value, q.device)
    _check(L.hp_prefix_attn(ctypes.byref(qs), ctypes.byref(node), out.data_ptr(), _ptr(lse),
                            _ptr(ws), nbytes.value, _stream(stream)), "hp_prefix_attn")
    return out, lse


def suffix_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                  block_table: torch.Tensor, seq_lens: torch.Tensor,
                  scale: Optional[float] = None, out=None, lse=None, stream=None):
    L = lib()
    qs = make_query(q, k_pool.shape[2], scale)
    kv = make_paged(k_pool, v_pool, block_table, seq_lens)
    out, lse = _out(q, out, lse, zero=False)
    nbytes = ctypes.c_size_t(0)
    _check(L.hp_suffix_decode_workspace_size(ctypes.byref(qs), ctypes.byref(kv),
                                             ctypes.byref(nbytes)),
           "hp_suffix_decode_workspace_size")
    ws = _workspace(nbytes.value, q.device)
    _check(L.hp_suffix_decode(ctypes.byref(qs), ctypes.byref(kv), out.data_ptr(), _ptr(lse),
                              _ptr(ws), nbytes.value, _stream(stream)), "hp_suffix_decode")
    return out, lse


def lse_merge(o_list: Sequence[torch.Tensor], lse_list: Sequence[torch.Tensor], out=None,
              lse=None, stream=None):
    """Merge n fp32 partials ([rows][d] / [rows], or [B][Hq][d] / [B][Hq])."""
    L = lib()
    n = len(o_list)
    if n != len(lse_list) or n == 0:
        raise ValueError("need matching non-empty o_list and lse_list")
    o0 = o_list[0]
    d = o0.shape[-1]
    rows = o0.numel() // d
    for o, l in zip(o_list, lse_list):
        _require_cuda(o, "o_in")
        _require_cuda(l, "lse_in")
        if o.dtype != torch.float32 or l.dtype != torch.float32 or not o.is_contiguous() or \
                not l.is_contiguous() or o.numel() != rows * d or l.numel() != rows:
            raise ValueError("partials must be contiguous fp32 with matching shapes")
    if out is None:
        out = torch.empty_like(o0)
    if lse is None:
        lse = torch.empty_like(lse_list[0])
    po = (ctypes.c_void_p * n)(*[o.data_ptr() for o in o_list])
    pl = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lse_list])
    _check(L.hp_lse_merge(n, ctypes.addressof(po), ctypes.addressof(pl), out.data_ptr(),
                          _ptr(lse), rows, d, _stream(stream)), "hp_lse_merge")
    return out, lse


class CascadeCall:
    """A prepared hp_cascade_step: structs, workspace and outputs built once, so a
    step costs one ctypes call (used for timing and graph capture)."""

    def __init__(self, q: torch.Tensor, levels, k_pool=None, v_pool=None, block_table=None,
                 seq_lens=None, scale: Optional[float] = None, out=None, lse=None):
        L = lib()
        self._L = L
        Hkv = (levels[0][0][0].shape[1] if levels and levels[0] else k_pool.shape[2])
        self.q = q
        self.query = make_query(q, Hkv, scale)
        self.tree, self._keep = make_tree(levels) if levels else (None, None)
        self.kv = make_paged(k_pool, v_pool, block_table, seq_lens) if k_pool is not None else None
        self.out, self.lse = _out(q, out, lse, zero=False)
        self._tree_p = ctypes.byref(self.tree) if self.tree is not None else None
        self._kv_p = ctypes.byref(self.kv) if self.kv is not None else None
        nbytes = ctypes.c_size_t(0)
        _check(L.hp_cascade_workspace_size(ctypes.byref(self.query), self._tree_p, self._kv_p,
                                           ctypes.byref(nbytes)), "hp_cascade_workspace_size")
        self.workspace_bytes = nbytes.value
        self.ws = _workspace(nbytes.value, q.device)
        self._refs = (levels, k_pool, v_pool, block_table, seq_lens)

    def __call__(self, stream=None):
        _check(self._L.hp_cascade_step(ctypes.byref(self.query), self._tree_p, self._kv_p,
                                       self.out.data_ptr(), _ptr(self.lse), _ptr(self.ws),
                                       self.workspace_bytes, _stream(stream)), "hp_cascade_step")
        return self.out, self.lse

    def timed(self, events, stream=None):
        """Run the step and record 4 caller-created hipEvent_t handles: before the
        prefix pass, after it, after the suffix pass and after the merge."""
        arr = (ctypes.c_void_p * 4)(*events)
        _check(self._L.hp_cascade_step_timed(ctypes.byref(self.query), self._tree_p, self._kv_p,
                                             self.out.data_ptr(), _ptr(self.lse), _ptr(self.ws),
                                             self.workspace_bytes, _stream(stream),
                                             ctypes.addressof(arr), 4), "hp_cascade_step_timed")
        return self.out, self.lse


def cascade_step(q: torch.Tensor, levels, k_pool=None, v_pool=None, block_table=None,
                 seq_lens=None, scale: Optional[float] = None, out=None, lse=None, stream=None):
    """levels: root first, each a list of (k, v, seq_begin, seq_end) device tensors/ints;
    the pools, table and lengths describe the paged suffixes (or None for prefix only)."""
    return CascadeCall(q, levels, k_pool, v_pool, block_table, seq_lens, scale, out, lse)(stream)
