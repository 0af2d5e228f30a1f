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
  tree_plan_build / TreeStep   a decode step over (C, i, j) chunk descriptors
                 whose plan lives in device memory (any depth, forests)
  stream_decode / StreamCall   shared-context requests: P streams per request
                 read their document once; a stream-id mask picks each
                 stream's own tokens from the request's KV row
  kv_append      scatter of new tokens' K/V rows into the pool
  Pakv           the host prefix-tree KV manager (insert, append, remove,
                 context) that produces those descriptors
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# HP_ATTN_LIB selects another build of the same library (the host-sanitizer build)
LIB_PATH = os.environ.get("HP_ATTN_LIB") or os.path.join(_HERE, "libhp_attn.so")

HP_F32, HP_F16, HP_BF16 = 0, 1, 2
HP_MAX_LEVELS = 4
HP_MAX_NODES = 32
HP_MAX_MERGE = 16
HP_BLOCK_SIZE = 16
HP_CHUNK = 64
HP_TREE_MAX_LAUNCHES = 4
HP_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024
HP_READ_PROBE_WGS = 512
STATUS = {0: "HP_OK", 1: "HP_ERR_NULL", 2: "HP_ERR_INVALID_ARG", 3: "HP_ERR_UNSUPPORTED",
          4: "HP_ERR_WORKSPACE", 5: "HP_ERR_HIP", 6: "HP_ERR_CAPACITY", 7: "HP_ERR_HOST"}
EXPORTS = ["hp_prefix_attn_workspace_size", "hp_prefix_attn", "hp_suffix_decode_workspace_size",
           "hp_suffix_decode", "hp_lse_merge", "hp_cascade_workspace_size", "hp_cascade_step",
           "hp_cascade_step_timed", "hp_stream_decode_workspace_size", "hp_stream_decode",
           "hp_stream_decode_overlap", "hp_stream_overlap_plan",
           "hp_tree_plan_build", "hp_share_decision", "hp_tree_step", "hp_kv_append",
           "hp_pakv_create", "hp_pakv_destroy", "hp_pakv_insert", "hp_pakv_append",
           "hp_pakv_remove", "hp_pakv_context", "hp_pakv_seq_rows", "hp_pakv_get_stats",
           "hp_cascade_step_overlap", "hp_cascade_overlap_plan", "hp_cascade_step_noalloc",
           "hp_read_probe", "hp_status_string", "hp_last_hip_error", "hp_version"]

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
                ("nodes", ctypes.POINTER(PrefixNode)),
                ("share_min", ctypes.c_int32)]


HP_KV_NHD, HP_KV_HND = 0, 1


class PagedKV(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("max_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("layout", ctypes.c_int32)]


class StreamRows(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("row_slots", ctypes.c_void_p), ("slot_sid", ctypes.c_void_p),
                ("row_len", ctypes.c_void_p), ("q_req", ctypes.c_void_p),
                ("q_sid", ctypes.c_void_p), ("num_requests", ctypes.c_int32),
                ("row_cap", ctypes.c_int32), ("pool_rows", ctypes.c_int64)]


class Overlap(ctypes.Structure):
    _fields_ = [("side_stream", ctypes.c_void_p), ("fork_event", ctypes.c_void_p),
                ("join_event", ctypes.c_void_p), ("mode", ctypes.c_int32)]


class ChunkDesc(ctypes.Structure):
    _fields_ = [("row", ctypes.c_int32), ("count", ctypes.c_int32),
                ("seq_begin", ctypes.c_int32), ("seq_end", ctypes.c_int32)]


class TreePlan(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("share_min", ctypes.c_int32),
                ("num_descs", ctypes.c_int32), ("num_segs", ctypes.c_int32),
                ("num_pieces", ctypes.c_int32), ("num_srcs", ctypes.c_int32),
                ("num_tok_rows", ctypes.c_int32), ("max_private", ctypes.c_int32),
                ("num_launches", ctypes.c_int32),
                ("launch_nw", ctypes.c_int32 * HP_TREE_MAX_LAUNCHES),
                ("launch_wgs", ctypes.c_int32 * HP_TREE_MAX_LAUNCHES),
                ("launch_wg0", ctypes.c_int32 * HP_TREE_MAX_LAUNCHES),
                ("part_rows", ctypes.c_int64), ("pool_rows", ctypes.c_int64),
                ("blob_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t)]


class PakvStats(ctypes.Structure):
    _fields_ = [("num_chunks", ctypes.c_int32), ("chunks_used", ctypes.c_int32),
                ("chunks_free", ctypes.c_int32), ("chunks_fresh", ctypes.c_int32),
                ("nodes", ctypes.c_int32), ("seqs", ctypes.c_int32),
                ("tokens_stored", ctypes.c_int64), ("tokens_logical", ctypes.c_int64)]


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
            L.hp_cascade_overlap_plan.restype = st
            L.hp_cascade_overlap_plan.argtypes = [ctypes.POINTER(Query), ctypes.POINTER(PrefixTree),
                                                  ctypes.POINTER(PagedKV), ctypes.c_int32,
                                                  ctypes.POINTER(ctypes.c_int32)]
            L.hp_cascade_step_overlap.restype = st
            L.hp_cascade_step_overlap.argtypes = [ctypes.POINTER(Query), ctypes.POINTER(PrefixTree),
                                                  ctypes.POINTER(PagedKV), p, p, p,
                                                  ctypes.c_size_t, p, ctypes.POINTER(Overlap)]
            L.hp_read_probe.restype = st
            L.hp_read_probe.argtypes = [p, ctypes.c_size_t, p, p]
            L.hp_cascade_step_noalloc.restype = st
            L.hp_cascade_step_noalloc.argtypes = [ctypes.POINTER(Query), ctypes.POINTER(PrefixTree),
                                                  ctypes.POINTER(PagedKV), p, p, p]
            L.hp_cascade_step.restype = st
            L.hp_cascade_step.argtypes = [ctypes.POINTER(Query), ctypes.POINTER(PrefixTree),
                                          ctypes.POINTER(PagedKV), p, p, p, ctypes.c_size_t, p]
            L.hp_cascade_step_timed.restype = st
            L.hp_cascade_step_timed.argtypes = [ctypes.POINTER(Query), ctypes.POINTER(PrefixTree),
                                                ctypes.POINTER(PagedKV), p, p, p,
                                                ctypes.c_size_t, p, ctypes.POINTER(Overlap), p,
                                                ctypes.c_int32]
            i32, i64 = ctypes.c_int32, ctypes.c_int64
            L.hp_stream_decode_workspace_size.restype = st
            L.hp_stream_decode_workspace_size.argtypes = [ctypes.POINTER(Query),
                                                          ctypes.POINTER(PrefixTree),
                                                          ctypes.POINTER(StreamRows),
                                                          ctypes.POINTER(ctypes.c_size_t)]
            L.hp_stream_decode.restype = st
            L.hp_stream_decode.argtypes = [ctypes.POINTER(Query), ctypes.POINTER(PrefixTree),
                                           ctypes.POINTER(StreamRows), p, p, p,
                                           ctypes.c_size_t, p]
            L.hp_stream_decode_overlap.restype = st
            L.hp_stream_decode_overlap.argtypes = [ctypes.POINTER(Query),
                                                   ctypes.POINTER(PrefixTree),
                                                   ctypes.POINTER(StreamRows), p, p, p,
                                                   ctypes.c_size_t, p, ctypes.POINTER(Overlap)]
            L.hp_stream_overlap_plan.restype = st
            L.hp_stream_overlap_plan.argtypes = [ctypes.POINTER(Query), ctypes.POINTER(PrefixTree),
                                                 ctypes.POINTER(StreamRows), i32,
                                                 ctypes.POINTER(ctypes.c_int32)]
            L.hp_tree_plan_build.restype = st
            L.hp_tree_plan_build.argtypes = [ctypes.POINTER(Query), p, i32, i32, i64, p,
                                             ctypes.c_size_t, ctypes.POINTER(TreePlan)]
            L.hp_share_decision.restype = st
            L.hp_share_decision.argtypes = [ctypes.POINTER(Query), i64, i32,
                                            ctypes.POINTER(ctypes.c_int32)]
            L.hp_tree_step.restype = st
            L.hp_tree_step.argtypes = [ctypes.POINTER(Query), ctypes.POINTER(TreePlan), p, p, p,
                                       p, p, p, p, ctypes.c_size_t, p]
            L.hp_kv_append.restype = st
            L.hp_kv_append.argtypes = [p, p, p, i32, i32, i32, i32, p, p, i64, p, p, i32, p]
            L.hp_pakv_create.restype = st
            L.hp_pakv_create.argtypes = [i32, ctypes.POINTER(p)]
            L.hp_pakv_destroy.restype = None
            L.hp_pakv_destroy.argtypes = [p]
            L.hp_pakv_insert.restype = st
            L.hp_pakv_insert.argtypes = [p, i64, p, i32, p, p]
            L.hp_pakv_append.restype = st
            L.hp_pakv_append.argtypes = [p, i64, i32, p, p]
            L.hp_pakv_remove.restype = st
            L.hp_pakv_remove.argtypes = [p, i64]
            L.hp_pakv_context.restype = st
            L.hp_pakv_context.argtypes = [p, p, p, i32, p, i32, p, p]
            L.hp_pakv_seq_rows.restype = st
            L.hp_pakv_seq_rows.argtypes = [p, i64, p, i32, p]
            L.hp_pakv_get_stats.restype = st
            L.hp_pakv_get_stats.argtypes = [p, ctypes.POINTER(PakvStats)]
            _lib = L
    return _lib


_hiprt = None


def _hip():
    """The HIP runtime (for the events a side-by-side step records); the binding owns
    every handle it creates."""
    global _hiprt
    if _hiprt is None:
        rt = ctypes.CDLL("libamdhip64.so")
        rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        rt.hipEventCreateWithFlags.restype = ctypes.c_int
        rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        rt.hipEventDestroy.restype = ctypes.c_int
        _hiprt = rt
    return _hiprt


# hipEventDisableTiming | hipEventDisableSystemFence: the fork and join only order two
# streams of one device, which needs no system-scope fence.
_SIDE_EVENT_FLAGS = 0x2 | 0x20000000


class SideStreams:
    """A second stream and the fork/join events for hp_cascade_step_overlap, owned here:
    a torch stream on ``device`` (default priority) and two hipEvent_t handles created
    with hipEventDisableTiming and hipEventDisableSystemFence (they only order two
    streams of one device), destroyed with this object."""

    def __init__(self, device, mode: int = 1):
        self.stream = torch.cuda.Stream(device=device)
        rt = _hip()
        self._events = []
        for _ in range(2):
            h = ctypes.c_void_p()
            with torch.cuda.device(device):
                if rt.hipEventCreateWithFlags(ctypes.byref(h), _SIDE_EVENT_FLAGS) != 0:
                    raise RuntimeError("hipEventCreateWithFlags failed")
            self._events.append(h.value)
        self.desc = Overlap(self.stream.cuda_stream, self._events[0], self._events[1], mode)

    def close(self):
        # destroying an event that is still pending is allowed: HIP releases it once
        # the work it marks has completed
        for h in self._events:
            _hip().hipEventDestroy(h)
        self._events = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


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


def _torch_stream(stream, device):
    """The torch stream object for ``stream`` (None: the current stream; an int: a raw
    hipStream_t handle, wrapped without taking ownership)."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream, device=device)
    return stream


def _on(stream, device):
    """Context in which temporaries are allocated from ``stream``'s pool of the caching
    allocator, so that freeing them after the call is ordered after the kernels that the
    call enqueued on that stream (not on whichever stream happens to be current)."""
    return torch.cuda.stream(_torch_stream(stream, device))


def _record(stream, tensors) -> None:
    """Mark long-lived buffers as in use by ``stream`` when it is not the stream they
    were allocated on, so the caching allocator does not reuse them early when freed."""
    if stream is None:
        return
    ts = None
    for t in tensors:
        if t is None:
            continue
        if ts is None:
            ts = _torch_stream(stream, t.device)
        t.record_stream(ts)


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


def make_tree(levels: Sequence[Sequence[Tuple[torch.Tensor, torch.Tensor, int, int]]],
              share_min: int = 0):
    """levels: root first; each a list of (k, v, seq_begin, seq_end).  share_min: which nodes
    a cascade step batches (0: the batching policy per node; k >= 1: nodes over at least k
    sequences; the others are read by each of their sequences in the suffix pass).
    Returns (tree, keepalive)."""
    if len(levels) > HP_MAX_LEVELS:
        raise ValueError(f"at most {HP_MAX_LEVELS} levels")
    flat = [make_node(k, v, b0, b1) for level in levels for (k, v, b0, b1) in level]
    arr = (PrefixNode * max(1, len(flat)))(*flat)
    counts = (ctypes.c_int32 * HP_MAX_LEVELS)(*([len(l) for l in levels] +
                                                [0] * (HP_MAX_LEVELS - len(levels))))
    tree = PrefixTree(len(levels), counts, ctypes.cast(arr, ctypes.POINTER(PrefixNode)),
                      int(share_min))
    return tree, arr


_KV_LAYOUTS = {"NHD": HP_KV_NHD, "HND": HP_KV_HND}


def pool_heads(k_pool: torch.Tensor, kv_layout: str = "NHD") -> int:
    """KV heads of a paged pool: [blocks][block_size][Hkv][d] (NHD) or
    [blocks][Hkv][block_size][d] (HND)."""
    return int(k_pool.shape[2] if kv_layout == "NHD" else k_pool.shape[1])


def make_paged(k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
               seq_lens: torch.Tensor, kv_layout: str = "NHD") -> PagedKV:
    """kv_layout "NHD": pools [num_blocks][block_size][Hkv][d]; "HND": [num_blocks][Hkv]
    [block_size][d] (each block's rows of one KV head contiguous)."""
    for t, nm in ((k_pool, "k_pool"), (v_pool, "v_pool"), (block_table, "block_table"),
                  (seq_lens, "seq_lens")):
        _require_cuda(t, nm)
    if kv_layout not in _KV_LAYOUTS:
        raise ValueError(f"kv_layout must be one of {sorted(_KV_LAYOUTS)}")
    if k_pool.dim() != 4 or k_pool.shape != v_pool.shape or not k_pool.is_contiguous() \
            or not v_pool.is_contiguous():
        raise ValueError("pools must be contiguous 4-d tensors of one shape")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or \
            not block_table.is_contiguous() or block_table.dim() != 2:
        raise ValueError("block_table [B][max_blocks] and seq_lens [B] must be int32")
    block_size = k_pool.shape[1] if kv_layout == "NHD" else k_pool.shape[2]
    return PagedKV(k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(),
                   seq_lens.data_ptr(), block_table.shape[1], block_size, k_pool.shape[0],
                   _KV_LAYOUTS[kv_layout])


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
    nbytes = ctypes.c_size_t(0)
    _check(L.hp_prefix_attn_workspace_size(ctypes.byref(qs), ctypes.byref(node),
                                           ctypes.byref(nbytes)), "hp_prefix_attn_workspace_size")
    with _on(stream, q.device):
        out, lse = _out(q, out, lse, zero=True)
        ws = _workspace(nbytes.value, q.device)
        _check(L.hp_prefix_attn(ctypes.byref(qs), ctypes.byref(node), out.data_ptr(), _ptr(lse),
                                _ptr(ws), nbytes.value, _stream(stream)), "hp_prefix_attn")
    return out, lse


def suffix_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                  block_table: torch.Tensor, seq_lens: torch.Tensor,
                  scale: Optional[float] = None, out=None, lse=None, stream=None,
                  kv_layout: str = "NHD"):
    L = lib()
    qs = make_query(q, pool_heads(k_pool, kv_layout), scale)
    kv = make_paged(k_pool, v_pool, block_table, seq_lens, kv_layout)
    nbytes = ctypes.c_size_t(0)
    _check(L.hp_suffix_decode_workspace_size(ctypes.byref(qs), ctypes.byref(kv),
                                             ctypes.byref(nbytes)),
           "hp_suffix_decode_workspace_size")
    with _on(stream, q.device):
        out, lse = _out(q, out, lse, zero=False)
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
    with _on(stream, o0.device):
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
    """A prepared cascade step: structs, workspace and outputs built once, so a step
    costs one ctypes call (used for timing and graph capture).

    overlap: 0 runs the passes one after the other on the caller's stream
    (hp_cascade_step); 1 (the default), 2 or 3 calls hp_cascade_step_overlap in that
    mode (1: side by side when the plan expects a gain, on a second stream or in one
    launch; 2: on a second stream whenever there is a prefix and a suffix; 3: in one
    launch whenever the step qualifies), with a second stream and two events owned by
    this object when the plan uses them.  ``concurrent`` says whether the passes run
    side by side, ``one_launch`` whether they share one launch.  share_min: which tree nodes the prefix pass batches (see
    make_tree; 0, the default, is the library's batching policy)."""

    def __init__(self, q: torch.Tensor, levels, k_pool=None, v_pool=None, block_table=None,
                 seq_lens=None, scale: Optional[float] = None, out=None, lse=None,
                 overlap: int = 1, share_min: int = 0, kv_layout: str = "NHD"):
        L = lib()
        self._L = L
        Hkv = (levels[0][0][0].shape[1] if levels and levels[0] else
               pool_heads(k_pool, kv_layout))
        self.q = q
        self.query = make_query(q, Hkv, scale)
        self.tree, self._keep = make_tree(levels, share_min) if levels else (None, None)
        self.kv = (make_paged(k_pool, v_pool, block_table, seq_lens, kv_layout)
                   if k_pool is not None else None)
        self.out, self.lse = _out(q, out, lse, zero=False)
        self._tree_p = ctypes.byref(self.tree) if self.tree is not None else None
        self._kv_p = ctypes.byref(self.kv) if self.kv is not None else None
        nbytes = ctypes.c_size_t(0)
        _check(L.hp_cascade_workspace_size(ctypes.byref(self.query), self._tree_p, self._kv_p,
                                           ctypes.byref(nbytes)), "hp_cascade_workspace_size")
        self.workspace_bytes = nbytes.value
        self.ws = _workspace(nbytes.value, q.device)
        flag = ctypes.c_int32(0)
        _check(L.hp_cascade_overlap_plan(ctypes.byref(self.query), self._tree_p, self._kv_p,
                                         int(overlap), ctypes.byref(flag)),
               "hp_cascade_overlap_plan")
        # the suffix pass beside the prefix pass: on a second stream (1) or in the
        # prefix pass's launch (2, no stream or event needed)
        self.concurrent = bool(flag.value)
        self.one_launch = flag.value == 2
        self.side = SideStreams(q.device, int(overlap)) if flag.value == 1 else None
        if self.side is not None:
            self._ov = self.side.desc
        elif self.one_launch:
            self._ov = Overlap(None, None, None, int(overlap))
        else:
            self._ov = None
        self._ov_p = ctypes.byref(self._ov) if self._ov is not None else None
        self._refs = (levels, k_pool, v_pool, block_table, seq_lens)

    def __call__(self, stream=None):
        _record(stream, (self.ws, self.out, self.lse))
        if self._ov_p is not None:
            st = self._L.hp_cascade_step_overlap(ctypes.byref(self.query), self._tree_p, self._kv_p,
                                                 self.out.data_ptr(), _ptr(self.lse),
                                                 _ptr(self.ws), self.workspace_bytes,
                                                 _stream(stream), self._ov_p)
            _check(st, "hp_cascade_step_overlap")
        else:
            _check(self._L.hp_cascade_step(ctypes.byref(self.query), self._tree_p, self._kv_p,
                                           self.out.data_ptr(), _ptr(self.lse), _ptr(self.ws),
                                           self.workspace_bytes, _stream(stream)),
                   "hp_cascade_step")
        return self.out, self.lse

    def timed(self, events, stream=None):
        """Run the step and record 4 or 5 caller-created hipEvent_t handles: before the
        prefix pass, after it, after the suffix pass, after the merge and (optional)
        right before the suffix pass on its stream."""
        n = len(events)
        arr = (ctypes.c_void_p * n)(*events)
        _record(stream, (self.ws, self.out, self.lse))
        _check(self._L.hp_cascade_step_timed(ctypes.byref(self.query), self._tree_p, self._kv_p,
                                             self.out.data_ptr(), _ptr(self.lse), _ptr(self.ws),
                                             self.workspace_bytes, _stream(stream), self._ov_p,
                                             ctypes.addressof(arr), n), "hp_cascade_step_timed")
        return self.out, self.lse


def cascade_step(q: torch.Tensor, levels, k_pool=None, v_pool=None, block_table=None,
                 seq_lens=None, scale: Optional[float] = None, out=None, lse=None, stream=None,
                 overlap: int = 1, share_min: int = 0, kv_layout: str = "NHD"):
    """levels: root first, each a list of (k, v, seq_begin, seq_end) device tensors/ints;
    the pools, table and lengths describe the paged suffixes (or None for prefix only).
    share_min: see make_tree; kv_layout: see make_paged."""
    with _on(stream, q.device):
        call = CascadeCall(q, levels, k_pool, v_pool, block_table, seq_lens, scale, out, lse,
                           overlap, share_min, kv_layout)
        return call(stream)


def cascade_step_noalloc(q: torch.Tensor, levels, k_pool=None, v_pool=None, block_table=None,
                         seq_lens=None, scale: Optional[float] = None, out=None, lse=None,
                         stream=None, share_min: int = 0, kv_layout: str = "NHD"):
    """hp_cascade_step_noalloc: cascade_step on one stream with the workspace taken from
    the library's fixed per-GPU scratch array (at most HP_NOALLOC_SCRATCH_BYTES).  The
    library allocates nothing; pass ``out`` (and ``lse``) to allocate nothing here either.
    Calls on one GPU share that array: the caller orders calls that could overlap."""
    L = lib()
    Hkv = (levels[0][0][0].shape[1] if levels and levels[0] else pool_heads(k_pool, kv_layout))
    query = make_query(q, Hkv, scale)
    tree, keep = make_tree(levels, share_min) if levels else (None, None)
    kv = (make_paged(k_pool, v_pool, block_table, seq_lens, kv_layout)
          if k_pool is not None else None)
    with _on(stream, q.device):
        out, lse = _out(q, out, lse, zero=False)
    _check(L.hp_cascade_step_noalloc(ctypes.byref(query),
                                     ctypes.byref(tree) if tree is not None else None,
                                     ctypes.byref(kv) if kv is not None else None,
                                     out.data_ptr(), _ptr(lse), _stream(stream)),
           "hp_cascade_step_noalloc")
    del keep
    return out, lse


def read_probe(buf: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None):
    """hp_read_probe: one streaming read of ``buf`` (contiguous device memory, a multiple
    of 16 bytes); returns ``sink`` (int32 [HP_READ_PROBE_WGS], the XOR partials).  For
    measuring the device's streaming-read rate."""
    L = lib()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    with _on(stream, buf.device):
        if sink is None:
            sink = torch.empty(HP_READ_PROBE_WGS, dtype=torch.int32, device=buf.device)
    if sink.dtype != torch.int32 or sink.numel() < HP_READ_PROBE_WGS or not sink.is_cuda:
        raise ValueError(f"sink must be a device int32 tensor of {HP_READ_PROBE_WGS} words")
    _check(L.hp_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), _stream(stream)),
           "hp_read_probe")
    return sink


# ------------------------------------------------------------------------------
# Chunked prefix tree: (C, i, j) descriptors, device-resident plans, append, PAKV
# ------------------------------------------------------------------------------

def make_stream_rows(k_pool: torch.Tensor, v_pool: torch.Tensor, row_slots: torch.Tensor,
                     slot_sid: torch.Tensor, row_len: torch.Tensor, q_req: torch.Tensor,
                     q_sid: torch.Tensor) -> StreamRows:
    """Pools [pool_rows][Hkv][d]; row_slots / slot_sid [R][row_cap], row_len [R],
    q_req / q_sid [B]: contiguous int32 device tensors."""
    for t, nm in ((k_pool, "k_pool"), (v_pool, "v_pool"), (row_slots, "row_slots"),
                  (slot_sid, "slot_sid"), (row_len, "row_len"), (q_req, "q_req"),
                  (q_sid, "q_sid")):
        _require_cuda(t, nm)
    if k_pool.dim() != 3 or k_pool.shape != v_pool.shape or not k_pool.is_contiguous() \
            or not v_pool.is_contiguous():
        raise ValueError("pools must be contiguous [pool_rows][Hkv][d]")
    for t, nm in ((row_slots, "row_slots"), (slot_sid, "slot_sid"), (row_len, "row_len"),
                  (q_req, "q_req"), (q_sid, "q_sid")):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous int32 tensor")
    if row_slots.dim() != 2 or row_slots.shape != slot_sid.shape or \
            row_len.shape != (row_slots.shape[0],) or q_req.shape != q_sid.shape:
        raise ValueError("row_slots/slot_sid [R][row_cap], row_len [R], q_req/q_sid [B]")
    return StreamRows(k_pool.data_ptr(), v_pool.data_ptr(), row_slots.data_ptr(),
                      slot_sid.data_ptr(), row_len.data_ptr(), q_req.data_ptr(),
                      q_sid.data_ptr(), row_slots.shape[0], row_slots.shape[1],
                      k_pool.shape[0])


class StreamCall:
    """A prepared hp_stream_decode: every stream query attends its document (the
    prefix tree ``doc_levels``, as in CascadeCall) and the positions of its
    request's KV row whose stream id is -1 or its own.

    overlap: 0 runs the passes one after the other on the caller's stream
    (hp_stream_decode); 1 (the default) or 2 calls hp_stream_decode_overlap in that
    mode, with a second stream and fork/join events owned by this object when the plan
    uses them.  ``concurrent`` says whether the stream pass runs beside the document's
    prefix pass."""

    def __init__(self, q: torch.Tensor, doc_levels, k_pool: torch.Tensor, v_pool: torch.Tensor,
                 row_slots: torch.Tensor, slot_sid: torch.Tensor, row_len: torch.Tensor,
                 q_req: torch.Tensor, q_sid: torch.Tensor, scale: Optional[float] = None,
                 out=None, lse=None, overlap: int = 1):
        L = lib()
        self._L = L
        if q_req.shape != (q.shape[0],):
            raise ValueError("q_req and q_sid need one entry per query")
        self.query = make_query(q, k_pool.shape[1], scale)
        self.tree, self._keep = make_tree(doc_levels) if doc_levels else (None, None)
        self.rows = make_stream_rows(k_pool, v_pool, row_slots, slot_sid, row_len, q_req, q_sid)
        self.out, self.lse = _out(q, out, lse, zero=False)
        self._tree_p = ctypes.byref(self.tree) if self.tree is not None else None
        nbytes = ctypes.c_size_t(0)
        _check(L.hp_stream_decode_workspace_size(ctypes.byref(self.query), self._tree_p,
                                                 ctypes.byref(self.rows), ctypes.byref(nbytes)),
               "hp_stream_decode_workspace_size")
        self.workspace_bytes = nbytes.value
        self.ws = _workspace(nbytes.value, q.device)
        self._refs = (q, doc_levels, k_pool, v_pool, row_slots, slot_sid, row_len, q_req, q_sid)
        flag = ctypes.c_int32(0)
        _check(L.hp_stream_overlap_plan(ctypes.byref(self.query), self._tree_p,
                                        ctypes.byref(self.rows), int(overlap),
                                        ctypes.byref(flag)), "hp_stream_overlap_plan")
        self.concurrent = bool(flag.value)
        self.side = SideStreams(q.device, int(overlap)) if self.concurrent else None
        self._ov_p = ctypes.byref(self.side.desc) if self.side is not None else None

    def __call__(self, stream=None):
        _record(stream, (self.ws, self.out, self.lse))
        if self._ov_p is not None:
            _check(self._L.hp_stream_decode_overlap(ctypes.byref(self.query), self._tree_p,
                                                    ctypes.byref(self.rows), self.out.data_ptr(),
                                                    _ptr(self.lse), _ptr(self.ws),
                                                    self.workspace_bytes, _stream(stream),
                                                    self._ov_p), "hp_stream_decode_overlap")
            return self.out, self.lse
        _check(self._L.hp_stream_decode(ctypes.byref(self.query), self._tree_p,
                                        ctypes.byref(self.rows), self.out.data_ptr(),
                                        _ptr(self.lse), _ptr(self.ws), self.workspace_bytes,
                                        _stream(stream)), "hp_stream_decode")
        return self.out, self.lse


def stream_decode(q: torch.Tensor, doc_levels, k_pool, v_pool, row_slots, slot_sid, row_len,
                  q_req, q_sid, scale: Optional[float] = None, out=None, lse=None, stream=None,
                  overlap: int = 1):
    with _on(stream, q.device):
        return StreamCall(q, doc_levels, k_pool, v_pool, row_slots, slot_sid, row_len, q_req,
                          q_sid, scale, out, lse, overlap)(stream)


def _descs_array(descs) -> Tuple[ctypes.Array, int]:
    """descs: an [n][4] int array-like of (row, count, seq_begin, seq_end)."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(descs, dtype=np.int32).reshape(-1, 4))
    n = a.shape[0]
    arr = (ChunkDesc * max(1, n))()
    if n:
        ctypes.memmove(arr, a.ctypes.data, a.nbytes)
    return arr, n


def tree_plan_build(B: int, Hq: int, Hkv: int, d: int, dtype: torch.dtype, descs,
                    share_min: int, pool_rows: int):
    """Plan a chunk-tree step.  Returns (TreePlan, blob) with blob a host uint8 tensor
    holding the plan's device image (copy it to the GPU; see TreeStep)."""
    L = lib()
    geom = Query(None, B, Hq, Hkv, d, _DTYPE[dtype], 1.0)
    arr, n = _descs_array(descs)
    plan = TreePlan()
    _check(L.hp_tree_plan_build(ctypes.byref(geom), ctypes.addressof(arr), n, share_min,
                                pool_rows, None, 0, ctypes.byref(plan)), "hp_tree_plan_build")
    blob = torch.zeros(max(16, plan.blob_bytes), dtype=torch.uint8)
    _check(L.hp_tree_plan_build(ctypes.byref(geom), ctypes.addressof(arr), n, share_min,
                                pool_rows, blob.data_ptr(), blob.numel(), ctypes.byref(plan)),
           "hp_tree_plan_build")
    return plan, blob


def share_decision(Hq: int, Hkv: int, tokens: int, nseq: int, d: int = 128,
                   dtype: torch.dtype = torch.bfloat16) -> bool:
    """True when `tokens` keys shared by `nseq` sequences are better read once for all of
    them (prefix pass plus merge) than by each sequence (hp_share_decision)."""
    L = lib()
    geom = Query(None, max(1, nseq), Hq, Hkv, d, _DTYPE[dtype], 1.0)
    out = ctypes.c_int32(0)
    _check(L.hp_share_decision(ctypes.byref(geom), tokens, nseq, ctypes.byref(out)),
           "hp_share_decision")
    return bool(out.value)


class TreeStep:
    """A planned chunk-tree step: the plan image copied to device memory once, its
    workspace allocated once; each call is one hp_tree_step."""

    def __init__(self, q_like: torch.Tensor, Hkv: int, descs, share_min: int, pool_rows: int,
                 scale: Optional[float] = None):
        _require_cuda(q_like, "q")
        B, Hq, d = q_like.shape
        self.plan, blob_host = tree_plan_build(B, Hq, Hkv, d, q_like.dtype, descs, share_min,
                                               pool_rows)
        self.blob = blob_host.to(q_like.device)  # the lazy context copy: once per tree shape
        self.Hkv = Hkv
        self.scale = scale
        self.ws = _workspace(self.plan.workspace_bytes, q_like.device)

    def __call__(self, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                 seq_lens: Optional[torch.Tensor] = None, out=None, lse=None, stream=None):
        L = lib()
        qs = make_query(q, self.Hkv, self.scale)
        for t, nm in ((k_pool, "k_pool"), (v_pool, "v_pool")):
            _require_cuda(t, nm)
            if t.dtype != q.dtype or not t.is_contiguous() or t.shape[-2:] != (self.Hkv, q.shape[2]):
                raise ValueError(f"{nm} must be a contiguous [rows][Hkv][d] tensor of q's dtype")
        if k_pool.shape[0] * (k_pool.numel() // max(1, k_pool.shape[0])) < \
                self.plan.pool_rows * self.Hkv * q.shape[2]:
            raise ValueError("pool has fewer rows than the plan was built for")
        if seq_lens is not None:
            _require_cuda(seq_lens, "seq_lens")
            if seq_lens.dtype != torch.int32 or seq_lens.numel() != q.shape[0]:
                raise ValueError("seq_lens must be int32 [B]")
        _record(stream, (self.ws, self.blob))
        with _on(stream, q.device):
            out, lse = _out(q, out, lse, zero=False)
        _check(L.hp_tree_step(ctypes.byref(qs), ctypes.byref(self.plan), self.blob.data_ptr(),
                              k_pool.data_ptr(), v_pool.data_ptr(), _ptr(seq_lens),
                              out.data_ptr(), _ptr(lse), _ptr(self.ws), self.plan.workspace_bytes,
                              _stream(stream)), "hp_tree_step")
        return out, lse


def kv_append(k_new: torch.Tensor, v_new: torch.Tensor, rows: torch.Tensor,
              k_pool: torch.Tensor, v_pool: torch.Tensor, seq_lens: Optional[torch.Tensor] = None,
              seq_idx: Optional[torch.Tensor] = None, stream=None) -> None:
    """Copy k_new[i], v_new[i] ([n][Hkv][d]) to pool row rows[i]; optionally
    seq_lens[seq_idx[i]] += 1 (all device tensors)."""
    L = lib()
    for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (rows, "rows"), (k_pool, "k_pool"),
                  (v_pool, "v_pool")):
        _require_cuda(t, nm)
    if k_new.shape != v_new.shape or k_new.dim() != 3 or not k_new.is_contiguous() or \
            not v_new.is_contiguous():
        raise ValueError("k_new, v_new must be contiguous [n][Hkv][d]")
    n, Hkv, d = k_new.shape
    if k_pool.dtype != k_new.dtype or v_pool.dtype != k_new.dtype or \
            not k_pool.is_contiguous() or not v_pool.is_contiguous() or \
            k_pool.shape != v_pool.shape or k_pool.numel() % (Hkv * d):
        raise ValueError("pools must be contiguous, of k_new's dtype, [rows][Hkv][d]")
    if rows.dtype != torch.int32 or rows.numel() != n:
        raise ValueError("rows must be int32 [n]")
    num_seqs = 0
    if seq_lens is not None:
        _require_cuda(seq_lens, "seq_lens")
        _require_cuda(seq_idx, "seq_idx")
        if seq_lens.dtype != torch.int32 or seq_idx.dtype != torch.int32 or seq_idx.numel() != n:
            raise ValueError("seq_lens and seq_idx must be int32, seq_idx [n]")
        num_seqs = seq_lens.numel()
    _check(L.hp_kv_append(k_new.data_ptr(), v_new.data_ptr(), rows.data_ptr(), n, Hkv, d,
                          _DTYPE[k_new.dtype], k_pool.data_ptr(), v_pool.data_ptr(),
                          k_pool.numel() // (Hkv * d), _ptr(seq_lens), _ptr(seq_idx), num_seqs,
                          _stream(stream)), "hp_kv_append")


class Pakv:
    """Host prefix-tree KV cache manager over a pool of num_chunks * 64 rows."""

    def __init__(self, num_chunks: int):
        self._L = lib()
        h = ctypes.c_void_p()
        _check(self._L.hp_pakv_create(num_chunks, ctypes.byref(h)), "hp_pakv_create")
        self._h = h
        self.num_chunks = num_chunks

    def close(self):
        if self._h:
            self._L.hp_pakv_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def insert(self, seq_id: int, tokens: Sequence[int]):
        """Returns (rows of every token, matched): tokens >= matched need K/V written."""
        import numpy as np
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        rows = np.zeros(max(1, t.shape[0]), dtype=np.int32)
        m = ctypes.c_int32(0)
        _check(self._L.hp_pakv_insert(self._h, seq_id, t.ctypes.data if t.size else None,
                                      t.shape[0], rows.ctypes.data, ctypes.byref(m)),
               "hp_pakv_insert")
        return rows[:t.shape[0]], m.value

    def append(self, seq_id: int, token: int):
        """Returns (row for the token's K/V, changed): changed = the tree's shape moved."""
        r, c = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(self._L.hp_pakv_append(self._h, seq_id, token, ctypes.byref(r), ctypes.byref(c)),
               "hp_pakv_append")
        return r.value, bool(c.value)

    def remove(self, seq_id: int) -> None:
        _check(self._L.hp_pakv_remove(self._h, seq_id), "hp_pakv_remove")

    def stats(self) -> PakvStats:
        st = PakvStats()
        _check(self._L.hp_pakv_get_stats(self._h, ctypes.byref(st)), "hp_pakv_get_stats")
        return st

    def context(self):
        """Returns (seq_order [B] int64, seq_lens [B] int32, descs [n][4] int32), numpy."""
        import numpy as np
        st = self.stats()
        order = np.zeros(max(1, st.seqs), dtype=np.int64)
        lens = np.zeros(max(1, st.seqs), dtype=np.int32)
        descs = np.zeros((max(1, st.nodes), 4), dtype=np.int32)
        ns, nd = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(self._L.hp_pakv_context(self._h, order.ctypes.data, lens.ctypes.data,
                                       order.shape[0], descs.ctypes.data, descs.shape[0],
                                       ctypes.byref(ns), ctypes.byref(nd)), "hp_pakv_context")
        return order[:ns.value], lens[:ns.value], descs[:nd.value]

    def seq_rows(self, seq_id: int):
        import numpy as np
        n = ctypes.c_int32(0)
        st = self._L.hp_pakv_seq_rows(self._h, seq_id, None, 0, ctypes.byref(n))
        if st not in (0, 6):
            _check(st, "hp_pakv_seq_rows")
        rows = np.zeros(max(1, n.value), dtype=np.int32)
        _check(self._L.hp_pakv_seq_rows(self._h, seq_id, rows.ctypes.data, rows.shape[0],
                                        ctypes.byref(n)), "hp_pakv_seq_rows")
        return rows[:n.value]
