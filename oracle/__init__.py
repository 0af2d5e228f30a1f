"""fp64 CPU oracle for shared-prefix decode attention (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the GPU library and never imports it; the one thing both sides share is the
seeded input generator in ``workloads`` (which holds no attention arithmetic).

Functions:
  attention(q, segs_per_seq, Hkv, scale, rows)  plain fp64 single-pass softmax
      attention of every (sequence, query head) row over the concatenation of
      that sequence's key segments.  Follows the definition of scaled
      dot-product attention and its log-sum-exp in "Hydragen: High-Throughput
      LLM Inference with Shared Prefixes", section "Attention Decomposition
      Across Subsequences" (the LSE definition and the SDP rewrite of its
      proof).
  merge(o_list, lse_list)  recombination of (O, LSE) partials by that page's
      Eq. 5, applied left to right.
  step_attention(step, part, rows)  the above over a generated ``workloads.Step``:
      "all" = every prefix node of the sequence then its suffix, "prefix" = its
      prefix nodes only, "suffix" = its suffix only, or ("level", i).
  tree_attention(step, rows)  the same definition over a ``workloads.ChunkTreeStep``:
      sequence b attends the pool rows of every descriptor holding it, cut at
      its length ("ChunkAttention: Efficient Self-Attention with Prefix-Aware
      KV Cache and Two-Phase Partition", section "Context Generation and
      GPU-CPU Coordination": a chunk descriptor (C, i, j) gives chunk C's keys
      to sequences i .. j-1).
  visible_positions(slot_sid, q_sid) / stream_attention(step, rows)  the
      stream-id mask of "Read Once, Answer Many: Parallel Prompting for
      Shared-Context LLM Inference" (section "Parallel Prompting", Eq. 2): a
      query of stream s attends the document and the positions of its
      request's KV row tagged -1 or s; the masked softmax is the plain softmax
      over those positions (a masked score contributes e^-inf = 0).
  kv_append(pool, rows, new)  the decode-step append of that page's section
      "Prefix-Aware KV Cache (PAKV): The Prefix Tree Structure": row i of
      ``new`` is stored at pool row rows[i] (entries outside the pool skipped).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


class _Segment(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("len", ctypes.c_int64),
                ("stride_tok", ctypes.c_int64), ("stride_head", ctypes.c_int64)]


class _Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("q", ctypes.c_void_p), ("seg_begin", ctypes.c_void_p),
                ("segs", ctypes.c_void_p), ("rows", ctypes.c_void_p), ("nrows", ctypes.c_int64)]


def compile_source(src: str, out: str) -> str:
    """gcc -O2 (no fast-math) with OpenMP: ``src`` -> shared library ``out``."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall",
                    "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile oracle.c when its library is missing or older than the source."""
    stale = (not os.path.exists(_LIB_PATH) or
             os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))
    if force or stale:
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def load(lib_path: str):
    """Load a build of oracle.c (the default one, or another build for tests)."""
    lib = ctypes.CDLL(lib_path)
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_int32]
    lib.oracle_merge.restype = ctypes.c_int
    lib.oracle_merge.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p]
    return lib


def _get(lib=None):
    global _lib
    if lib is not None:
        return lib
    with _lock:
        if _lib is None:
            build()
            _lib = load(_LIB_PATH)
    return _lib


def _check_kv(t: torch.Tensor, Hkv: int, d: int, dtype: torch.dtype) -> None:
    if t.device.type != "cpu" or t.dtype != dtype or t.dim() != 3 or \
            t.shape[1] != Hkv or t.shape[2] != d or t.stride(2) != 1:
        raise ValueError(f"key/value segment must be CPU [len][{Hkv}][{d}] {dtype} with the "
                         f"last dim contiguous, got {tuple(t.shape)} {t.dtype} {t.stride()}")


def attention(q: torch.Tensor, segs_per_seq: Sequence[Sequence[Tuple[torch.Tensor, torch.Tensor]]],
              Hkv: int, scale: float, rows: Optional[Sequence[int]] = None,
              nthreads: int = 0, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 attention for rows r = b*Hq + h (all rows when ``rows`` is None).

    q: CPU [B][Hq][d]; segs_per_seq[b]: list of (k, v), each [len][Hkv][d] of q's
    dtype.  Returns (O [n][d] float64, LSE [n] float64)."""
    lib = _get(lib)
    q = q.contiguous()
    B, Hq, d = q.shape
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if len(segs_per_seq) != B:
        raise ValueError("need one segment list per sequence")
    keep = []            # keep tensors alive while C holds their pointers
    seg_arr = []
    seg_begin = np.zeros(B + 1, dtype=np.int64)
    for b, segs in enumerate(segs_per_seq):
        for (k, v) in segs:
            _check_kv(k, Hkv, d, q.dtype)
            _check_kv(v, Hkv, d, q.dtype)
            if k.shape[0] != v.shape[0]:
                raise ValueError("k and v lengths differ")
            if v.stride() != k.stride():
                v = v.contiguous()
                k = k.contiguous()
            keep += [k, v]
            seg_arr.append(_Segment(k.data_ptr(), v.data_ptr(), k.shape[0], k.stride(0),
                                    k.stride(1)))
        seg_begin[b + 1] = len(seg_arr)
    segs_c = (_Segment * max(1, len(seg_arr)))(*seg_arr)
    if rows is None:
        n = B * Hq
        rows_np = None
    else:
        rows_np = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = int(rows_np.shape[0])
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    prob = _Problem(B, Hq, Hkv, d, _DTYPE_CODE[q.dtype], ctypes.c_float(scale).value,
                    q.data_ptr(), seg_begin.ctypes.data, ctypes.addressof(segs_c),
                    rows_np.ctypes.data if rows_np is not None else None, n)
    rc = lib.oracle_attention(ctypes.byref(prob), o.ctypes.data, lse.ctypes.data, nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_attention failed with code {rc}")
    return o, lse


def merge(o_list: Sequence[np.ndarray], lse_list: Sequence[np.ndarray], lib=None
          ) -> Tuple[np.ndarray, np.ndarray]:
    """Merge n partials ([rows][d] and [rows], fp32 or fp64, widened exactly) in fp64."""
    lib = _get(lib)
    n = len(o_list)
    if n != len(lse_list):
        raise ValueError("o_list and lse_list differ in length")
    os_ = [np.ascontiguousarray(np.asarray(o, dtype=np.float64)) for o in o_list]
    ls_ = [np.ascontiguousarray(np.asarray(l, dtype=np.float64)) for l in lse_list]
    if n == 0:
        raise ValueError("need at least one partial")
    rows, d = os_[0].shape
    for o, l in zip(os_, ls_):
        if o.shape != (rows, d) or l.shape != (rows,):
            raise ValueError("partials differ in shape")
    po = (ctypes.c_void_p * n)(*[o.ctypes.data for o in os_])
    pl = (ctypes.c_void_p * n)(*[l.ctypes.data for l in ls_])
    out = np.zeros((rows, d), dtype=np.float64)
    lse = np.zeros(rows, dtype=np.float64)
    rc = lib.oracle_merge(n, rows, d, ctypes.addressof(po), ctypes.addressof(pl),
                          out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_merge failed with code {rc}")
    return out, lse


def step_segments(step, part="all") -> List[List[Tuple[torch.Tensor, torch.Tensor]]]:
    """Key segments of every sequence of a ``workloads.Step``, from its logical arrays
    (never through the block table)."""
    out = []
    for b in range(step.cfg.B):
        segs = []
        if part in ("all", "prefix") or (isinstance(part, tuple) and part[0] == "level"):
            for li, level in enumerate(step.levels):
                if isinstance(part, tuple) and li != part[1]:
                    continue
                for node in level:
                    if node.seq_begin <= b < node.seq_end:
                        segs.append((node.k, node.v))
        if part in ("all", "suffix"):
            k, v = step.suffix(b)
            segs.append((k, v))
        out.append(segs)
    return out


def step_attention(step, part="all", rows: Optional[Sequence[int]] = None,
                   nthreads: int = 0, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    return attention(step.q, step_segments(step, part), step.cfg.Hkv, step.scale, rows,
                     nthreads, lib)


def tree_attention(step, rows: Optional[Sequence[int]] = None, nthreads: int = 0,
                   lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 attention of a ``workloads.ChunkTreeStep`` (every row, or ``rows``)."""
    need = set(range(step.B)) if rows is None else {int(r) // step.Hq for r in rows}
    segs = [step.keys_of(b) if b in need else [] for b in range(step.B)]
    return attention(step.q, segs, step.Hkv, step.scale, rows, nthreads, lib)


def visible_positions(slot_sid: Sequence[int], q_sid: int) -> np.ndarray:
    """Row positions a query of stream ``q_sid`` may attend: those whose stream id is
    -1 (every stream) or ``q_sid`` ("Read Once, Answer Many: Parallel Prompting for
    Shared-Context LLM Inference", section "Parallel Prompting", Eq. 2; the causal
    term holds for every position of a decode step's row, which ends at the new
    tokens).  In row order."""
    sid = np.asarray(slot_sid, dtype=np.int64)
    return np.nonzero((sid == -1) | (sid == int(q_sid)))[0]


def stream_segments(step, rows: Optional[Sequence[int]] = None
                    ) -> List[List[Tuple[torch.Tensor, torch.Tensor]]]:
    """Key segments of every query of a ``workloads.StreamStep``: its document nodes
    (root first), then the visible positions of its request's row, read from the
    logical row arrays (never through the pool)."""
    cfg = step.cfg
    need = set(range(cfg.B)) if rows is None else {int(r) // cfg.Hq for r in rows}
    out = []
    for b in range(cfg.B):
        if b not in need:
            out.append([])
            continue
        segs = []
        for level in step.levels:
            for node in level:
                if node.seq_begin <= b < node.seq_end:
                    segs.append((node.k, node.v))
        r = int(step.q_req[b])
        n = int(step.row_len[r])
        vis = torch.as_tensor(visible_positions(step.row_sid[r, :n].tolist(),
                                                int(step.q_sid[b])), dtype=torch.int64)
        segs.append((step.row_k[r][vis], step.row_v[r][vis]))
        out.append(segs)
    return out


def stream_attention(step, rows: Optional[Sequence[int]] = None, nthreads: int = 0,
                     lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 attention of a ``workloads.StreamStep`` (every row, or ``rows``)."""
    return attention(step.q, stream_segments(step, rows), step.cfg.Hkv, step.scale, rows,
                     nthreads, lib)


def kv_append(pool: torch.Tensor, rows: Sequence[int], new: torch.Tensor) -> torch.Tensor:
    """A copy of ``pool`` ([rows][...]) with new[i] stored at row rows[i]; rows
    outside [0, len(pool)) are skipped.  Plain element copy, no arithmetic."""
    out = pool.clone()
    for i, r in enumerate(list(rows)):
        if 0 <= int(r) < out.shape[0]:
            out[int(r)] = new[i]
    return out
