"""The C ABI on the host: exports, status strings, workspace sizing and every validation
path (each returns before anything is enqueued, so no GPU is needed)."""
import ctypes
import os
import re

import pytest

import decode_attention_shared_amd as hp
import workloads
from decode_attention_shared_amd import (PagedKV, PrefixNode, PrefixTree, Query, HP_BF16, HP_F16,
                                         HP_F32)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hp_attn.h")

OK, NULL, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3, 4
FAKE = 0x10000          # an aligned non-null address; never dereferenced by validation
p = ctypes.c_void_p


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hp.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return hp.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hp_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 10
    assert set(names) == set(hp.EXPORTS)
    for n in names:
        assert hasattr(L, n), f"libhp_attn.so does not export {n}"


def test_status_strings_and_version(L):
    for code in range(8):
        assert L.hp_status_string(code)
    assert L.hp_status_string(99) == b"unknown status"
    assert b"gfx950" in L.hp_version()
    assert L.hp_last_hip_error() == 0


def q_(B=4, Hq=8, Hkv=2, d=128, dtype=HP_BF16, scale=0.088, q=FAKE):
    return Query(q, B, Hq, Hkv, d, dtype, scale)


def node_(len_=100, b0=0, b1=4, k=FAKE, v=FAKE, st=256, sh=128):
    return PrefixNode(k, v, st, sh, len_, b0, b1)


def kv_(max_blocks=4, block_size=16, num_blocks=20, k=FAKE, v=FAKE, tbl=FAKE, lens=FAKE,
        layout=0):
    return PagedKV(k, v, tbl, lens, max_blocks, block_size, num_blocks, layout)


def prefix_status(L, q, n, o=FAKE, lse=FAKE, ws=None, wsb=0):
    return L.hp_prefix_attn(ctypes.byref(q) if q is not None else None,
                            ctypes.byref(n) if n is not None else None, o, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=6, Hkv=4), INVALID),
    (dict(B=-1), INVALID),
    (dict(Hkv=0), INVALID),
    (dict(dtype=7), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=-0.088), INVALID),          # negative scale: the max of the raw scores is not
    (dict(scale=float("-inf")), INVALID),   # the max of the scaled ones
    (dict(d=96), UNSUPPORTED),
    (dict(Hq=48, Hkv=3), UNSUPPORTED),      # group of 16
    (dict(Hq=6, Hkv=2), UNSUPPORTED),       # group of 3
    (dict(q=0), NULL),
    (dict(q=FAKE + 8), INVALID),            # misaligned
])
def test_query_validation(L, kw, code):
    assert prefix_status(L, q_(**kw), node_()) == code


@pytest.mark.parametrize("kw,code", [
    (dict(b0=2, b1=2), INVALID),
    (dict(b0=-1), INVALID),
    (dict(b1=5), INVALID),
    (dict(len_=-3), INVALID),
    (dict(k=0), NULL),
    (dict(k=FAKE + 4), INVALID),
    (dict(st=100), INVALID),                # not a multiple of 16 bytes
    (dict(sh=0), INVALID),
    (dict(sh=64), INVALID),                 # heads would overlap (Hkv > 1, d = 128)
])
def test_node_validation(L, kw, code):
    assert prefix_status(L, q_(), node_(**kw)) == code


def test_null_and_output_checks(L):
    assert prefix_status(L, None, node_()) == NULL
    assert prefix_status(L, q_(), None) == NULL
    assert prefix_status(L, q_(), node_(), o=None) == NULL
    assert prefix_status(L, q_(), node_(), o=FAKE + 4) == INVALID
    assert prefix_status(L, q_(), node_(), lse=FAKE + 2) == INVALID


def test_prefix_workspace_sizing_and_check(L):
    # a long node is split across workgroups: needs workspace, and refuses a short one
    q = q_(B=64, Hq=32, Hkv=8)
    n = node_(len_=4096, b0=0, b1=64, st=8 * 128, sh=128)
    sz = ctypes.c_size_t()
    assert L.hp_prefix_attn_workspace_size(ctypes.byref(q), ctypes.byref(n), ctypes.byref(sz)) == OK
    assert sz.value > 0
    assert prefix_status(L, q, n, ws=None, wsb=0) == WORKSPACE
    assert prefix_status(L, q, n, ws=FAKE, wsb=sz.value - 1) == WORKSPACE
    assert L.hp_prefix_attn_workspace_size(ctypes.byref(q), ctypes.byref(n), None) == NULL


def suffix_status(L, q, kv, o=FAKE, ws=None, wsb=0):
    return L.hp_suffix_decode(ctypes.byref(q), ctypes.byref(kv) if kv is not None else None, o,
                              FAKE, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(block_size=32), UNSUPPORTED),
    (dict(max_blocks=0), INVALID),
    (dict(num_blocks=0), INVALID),
    (dict(k=0), NULL),
    (dict(tbl=0), NULL),
    (dict(lens=0), NULL),
    (dict(v=FAKE + 2), INVALID),
    (dict(tbl=FAKE + 2), INVALID),
    (dict(layout=2), INVALID),
    (dict(layout=-1), INVALID),
])
def test_paged_validation(L, kw, code):
    assert suffix_status(L, q_(), kv_(**kw)) == code


def test_suffix_workspace(L):
    """The suffix pass combines the waves of one (sequence, KV head) in LDS: it never
    needs workspace, for short or long suffixes."""
    q = q_(B=256, Hq=32, Hkv=32)
    sz = ctypes.c_size_t(1)
    for mb in (1, 8, 32, 64):
        kv = kv_(max_blocks=mb)
        assert L.hp_suffix_decode_workspace_size(ctypes.byref(q), ctypes.byref(kv),
                                                 ctypes.byref(sz)) == OK
        assert sz.value == 0


def merge_status(L, n, outs, lses, o, lse, rows=10, d=128):
    po = (p * max(1, n))(*outs)
    pl = (p * max(1, n))(*lses)
    return L.hp_lse_merge(n, ctypes.addressof(po), ctypes.addressof(pl), o, lse, rows, d, None)


def test_merge_validation(L):
    a, b = 0x100000, 0x200000
    out, lse = 0x300000, 0x400000
    assert merge_status(L, 0, [a], [b], out, lse) == INVALID
    assert merge_status(L, 17, [a] * 17, [b] * 17, out, lse) == INVALID
    assert merge_status(L, 1, [a], [b], out, lse, d=96) == UNSUPPORTED
    assert merge_status(L, 1, [a], [b], out, lse, rows=-1) == INVALID
    assert merge_status(L, 1, [0], [b], out, lse) == NULL
    assert merge_status(L, 1, [a + 4], [b], out, lse) == INVALID
    assert merge_status(L, 1, [a], [b], a + 512, lse) == INVALID      # output overlaps an input
    assert merge_status(L, 1, [a], [b], out, b + 4) == INVALID        # lse overlaps an input lse
    assert merge_status(L, 2, [a, b], [out, lse], 0x500000, 0x600000, rows=0) == OK  # nothing to do
    assert L.hp_lse_merge(1, None, None, out, lse, 10, 128, None) == NULL


def tree_status(L, q, levels, kv=None, o=FAKE, num_levels=None, share_min=1):
    flat = [n for lvl in levels for n in lvl]
    arr = (PrefixNode * max(1, len(flat)))(*flat)
    counts = (ctypes.c_int32 * 4)(*([len(l) for l in levels[:4]] + [0] * (4 - len(levels[:4]))))
    tree = PrefixTree(len(levels) if num_levels is None else num_levels, counts,
                      ctypes.cast(arr, ctypes.POINTER(PrefixNode)), share_min)
    sz = ctypes.c_size_t()
    st = L.hp_cascade_workspace_size(ctypes.byref(q), ctypes.byref(tree),
                                     ctypes.byref(kv) if kv else None, ctypes.byref(sz))
    st2 = L.hp_cascade_step(ctypes.byref(q), ctypes.byref(tree), ctypes.byref(kv) if kv else None,
                            o, FAKE, None, 0, None)
    return st, st2, sz.value


def test_tree_validation(L):
    q = q_(B=8)
    good = [[node_(64, 0, 8)], [node_(16, 0, 3), node_(16, 5, 8)]]
    st, st2, sz = tree_status(L, q, good, kv_())
    assert st == OK and sz > 0 and st2 == WORKSPACE
    overlap = [[node_(64, 0, 8)], [node_(16, 0, 4), node_(16, 3, 8)]]
    assert tree_status(L, q, overlap)[0] == INVALID
    unsorted = [[node_(64, 0, 8)], [node_(16, 5, 8), node_(16, 0, 3)]]
    assert tree_status(L, q, unsorted)[0] == INVALID
    deep = [[node_(16, 0, 8)]] * 4
    assert tree_status(L, q, deep, num_levels=5)[0] == UNSUPPORTED   # 5 levels
    assert tree_status(L, q, deep, num_levels=-1)[0] == UNSUPPORTED
    wide = [[node_(16, i % 8, i % 8 + 1) for i in range(8)] for _ in range(4)]
    wide[3] = wide[3] + [node_(16, 0, 1)]                     # 33 nodes
    assert tree_status(L, q, wide)[0] in (UNSUPPORTED, INVALID)
    bad_node = [[node_(64, 0, 9)]]
    assert tree_status(L, q, bad_node)[0] == INVALID


def tree_ws(L, q, levels, kv=None, share_min=1):
    """hp_cascade_workspace_size only (a step with nothing to batch would enqueue)."""
    flat = [n for lvl in levels for n in lvl]
    arr = (PrefixNode * max(1, len(flat)))(*flat)
    counts = (ctypes.c_int32 * 4)(*([len(l) for l in levels] + [0] * (4 - len(levels))))
    tree = PrefixTree(len(levels), counts, ctypes.cast(arr, ctypes.POINTER(PrefixNode)),
                      share_min)
    sz = ctypes.c_size_t(7)
    st = L.hp_cascade_workspace_size(ctypes.byref(q), ctypes.byref(tree),
                                     ctypes.byref(kv) if kv else None, ctypes.byref(sz))
    return st, sz.value


def test_tree_share_min(L):
    """share_min picks the nodes the prefix pass batches; the others need no partials
    (each of their sequences reads them in the suffix pass)."""
    q = q_(B=64, Hq=32, Hkv=8)
    levels = [[node_(4096, 0, 64)], [node_(300, 0, 32), node_(300, 32, 64)]]
    sizes = {}
    for smin in (0, 1, 2, 33, 64, 65):
        st, sz = tree_ws(L, q, levels, kv_(), share_min=smin)
        assert st == OK, smin
        sizes[smin] = sz
    # automatic: the 4096-token root over 64 sequences is batched, the 300-token
    # group nodes (32 sequences, 4 query heads per KV head) are read privately
    assert hp.share_decision(32, 8, 4096, 64) and not hp.share_decision(32, 8, 300, 32)
    assert sizes[1] == sizes[2] > sizes[0] == sizes[33] == sizes[64] > 0
    assert sizes[65] == 0                      # no node has 65 sequences: nothing batched
    assert tree_ws(L, q, levels, kv_(), share_min=-1)[0] == INVALID
    assert tree_ws(L, q, levels, None, share_min=65) == (OK, 0)
    # a step with batched nodes still checks its workspace before enqueuing anything
    for smin in (0, 1):
        assert tree_status(L, q, levels, kv_(), share_min=smin)[1] == WORKSPACE
    assert tree_status(L, q, levels, kv_(), share_min=-1)[1] == INVALID
    assert tree_status(L, q, levels, kv_(), o=None, share_min=65)[1] == NULL


def test_cascade_null_tree_and_kv(L):
    q = q_(B=8)
    sz = ctypes.c_size_t(123)
    assert L.hp_cascade_workspace_size(ctypes.byref(q), None, None, ctypes.byref(sz)) == OK
    assert sz.value == 0
    assert L.hp_cascade_step(ctypes.byref(q), None, None, None, None, None, 0, None) == NULL
    q0 = q_(B=0)
    assert L.hp_cascade_step(ctypes.byref(q0), None, None, FAKE, FAKE, None, 0, None) == OK


@pytest.mark.parametrize("cfg", workloads.all_configs(), ids=lambda c: c.name)
def test_workspace_for_every_workload(L, cfg):
    """The size query accepts every workload shape (nodes and pool described with fake
    aligned pointers) and asks for at least the split partials of the suffix pass."""
    q = q_(B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d,
           dtype={"f32": HP_F32, "f16": HP_F16, "bf16": HP_BF16}[cfg.dtype],
           scale=workloads.scale_for(cfg.d))
    levels = [[node_(ln, b0, b1, st=cfg.Hkv * cfg.d, sh=cfg.d) for (ln, b0, b1) in lvl]
              for lvl in cfg.levels]
    st, st2, sz = tree_status(L, q, levels, kv_(max_blocks=cfg.max_blocks))
    assert st == OK and st2 == WORKSPACE and sz > 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(hp, "_lib", None)
    monkeypatch.setattr(hp, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        hp.lib()


def test_timed_step_events_checked(L):
    """hp_cascade_step_timed: a NULL event array with a nonzero count is rejected before
    anything is enqueued, and counts other than 0, 4 and 5 are invalid."""
    q = q_()
    kv = kv_()
    step = L.hp_cascade_step_timed
    assert step(ctypes.byref(q), None, ctypes.byref(kv), FAKE, FAKE, FAKE, 1 << 30, None, None,
                None, 4) == NULL
    assert step(ctypes.byref(q), None, ctypes.byref(kv), FAKE, FAKE, FAKE, 1 << 30, None, None,
                None, 5) == NULL
    ev = (ctypes.c_void_p * 3)()
    assert step(ctypes.byref(q), None, ctypes.byref(kv), FAKE, FAKE, FAKE, 1 << 30, None, None,
                ctypes.addressof(ev), 3) == INVALID


def test_negative_scale_rejected_by_every_step(L):
    """Every entry point that reads a query rejects a negative scale before any launch."""
    q = q_(scale=-1.0)
    n = node_()
    assert prefix_status(L, q, n) == INVALID
    kv = kv_()
    assert L.hp_suffix_decode(ctypes.byref(q), ctypes.byref(kv), FAKE, FAKE, None, 0,
                              None) == INVALID
    assert L.hp_cascade_step(ctypes.byref(q), None, ctypes.byref(kv), FAKE, FAKE, FAKE, 1 << 30,
                             None) == INVALID
    q0 = q_(scale=0.0)  # zero is allowed: every score is 0
    sz = ctypes.c_size_t(0)
    assert L.hp_cascade_workspace_size(ctypes.byref(q0), None, ctypes.byref(kv),
                                       ctypes.byref(sz)) == OK


def test_read_probe_validation(L):
    """hp_read_probe: pointer, size and alignment checks (before anything is enqueued)."""
    assert L.hp_read_probe(None, 16, FAKE, None) == NULL
    assert L.hp_read_probe(FAKE, 16, None, None) == NULL
    assert L.hp_read_probe(FAKE, 15, FAKE, None) == INVALID
    assert L.hp_read_probe(FAKE + 8, 16, FAKE, None) == INVALID
    assert L.hp_read_probe(FAKE, 16, FAKE + 2, None) == INVALID
