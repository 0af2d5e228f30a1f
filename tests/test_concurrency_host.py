"""Policy for running a cascade step's suffix pass beside its prefix pass, on the CPU:
hp_cascade_overlap_plan reports the plan's choice for a mode (planning reads no device
memory, so fake addresses stand in for the device buffers), the workspace size covers
every mode, and hp_cascade_step_overlap validates the caller's streams and events
before anything is enqueued."""
import ctypes

import pytest

import decode_attention_shared_amd as hp


@pytest.fixture(scope="module")
def L():
    import os
    if not os.path.exists(hp.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return hp.lib()


FAKE = 1 << 40  # an aligned address: planning checks pointers, never reads them


def _args(B, Hq, Hkv, d, P, max_blocks, prefix=True, suffix=True, share_min=0):
    query = hp.Query(FAKE, B, Hq, Hkv, d, hp.HP_F16, 1.0)
    tree = kv = None
    keep = []
    if prefix:
        nodes = (hp.PrefixNode * 1)(hp.PrefixNode(FAKE, FAKE, Hkv * d, d, P, 0, B))
        tree = hp.PrefixTree()
        tree.num_levels = 1
        tree.nodes_per_level[0] = 1
        tree.share_min = share_min
        tree.nodes = ctypes.cast(nodes, ctypes.POINTER(hp.PrefixNode))
        keep.append(nodes)
    if suffix:
        kv = hp.PagedKV(FAKE, FAKE, FAKE, FAKE, max_blocks, 16, B * max_blocks)
    return query, tree, kv, keep


def _plan(L, args, mode=1):
    query, tree, kv, _ = args
    flag = ctypes.c_int32(-1)
    nbytes = ctypes.c_size_t(0)
    tp = ctypes.byref(tree) if tree is not None else None
    kp = ctypes.byref(kv) if kv is not None else None
    assert L.hp_cascade_overlap_plan(ctypes.byref(query), tp, kp, mode, ctypes.byref(flag)) == 0
    assert L.hp_cascade_workspace_size(ctypes.byref(query), tp, kp, ctypes.byref(nbytes)) == 0
    return flag.value, nbytes.value


@pytest.mark.parametrize("shape,want", [
    ((256, 40, 40, 128, 16384, 8), 1),    # the 16K MHA step: 64 tiles per split at 160 CUs
    ((256, 32, 32, 128, 16384, 32), 1),   # a 16K document, long suffixes
    ((256, 40, 40, 128, 8192, 8), 1),     # 8K: 32 tiles per split
    ((256, 40, 40, 128, 4096, 8), 1),     # 4K: 16 tiles per split
    ((256, 40, 40, 128, 2048, 8), 1),     # 2K: 8 tiles per split
    ((256, 40, 40, 128, 1024, 8), 1),     # 1K: 4 tiles per split
    ((256, 40, 40, 128, 512, 8), 0),      # 2 tiles per split
    ((64, 32, 8, 128, 4096, 16), 0),      # GQA, 512 suffix units
    ((128, 32, 8, 128, 16384, 8), 0),     # GQA, 1024 suffix units
    ((256, 5, 5, 128, 16384, 8), 2),      # one 8-way head share, 1280 units: one launch
    ((160, 8, 8, 128, 900, 9), 2),        # a small MHA step: one launch
    ((160, 8, 8, 64, 900, 9), 0),         # the same at d = 64: serial
    ((256, 32, 8, 128, 4096, 8), 1),      # GQA, 2048 suffix units
    ((16, 8, 8, 64, 16384, 4), 0),        # too few suffix units
])
def test_auto_policy(L, shape, want):
    assert _plan(L, _args(*shape))[0] == want


def test_auto_policy_two_level_gqa_side_by_side(L):
    # global 2K prefix over 256 sequences, eight 1K sub-prefixes of 32 each, GQA 32/8:
    # 2048 suffix units (measured 5 % faster side by side with the caches flushed)
    B, Hq, Hkv, d = 256, 32, 8, 128
    query = hp.Query(FAKE, B, Hq, Hkv, d, hp.HP_F16, 1.0)
    specs = [(2048, 0, B)] + [(1024, 32 * i, 32 * i + 32) for i in range(8)]
    nodes = (hp.PrefixNode * len(specs))(*[hp.PrefixNode(FAKE, FAKE, Hkv * d, d, P, b0, b1)
                                           for (P, b0, b1) in specs])
    tree = hp.PrefixTree()
    tree.num_levels = 2
    tree.nodes_per_level[0] = 1
    tree.nodes_per_level[1] = 8
    tree.nodes = ctypes.cast(nodes, ctypes.POINTER(hp.PrefixNode))
    kv = hp.PagedKV(FAKE, FAKE, FAKE, FAKE, 8, 16, B * 8)
    assert _plan(L, (query, tree, kv, [nodes]))[0] == 1


def test_modes_and_workspace(L):
    # a node the batching policy would leave to the suffix pass, batched on request
    B, Hq, Hkv, d = 8, 4, 2, 64
    args = _args(B, Hq, Hkv, d, 300, 4, share_min=1)
    off, ws = _plan(L, args, mode=0)
    assert off == 0
    on, ws_on = _plan(L, args, mode=2)
    assert on == 1
    assert ws_on == ws, "one workspace size serves every mode"

    def up(x):
        return (x + 255) // 256 * 256
    # the prefix partials for 160 compute units plus the suffix rows (O and LSE)
    assert ws >= up(B * Hq * d * 4) + up(B * Hq * 4)
    # prefix only or suffix only: nothing to run side by side
    assert _plan(L, _args(B, Hq, Hkv, d, 300, 4, suffix=False, share_min=1), mode=2)[0] == 0
    assert _plan(L, _args(B, Hq, Hkv, d, 300, 4, prefix=False), mode=2)[0] == 0
    assert _plan(L, args, mode=1)[0] == 0
    # the automatic policy reads this node in the suffix pass: nothing to overlap
    assert _plan(L, _args(B, Hq, Hkv, d, 300, 4), mode=2) == (0, 0)


def test_one_launch_mode(L):
    """Mode 3 puts both passes in one launch whenever the step qualifies (one prefix
    launch of the 256-row kernel, 16-bit, d = 128, G in {1, 2, 4}, K/V within the
    last-level cache, no private nodes), else it runs them one after the other."""
    assert _plan(L, _args(64, 32, 8, 128, 4096, 16), mode=3)[0] == 2    # GQA, 4 per KV head
    assert _plan(L, _args(96, 16, 8, 128, 700, 13), mode=3)[0] == 2     # GQA, 2 per KV head
    assert _plan(L, _args(160, 8, 8, 128, 900, 9), mode=3)[0] == 2      # MHA
    assert _plan(L, _args(256, 40, 40, 128, 16384, 8), mode=3)[0] == 0  # K/V beyond 256 MiB
    assert _plan(L, _args(160, 8, 8, 64, 900, 9), mode=3)[0] == 0       # d = 64
    assert _plan(L, _args(64, 64, 8, 128, 4096, 16), mode=3)[0] == 0    # 8 per KV head
    assert _plan(L, _args(64, 32, 8, 128, 4096, 16, suffix=False), mode=3)[0] == 0
    # the one-launch plan lays out the same workspace as the side-by-side one
    assert _plan(L, _args(160, 8, 8, 128, 900, 9), mode=3)[1] == \
        _plan(L, _args(160, 8, 8, 128, 900, 9), mode=2)[1]


def test_mode_validation(L):
    query, tree, kv, _ = _args(4, 2, 2, 64, 100, 2)
    flag = ctypes.c_int32(0)
    for bad in (4, -1):
        assert L.hp_cascade_overlap_plan(ctypes.byref(query), ctypes.byref(tree),
                                         ctypes.byref(kv), bad, ctypes.byref(flag)) == 2
    assert L.hp_cascade_overlap_plan(ctypes.byref(query), ctypes.byref(tree), ctypes.byref(kv),
                                     1, None) == 1


def test_overlap_handles_validated(L):
    """A side-by-side plan needs the caller's side stream and both events, and the side
    stream must differ from the step's stream; each is checked before any launch."""
    query, tree, kv, _ = _args(8, 4, 2, 64, 300, 4, share_min=1)
    step = L.hp_cascade_step_overlap
    args = (ctypes.byref(query), ctypes.byref(tree), ctypes.byref(kv), FAKE, FAKE, FAKE, 1 << 30)
    assert step(*args, None, None) == 1
    S, E1, E2 = 0x1000, 0x2000, 0x3000  # never dereferenced: validation fails first
    assert step(*args, None, ctypes.byref(hp.Overlap(None, E1, E2, 2))) == 1
    assert step(*args, None, ctypes.byref(hp.Overlap(S, None, E2, 2))) == 1
    assert step(*args, None, ctypes.byref(hp.Overlap(S, E1, None, 2))) == 1
    assert step(*args, S, ctypes.byref(hp.Overlap(S, E1, E2, 2))) == 2
    assert step(*args, None, ctypes.byref(hp.Overlap(S, E1, E2, 7))) == 2


def test_timed_event_count_validation(L):
    query, tree, kv, _ = _args(4, 2, 2, 64, 100, 2)
    ev = (ctypes.c_void_p * 6)()
    for n in (1, 3, 6, -1):
        assert L.hp_cascade_step_timed(ctypes.byref(query), ctypes.byref(tree), ctypes.byref(kv),
                                       FAKE, FAKE, None, 0, None, None, ctypes.addressof(ev),
                                       n) == 2


def _stream_args(B, Hq, Hkv, d, P, R=4, cap=512):
    query, tree, _, keep = _args(B, Hq, Hkv, d, P, 1, suffix=False)
    rows = hp.StreamRows(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, R, cap, R * cap)
    return query, tree, rows, keep


def _stream_plan(L, args, mode):
    query, tree, rows, _ = args
    flag = ctypes.c_int32(-1)
    tp = ctypes.byref(tree) if tree is not None else None
    st = L.hp_stream_overlap_plan(ctypes.byref(query), tp, ctypes.byref(rows), mode,
                                  ctypes.byref(flag))
    return st, flag.value


@pytest.mark.parametrize("shape,want", [
    ((256, 32, 8, 128, 16384), 1),   # 2048 (query, KV head) units, 64 tiles per split
    ((256, 32, 8, 128, 512), 0),     # 2 tiles per split
    ((128, 32, 8, 128, 16384), 0),   # 1024 units
])
def test_stream_decode_policy(L, shape, want):
    args = _stream_args(*shape)
    assert _stream_plan(L, args, 1) == (0, want)
    assert _stream_plan(L, args, 0) == (0, 0)
    assert _stream_plan(L, args, 2) == (0, 1)


def test_stream_decode_modes_validated(L):
    query, tree, rows, _ = args = _stream_args(8, 4, 2, 64, 300)
    for bad in (3, 4, -1):
        assert _stream_plan(L, args, bad)[0] == 2
    # no document: nothing to put beside the stream pass
    assert L.hp_stream_overlap_plan(ctypes.byref(query), None, ctypes.byref(rows), 2,
                                    ctypes.byref(ctypes.c_int32())) == 0
    nb = ctypes.c_size_t(0)
    assert L.hp_stream_decode_workspace_size(ctypes.byref(query), ctypes.byref(tree),
                                             ctypes.byref(rows), ctypes.byref(nb)) == 0
    step = L.hp_stream_decode_overlap
    a = (ctypes.byref(query), ctypes.byref(tree), ctypes.byref(rows), FAKE, FAKE, FAKE, 1 << 30)
    S, E1, E2 = 0x1000, 0x2000, 0x3000  # never dereferenced: validation fails first
    assert step(*a, None, None) == 1
    assert step(*a, None, ctypes.byref(hp.Overlap(None, E1, E2, 2))) == 1
    assert step(*a, None, ctypes.byref(hp.Overlap(S, None, E2, 2))) == 1
    assert step(*a, None, ctypes.byref(hp.Overlap(S, E1, None, 2))) == 1
    assert step(*a, S, ctypes.byref(hp.Overlap(S, E1, E2, 2))) == 2
    assert step(*a, None, ctypes.byref(hp.Overlap(S, E1, E2, 3))) == 2
