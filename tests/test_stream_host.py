"""Shared-context streams on the CPU: the stream-id mask of the oracle against the
Parallel Prompting page's Figure 2, the generator's row layout against the rule that a
stream's visible tokens are the shared ones and its own, the masked softmax against a
dense -inf mask, and the C ABI's validation of hp_stream_decode (no GPU needed)."""
import ctypes
import json
import os

import numpy as np
import pytest
import torch

import decode_attention_shared_amd as hp
import oracle
import workloads
from decode_attention_shared_amd import HP_BF16, PrefixNode, PrefixTree, Query, StreamRows

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
OK, NULL, INVALID, WORKSPACE = 0, 1, 2, 4
FAKE = 0x10000


def small_step(seed=0, dtype="bf16", P=5, shared=2, answer=3):
    cfg = workloads.custom("streams_small", B=12, Hq=4, Hkv=2, d=64, dtype=dtype,
                           levels=(((40, 0, 12),),), suffix_lo=answer, suffix_hi=20)
    return workloads.stream_step(cfg, P=P, seed=seed, answer_len=answer, shared_len=shared)


def test_mask_matches_figure2():
    g = json.load(open(os.path.join(GOLDEN, "stream_mask_figure2.json")))
    vis = oracle.visible_positions(g["slot_sid"], g["query_sid"])
    assert vis.tolist() == g["visible"]
    # the other two streams see the document and their own slots, by the same rule
    assert oracle.visible_positions(g["slot_sid"], 0).tolist() == [0, 1, 2, 3, 6, 9]
    assert oracle.visible_positions(g["slot_sid"], 2).tolist() == [0, 1, 2, 5, 8, 11]


@pytest.mark.parametrize("seed,P,shared,answer", [(0, 5, 2, 3), (1, 1, 0, 0), (2, 12, 3, 1),
                                                  (3, 4, 0, 3)])
def test_each_stream_sees_what_it_would_see_alone(seed, P, shared, answer):
    st = small_step(seed, P=P, shared=shared, answer=answer)
    for b in range(st.cfg.B):
        r, s = int(st.q_req[b]), int(st.q_sid[b])
        n = int(st.row_len[r])
        vis = oracle.visible_positions(st.row_sid[r, :n].tolist(), s)
        assert vis.tolist() == st.own_positions(b)
        assert len(vis) == shared + int(st.own_lens[b])


def test_pool_holds_the_row_bytes_and_padding_is_never_visible():
    st = small_step(4)
    for r in range(st.R):
        n = int(st.row_len[r])
        idx = st.row_slots[r, :n].long()
        assert torch.equal(st.k_pool[idx].view(torch.int16), st.row_k[r].view(torch.int16))
        assert torch.equal(st.v_pool[idx].view(torch.int16), st.row_v[r].view(torch.int16))
        assert (st.row_sid[r, n:] == -3).all()
    used = torch.cat([st.row_slots[r, :int(st.row_len[r])] for r in range(st.R)])
    assert len(set(used.tolist())) == used.numel()       # distinct pool rows
    free = sorted(set(range(st.k_pool.shape[0])) - set(used.tolist()))
    assert torch.isnan(st.k_pool[free].float()).all()    # everything else is a NaN trap


def dense_masked(step, b, h):
    """fp64 softmax over the document and the whole request row, masked scores -inf."""
    cfg = step.cfg
    g = h // cfg.G
    r, s = int(step.q_req[b]), int(step.q_sid[b])
    n = int(step.row_len[r])
    ks = [nd.k[:, g].double() for lv in step.levels for nd in lv if nd.seq_begin <= b < nd.seq_end]
    vs = [nd.v[:, g].double() for lv in step.levels for nd in lv if nd.seq_begin <= b < nd.seq_end]
    ks.append(step.row_k[r][:, g].double())
    vs.append(step.row_v[r][:, g].double())
    K, V = torch.cat(ks), torch.cat(vs)
    sc = (K @ step.q[b, h].double()) * float(np.float32(step.scale))
    doc = K.shape[0] - n
    sid = step.row_sid[r, :n]
    masked = torch.cat([torch.zeros(doc, dtype=torch.bool), ~((sid == -1) | (sid == s))])
    sc[masked] = float("-inf")
    m = sc.max()
    w = torch.exp(sc - m)
    return (w @ V / w.sum()).numpy(), float(m + torch.log(w.sum()))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_oracle_equals_dense_masked_softmax(dtype):
    st = small_step(5, dtype=dtype)
    o, lse = oracle.stream_attention(st)
    for b in range(st.cfg.B):
        for h in range(st.cfg.Hq):
            od, ld = dense_masked(st, b, h)
            r = b * st.cfg.Hq + h
            assert np.max(np.abs(o[r] - od)) < 1e-12
            assert abs(lse[r] - ld) < 1e-12


def test_other_streams_do_not_change_a_stream():
    """Rewriting every other stream's keys and values leaves a stream's result as is."""
    st = small_step(6)
    o1, l1 = oracle.stream_attention(st)
    b = 6
    r, s = int(st.q_req[b]), int(st.q_sid[b])
    n = int(st.row_len[r])
    other = ~((st.row_sid[r, :n] == -1) | (st.row_sid[r, :n] == s))
    st.row_k[r][other] = -st.row_k[r][other] * 3
    st.row_v[r][other] = st.row_v[r][other] + 5
    o2, l2 = oracle.stream_attention(st)
    rows = slice(b * st.cfg.Hq, (b + 1) * st.cfg.Hq)
    assert np.array_equal(o1[rows], o2[rows]) and np.array_equal(l1[rows], l2[rows])


# ------------------------------- C ABI --------------------------------------

@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hp.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return hp.lib()


def rows_(**kw):
    f = dict(k_pool=FAKE, v_pool=FAKE, row_slots=FAKE, slot_sid=FAKE, row_len=FAKE, q_req=FAKE,
             q_sid=FAKE, num_requests=3, row_cap=100, pool_rows=500)
    f.update(kw)
    return StreamRows(*[f[n] for n, _ in StreamRows._fields_])


def size(L, q, tree, rows):
    n = ctypes.c_size_t(0)
    st = L.hp_stream_decode_workspace_size(ctypes.byref(q) if q else None,
                                           ctypes.byref(tree) if tree else None,
                                           ctypes.byref(rows) if rows else None,
                                           ctypes.byref(n))
    return st, n.value


def q_(B=12):
    return Query(FAKE, B, 4, 2, 128, HP_BF16, 0.088)


def doc_():
    nodes = (PrefixNode * 1)(PrefixNode(FAKE, FAKE, 256, 128, 300, 0, 12))
    counts = (ctypes.c_int32 * hp.HP_MAX_LEVELS)(1, 0, 0, 0)
    return PrefixTree(1, counts, ctypes.cast(nodes, ctypes.POINTER(PrefixNode))), nodes


def test_workspace_covers_tables(L):
    tree, keep = doc_()
    st, n_doc = size(L, q_(), tree, rows_())
    assert st == OK
    st, n_none = size(L, q_(), None, rows_())
    assert st == OK and n_none >= 12 * 100 * 4 + 12 * 4
    st, n_big = size(L, q_(), None, rows_(row_cap=1000))
    assert st == OK and n_big - n_none >= 12 * 900 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(k_pool=0), NULL), (dict(row_slots=0), NULL), (dict(slot_sid=0), NULL),
    (dict(row_len=0), NULL), (dict(q_req=0), NULL), (dict(q_sid=0), NULL),
    (dict(num_requests=0), INVALID), (dict(row_cap=0), INVALID), (dict(pool_rows=0), INVALID),
    (dict(pool_rows=1 << 31), INVALID), (dict(k_pool=FAKE + 4), INVALID),
    (dict(row_len=FAKE + 2), INVALID), (dict(q_sid=FAKE + 1), INVALID),
])
def test_rows_validation(L, kw, code):
    assert size(L, q_(), None, rows_(**kw))[0] == code
    # the step itself refuses the same arguments before enqueueing anything
    st = L.hp_stream_decode(ctypes.byref(q_()), None, ctypes.byref(rows_(**kw)), FAKE, FAKE,
                            FAKE, 1 << 30, None)
    assert st == code


def test_step_checks_workspace_and_outputs(L):
    r = rows_()
    q = q_()
    need = size(L, q, None, r)[1]
    assert L.hp_stream_decode(ctypes.byref(q), None, ctypes.byref(r), FAKE, FAKE, None, need,
                              None) == WORKSPACE
    assert L.hp_stream_decode(ctypes.byref(q), None, ctypes.byref(r), FAKE, FAKE, FAKE,
                              need - 1, None) == WORKSPACE
    assert L.hp_stream_decode(ctypes.byref(q), None, ctypes.byref(r), None, FAKE, FAKE, need,
                              None) == NULL
    assert L.hp_stream_decode(ctypes.byref(q), None, None, FAKE, FAKE, FAKE, need,
                              None) == NULL
    # B = 0 is a valid empty step: nothing to enqueue
    q0 = q_(B=0)
    assert L.hp_stream_decode(ctypes.byref(q0), None, ctypes.byref(r), FAKE, FAKE, None, 0,
                              None) == OK
