"""Host tests of the chunk-tree plan builder and the oracle's tree pins (no GPU).

Plan: argument validation, the segment grouping of batched descriptors, the
split bound the kernels rely on (at most 64 tiles per split), the row counts
of the image, and the size query / capacity protocol of hp_tree_plan_build.

Oracle pins: ``oracle.tree_attention`` (a gather of each sequence's rows,
then the pinned fp64 attention) is checked against an independent dense
formulation -- a [B][rows] visibility mask built from the descriptors with
numpy, and a masked softmax over the whole pool -- and ``oracle.kv_append``
against numpy fancy assignment.
"""
import ctypes

import numpy as np
import pytest
import torch

import decode_attention_shared_amd as hp
import oracle
import workloads


def _plan(descs, B=8, Hq=4, Hkv=2, d=64, dtype=torch.bfloat16, share_min=2, pool_rows=4096):
    return hp.tree_plan_build(B, Hq, Hkv, d, dtype, descs, share_min, pool_rows)


def test_plan_segments_and_rows():
    # root run of 2 chunks over [0,8), a 1-chunk child over [0,4), a 3-chunk child
    # over [4,8), then private pieces; share_min 2 batches the first three runs.
    descs = [(0, 64, 0, 8), (64, 64, 0, 8), (128, 10, 0, 4), (192, 64, 4, 8),
             (256, 64, 4, 8), (320, 5, 4, 8), (384, 3, 0, 1), (448, 64, 5, 6)]
    plan, blob = _plan(descs)
    assert plan.num_segs == 3 and plan.num_pieces == 6
    assert plan.num_tok_rows == 3 + 64
    assert plan.max_private == 64
    assert plan.num_srcs == 8 + 4 + 4
    assert blob.numel() >= plan.blob_bytes > 0
    # a higher threshold makes the 4-sequence children private
    plan5, _ = _plan(descs, share_min=5)
    assert plan5.num_segs == 1 and plan5.num_pieces == 2
    assert plan5.num_tok_rows == 4 * 10 + 4 * (64 + 64 + 5) + 3 + 64


def test_plan_split_bound():
    # 300 full tiles over 4 sequences: every split holds at most 64 tiles
    descs = [(64 * i, 64, 0, 4) for i in range(300)]
    plan, _ = _plan(descs, B=4, Hq=8, Hkv=8, pool_rows=64 * 300)
    assert plan.num_segs == 1
    # partial rows = sequences x splits, splits >= ceil(300 / 64)
    assert plan.part_rows >= 4 * 5
    assert plan.workspace_bytes >= plan.part_rows * 8 * 64 * 4


def test_plan_same_range_not_adjacent_is_two_segments():
    descs = [(0, 64, 0, 4), (64, 1, 0, 1), (128, 64, 0, 4)]
    plan, _ = _plan(descs, B=4)
    assert plan.num_segs == 2


@pytest.mark.parametrize("bad,status", [
    ((0, 0, 0, 1), 2), ((0, 65, 0, 1), 2), ((-1, 4, 0, 1), 2), ((4090, 10, 0, 1), 2),
    ((0, 4, 1, 1), 2), ((0, 4, 0, 9), 2), ((0, 4, -1, 2), 2)])
def test_plan_rejects(bad, status):
    with pytest.raises(hp.HpError) as e:
        _plan([(0, 64, 0, 8), bad])
    assert e.value.status == status


def test_plan_threshold_and_geometry():
    with pytest.raises(hp.HpError) as e:
        _plan([(0, 64, 0, 8)], share_min=1)
    assert e.value.status == 2
    with pytest.raises(hp.HpError) as e:
        _plan([(0, 64, 0, 8)], d=96)
    assert e.value.status == 3


def test_plan_capacity_protocol():
    L = hp.lib()
    geom = hp.Query(None, 8, 4, 2, 64, hp.HP_BF16, 1.0)
    arr, n = hp._descs_array([(0, 64, 0, 8), (64, 7, 2, 3)])
    plan = hp.TreePlan()
    assert L.hp_tree_plan_build(ctypes.byref(geom), ctypes.addressof(arr), n, 2, 4096, None, 0,
                                ctypes.byref(plan)) == 0
    small = (ctypes.c_uint8 * max(1, plan.blob_bytes - 4))()
    assert L.hp_tree_plan_build(ctypes.byref(geom), ctypes.addressof(arr), n, 2, 4096,
                                ctypes.addressof(small), ctypes.sizeof(small),
                                ctypes.byref(plan)) == 6


def test_empty_plan():
    plan, _ = _plan([], B=5)
    assert plan.num_segs == 0 and plan.num_tok_rows == 0 and plan.workspace_bytes == 0


# ------------------------------------------------------------------ oracle pins

def _dense_masked_attention(step):
    """Every pool row is a candidate key; row r is visible to sequence b iff some
    descriptor holding b names it and it falls within b's first seq_lens[b] rows
    (counted in descriptor order).  Plain masked softmax in float64."""
    R = step.pool_rows
    order = np.full((step.B, R), -1, dtype=np.int64)  # position of row r in b's list
    pos = np.zeros(step.B, dtype=np.int64)
    for (r, c, b0, b1) in step.descs.tolist():
        for b in range(b0, b1):
            order[b, r:r + c] = pos[b] + np.arange(c)
            pos[b] += c
    visible = (order >= 0) & (order < step.seq_lens[:, None])
    K = step.k_pool.double().numpy()
    V = step.v_pool.double().numpy()
    Q = step.q.double().numpy()
    G = step.Hq // step.Hkv
    o = np.zeros((step.B, step.Hq, step.d))
    lse = np.full((step.B, step.Hq), -np.inf)
    for b in range(step.B):
        idx = np.nonzero(visible[b])[0]
        if idx.size == 0:
            continue
        for h in range(step.Hq):
            s = step.scale * (K[idx, h // G] @ Q[b, h])
            m = s.max()
            w = np.exp(s - m)
            o[b, h] = (w @ V[idx, h // G]) / w.sum()
            lse[b, h] = m + np.log(w.sum())
    return o.reshape(-1, step.d), lse.reshape(-1)


@pytest.mark.parametrize("seed", range(3))
def test_oracle_tree_attention_pin(seed):
    step = workloads.random_chunk_tree(seed, B=9, Hq=4, Hkv=2, d=64, dtype="bf16", depth=3,
                                       max_chunks=2, root_chunks=2)
    o, l = oracle.tree_attention(step)
    ro, rl = _dense_masked_attention(step)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(l), fin)
    assert np.abs(o - ro).max() < 1e-12
    assert np.abs(l[fin] - rl[fin]).max() < 1e-12


def test_chunk_tree_generator_layout():
    step = workloads.random_chunk_tree(7, B=20, Hq=2, Hkv=1, d=64, dtype="f16")
    named = set()
    for (r, c, b0, b1) in step.descs.tolist():
        assert r // 64 == (r + c - 1) // 64 and 1 <= c <= 64 and 0 <= b0 < b1 <= 20
    for b in range(step.B):
        rows = step.rows_of(b)
        named.update(rows)
        assert len(rows) == step.seq_lens[b]
        assert torch.isfinite(step.k_pool[rows].float()).all()
    unnamed = sorted(set(range(step.pool_rows)) - named)
    assert torch.isnan(step.k_pool[unnamed].float()).all()


def test_oracle_kv_append_pin():
    g = torch.Generator().manual_seed(0)
    pool = torch.randn(50, 2, 8, generator=g).to(torch.bfloat16)
    new = torch.randn(6, 2, 8, generator=g).to(torch.bfloat16)
    rows = [3, 49, 0, -1, 50, 17]
    got = oracle.kv_append(pool, rows, new)
    ref = pool.clone().numpy() if pool.dtype != torch.bfloat16 else pool.view(torch.int16).numpy().copy()
    newb = new.view(torch.int16).numpy()
    ok = [i for i, r in enumerate(rows) if 0 <= r < 50]
    ref[np.asarray(rows)[ok]] = newb[ok]
    assert np.array_equal(got.view(torch.int16).numpy(), ref)
