"""The batching policy (hp_share_decision) on the CPU: it picks the faster path at every
decisive point of the measured crossover grids (profiles/share_sweep_<dtype>_d<d>.json, MI355X
timings of both paths for bf16, fp16 and fp32 at d = 128 and 64), it is monotone, and the
chunk-tree planner's automatic mode (share_min = 0) batches exactly the runs it chooses."""
import ctypes
import json
import os

import pytest
import torch

import decode_attention_shared_amd as hp
from decode_attention_shared_amd import HP_BF16, Query

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SWEEPS = [("bf16", 128), ("f16", 128), ("bf16", 64), ("f16", 64), ("f32", 128), ("f32", 64)]
TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hp.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return hp.lib()


@pytest.mark.parametrize("dtype,d", SWEEPS)
def test_policy_picks_the_measured_winner(L, dtype, d):
    data = json.load(open(os.path.join(ROOT, "profiles", f"share_sweep_{dtype}_d{d}.json")))
    assert (data["dtype"], data["d"]) == (dtype, d)
    decisive = 0
    for r in data["share_sweep"]:
        ratio = r["private_us"] / r["batched_us"]
        if abs(ratio - 1.0) < 0.05:       # a tie within timing noise: either path is fine
            continue
        decisive += 1
        got = hp.share_decision(r["Hq"], r["Hkv"], r["tokens"], r["nseq"], d=d, dtype=TORCH[dtype])
        assert got == (ratio > 1.0), r
    assert decisive >= 90


@pytest.mark.parametrize("dtype,d", SWEEPS)
@pytest.mark.parametrize("Hq,Hkv", [(32, 32), (32, 8), (16, 8), (8, 1)])
def test_policy_monotone(L, Hq, Hkv, dtype, d):
    toks = [0, 1, 63, 64, 128, 255, 256, 511, 512, 1023, 1024, 2047, 2048, 4096, 1 << 20]
    seqs = [0, 1, 2, 3, 4, 7, 8, 9, 16, 31, 32, 33, 64, 65, 128, 129, 255, 256, 1000]

    def dec(t, n):
        return hp.share_decision(Hq, Hkv, t, n, d=d, dtype=TORCH[dtype])
    for n in seqs:
        row = [dec(t, n) for t in toks]
        assert row == sorted(row), (n, row)          # more shared tokens never un-batches
    for t in toks:
        col = [dec(t, n) for n in seqs]
        assert col == sorted(col), (t, col)          # more sharers never un-batches
    assert not any(dec(t, n) for t in toks for n in (0, 1))
    assert all(dec(2048, n) for n in seqs if n >= 2)


def test_policy_validation(L):
    out = ctypes.c_int32(7)
    q = Query(None, 64, 32, 8, 128, HP_BF16, 1.0)
    assert L.hp_share_decision(ctypes.byref(q), 100, 65, ctypes.byref(out)) == 2   # nseq > B
    assert L.hp_share_decision(ctypes.byref(q), -1, 2, ctypes.byref(out)) == 2
    assert L.hp_share_decision(ctypes.byref(q), 100, 2, None) == 1
    q.d = 96
    assert L.hp_share_decision(ctypes.byref(q), 100, 2, ctypes.byref(out)) == 3
    assert out.value == 7                                 # nothing written on an error


def test_auto_plan_batches_the_chosen_runs(L):
    # run A: 512 rows over 64 sequences (batched: 512 >= 256); run B: 128 rows over
    # [64, 66) (private: 2 sequences need 1024 rows with one query head per KV head);
    # run C: 1024 rows over [66, 70) (batched); then one private chunk per sequence.
    descs = [(64 * i, 64, 0, 64) for i in range(8)]
    descs += [(512 + 64 * i, 64, 64, 66) for i in range(2)]
    descs += [(640 + 64 * i, 64, 66, 70) for i in range(16)]
    descs += [(1664 + 64 * b, 64, b, b + 1) for b in range(70)]
    B = 70
    assert hp.share_decision(4, 4, 512, 64) and not hp.share_decision(4, 4, 128, 2)
    assert hp.share_decision(4, 4, 1024, 4)
    plan, _ = hp.tree_plan_build(B, 4, 4, 128, torch.bfloat16, descs, 0, 1664 + 64 * B)
    assert plan.num_segs == 2 and plan.num_pieces == 8 + 16
    assert plan.num_tok_rows == 2 * 128 + 64 * B       # run B read by each of its 2 sequences
    # a fixed threshold of 2 batches all three runs
    plan2, _ = hp.tree_plan_build(B, 4, 4, 128, torch.bfloat16, descs, 2, 1664 + 64 * B)
    assert plan2.num_segs == 3 and plan2.num_tok_rows == 64 * B
