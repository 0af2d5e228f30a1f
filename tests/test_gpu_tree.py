"""GPU parity of the chunk-tree path, the KV append kernel and the PAKV manager
driving both, against the fp64 oracle, through the C ABI.

Tolerances as for the cascade (gpu_util.TOL).  Pool rows that no descriptor
names, and the room past each sequence's length, are NaN: a read of any of
them would show as a non-finite output.  The append kernel is checked
bit-exactly (it is a copy)."""
import numpy as np
import pytest
import torch

import decode_attention_shared_amd as hp
import oracle
import workloads
from gpu_util import DEV, compare, say

pytestmark = pytest.mark.gpu

_TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X (no GPU visible)")
    hp.lib()


def _run_tree(step, share_min, use_lens=True):
    q = step.q.to(DEV)
    ts = hp.TreeStep(q, step.Hkv, step.descs, share_min, step.pool_rows, step.scale)
    lens = torch.as_tensor(step.seq_lens, dtype=torch.int32, device=DEV) if use_lens else None
    out = torch.full(tuple(q.shape), 7.0, device=DEV)
    lse = torch.full(tuple(q.shape[:2]), 7.0, device=DEV)
    o, l = ts(q, step.k_pool.to(DEV), step.v_pool.to(DEV), lens, out=out, lse=lse)
    torch.cuda.synchronize()
    return o, l, ts.plan


# ------------------------------------------------------------------ random forests

TREE_CASES = [
    # dtype, d, B, Hq, Hkv, depth, share_min, seed
    ("bf16", 128, 37, 8, 2, 4, 2, 1),     # GQA 4, deep forest, partial pieces
    ("f16", 64, 21, 4, 4, 6, 2, 2),       # MHA, depth 6
    ("bf16", 64, 64, 8, 1, 3, 3, 3),      # MQA-like group of 8, threshold 3
    ("f16", 128, 300, 2, 2, 2, 2, 4),     # 300 rows per KV head at the root: 2 row blocks
    ("bf16", 128, 12, 8, 8, 5, 64, 5),    # threshold above B: everything private
    ("f32", 64, 10, 2, 1, 3, 2, 6),       # fp32 matrix path
    ("f32", 128, 33, 4, 2, 4, 4, 7),      # fp32, d=128
    ("bf16", 128, 160, 8, 2, 3, 0, 8),    # automatic batching policy, run by run
    ("f16", 128, 96, 4, 4, 4, 0, 9),      # automatic, MHA
]


@pytest.mark.parametrize("case", TREE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_tree_random_forest(case):
    dtype, d, B, Hq, Hkv, depth, share_min, seed = case
    say(f"tree {case}")
    step = workloads.random_chunk_tree(seed, B=B, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, depth=depth)
    o, l, plan = _run_tree(step, share_min)
    say(f"  segs {plan.num_segs} pieces {plan.num_pieces} private rows {plan.num_tok_rows} "
        f"launches {[plan.launch_nw[i] for i in range(plan.num_launches)]}")
    ro, rl = oracle.tree_attention(step)
    compare(o, l, ro, rl, dtype, f"tree {case}")


def test_tree_long_segment_splits():
    # a 20000-row root (313 pieces, the last partial) over 256 sequences of an MHA
    # layer, then private pieces: splits of at most 64 tiles, 8-wave row blocks
    cfg = workloads.custom("long", B=256, Hq=8, Hkv=8, d=128, dtype="bf16",
                           levels=(((20000, 0, 256),),), suffix_lo=1, suffix_hi=100)
    step = workloads.chunked_config(cfg, seed=3)
    say("tree long segment")
    o, l, plan = _run_tree(step, 2)
    assert plan.num_segs == 1 and plan.num_pieces == 313
    per = 64  # sequences per oracle pass (each pass gathers their keys from the pool)
    for b0 in range(0, step.B, per):
        rows = np.arange(b0 * step.Hq, min(step.B, b0 + per) * step.Hq)
        ro, rl = oracle.tree_attention(step, rows=rows)
        compare(o, l, ro, rl, "bf16", f"tree long segment, sequences {b0}..", rows=rows)


def test_tree_without_lengths_reads_every_row():
    step = workloads.random_chunk_tree(11, B=16, Hq=4, Hkv=2, d=64, dtype="bf16", room=False)
    say("tree without seq_lens")
    o, l, _ = _run_tree(step, 2, use_lens=False)
    ro, rl = oracle.tree_attention(step)
    compare(o, l, ro, rl, "bf16", "tree without seq_lens")


def test_tree_bad_lengths_give_nan_rows():
    step = workloads.random_chunk_tree(12, B=16, Hq=4, Hkv=2, d=64, dtype="bf16")
    q = step.q.to(DEV)
    ts = hp.TreeStep(q, step.Hkv, step.descs, 2, step.pool_rows, step.scale)
    lens = step.seq_lens.copy()
    bad = [2, 9]
    lens[2] = -1
    lens[9] = 100000
    o, l = ts(q, step.k_pool.to(DEV), step.v_pool.to(DEV),
              torch.as_tensor(lens, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    for b in bad:
        assert torch.isnan(o[b]).all() and torch.isnan(l[b]).all()
    good = [b for b in range(step.B) if b not in bad]
    rows = np.array([b * step.Hq + h for b in good for h in range(step.Hq)])
    ro, rl = oracle.tree_attention(step, rows=rows)
    compare(o, l, ro, rl, "bf16", "tree good rows", rows=rows)


def test_tree_empty_batch_rows():
    # descriptors only over [3, 6): the other sequences attend nothing
    step = workloads.random_chunk_tree(13, B=6, Hq=2, Hkv=1, d=64, dtype="f16", room=False)
    keep = [list(r) for r in step.descs.tolist() if r[2] >= 3]
    step.descs = np.asarray(keep, dtype=np.int32).reshape(-1, 4)
    step.seq_lens = np.array([len(step.rows_of(b)) if b >= 3 else 0 for b in range(6)],
                             dtype=np.int32)
    o, l, _ = _run_tree(step, 2)
    ro, rl = oracle.tree_attention(step)
    compare(o, l, ro, rl, "f16", "tree with empty rows")


# ------------------------------------------------------------- headline shape

def test_tree_codellama13b_16k_every_row():
    """The 16K-prefix CodeLlama-13B step as 256 root chunks + private suffix chunks: every
    row against the oracle, 16 sequences per oracle pass (each pass gathers its
    sequences' keys from the pool)."""
    step = workloads.chunked_config(workloads.codellama13b_mha(16384), seed=0)
    say("tree codellama13b 16K")
    o, l, plan = _run_tree(step, 2)
    per = 16
    for b0 in range(0, step.B, per):
        rows = np.arange(b0 * step.Hq, min(step.B, b0 + per) * step.Hq)
        ro, rl = oracle.tree_attention(step, rows=rows)
        compare(o, l, ro, rl, "f16", f"tree codellama13b 16K, sequences {b0}..", rows=rows)
    say(f"  tree 16K: all {step.B * step.Hq} rows checked")


# ------------------------------------------------------------------ append

@pytest.mark.parametrize("dtype,Hkv,d", [("bf16", 8, 128), ("f32", 2, 64), ("f16", 40, 128)])
def test_kv_append_bit_exact(dtype, Hkv, d):
    g = torch.Generator().manual_seed(5)
    dt = _TD[dtype]
    pool_rows, n = 300, 40
    kp = torch.randn(pool_rows, Hkv, d, generator=g).to(dt)
    vp = torch.randn(pool_rows, Hkv, d, generator=g).to(dt)
    kn = torch.randn(n, Hkv, d, generator=g).to(dt)
    vn = torch.randn(n, Hkv, d, generator=g).to(dt)
    rows = torch.randperm(pool_rows, generator=g)[:n].to(torch.int32)
    rows[3] = -5
    rows[7] = pool_rows
    seq_idx = torch.randint(0, 12, (n,), generator=g, dtype=torch.int32)
    seq_idx[5] = 99
    lens0 = torch.randint(0, 50, (12,), generator=g, dtype=torch.int32)
    kd, vd, ld = kp.to(DEV), vp.to(DEV), lens0.to(DEV)
    hp.kv_append(kn.to(DEV), vn.to(DEV), rows.to(DEV), kd, vd, ld, seq_idx.to(DEV))
    torch.cuda.synchronize()
    rk = oracle.kv_append(kp, rows.tolist(), kn)
    rv = oracle.kv_append(vp, rows.tolist(), vn)
    assert torch.equal(kd.cpu().view(torch.uint8), rk.view(torch.uint8))
    assert torch.equal(vd.cpu().view(torch.uint8), rv.view(torch.uint8))
    si, rr = seq_idx.numpy(), rows.numpy()
    written = (rr >= 0) & (rr < pool_rows)
    inc = np.bincount(si[written & (si >= 0) & (si < 12)], minlength=12)
    # every written token advances its sequence once; skipped rows advance nothing
    assert np.array_equal(ld.cpu().numpy(), lens0.numpy() + inc)


# ------------------------------------------------------ manager + append + step

def _lcp(a, b):
    n = 0
    for x, y in zip(a, b):
        if x != y:
            break
        n += 1
    return n


@pytest.mark.parametrize("dtype,Hq,Hkv,d", [("bf16", 8, 2, 128), ("f16", 4, 4, 64)])
def test_pakv_decode_scenario(dtype, Hq, Hkv, d):
    """Requests join (sharing prompt prefixes), decode for several steps (one token
    per sequence per step, appended by the kernel, lengths advanced on the device),
    and leave.  After every step each sequence's attention must match the oracle
    over that sequence's own token history."""
    g = torch.Generator().manual_seed(17)
    dt = _TD[dtype]
    num_chunks = 200
    P = hp.Pakv(num_chunks)
    kp = torch.full((num_chunks * 64, Hkv, d), float("nan"), dtype=dt, device=DEV)
    vp = torch.full_like(kp, float("nan"))
    toks, kv = {}, {}   # sid -> tokens, (K [n][Hkv][d], V) on the CPU
    system = torch.randint(0, 5, (150,), generator=g).tolist()

    def insert(sid, t):
        best = max(toks, key=lambda s: _lcp(t, toks[s]), default=None)
        rows, matched = P.insert(sid, t)
        k_new = torch.randn(len(t) - matched, Hkv, d, generator=g).to(dt)
        v_new = torch.randn(len(t) - matched, Hkv, d, generator=g).to(dt)
        if matched:
            assert best is not None and _lcp(t, toks[best]) == matched
            k = torch.cat([kv[best][0][:matched], k_new])
            v = torch.cat([kv[best][1][:matched], v_new])
        else:
            k, v = k_new, v_new
        if len(t) > matched:
            hp.kv_append(k_new.to(DEV), v_new.to(DEV),
                         torch.as_tensor(rows[matched:], dtype=torch.int32, device=DEV), kp, vp)
        toks[sid], kv[sid] = list(t), (k, v)

    for sid in range(6):
        insert(sid, system[:int(torch.randint(90, 151, (1,), generator=g))] +
               torch.randint(0, 5, (int(torch.randint(0, 80, (1,), generator=g)),),
                             generator=g).tolist())
    insert(6, torch.randint(0, 5, (70,), generator=g).tolist())  # no shared prefix

    ts = None
    lens_dev = None
    order = None
    next_sid = 7
    for step_i in range(12):
        if step_i == 4:
            P.remove(2)
            del toks[2], kv[2]
            ts = None
        if step_i == 7:
            insert(next_sid, toks[0][:120] + [9, 9, 9])
            next_sid += 1
            ts = None
        if ts is None:
            order, lens, descs = P.context()
            lens_dev = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
        # decode: one new token per sequence, its K/V written by the kernel
        rows, idx, changed_any = [], [], False
        k_new = torch.randn(len(order), Hkv, d, generator=g).to(dt)
        v_new = torch.randn(len(order), Hkv, d, generator=g).to(dt)
        for b, sid in enumerate(order.tolist()):
            tok = int(torch.randint(0, 5, (1,), generator=g))
            r, changed = P.append(sid, tok)
            changed_any |= changed
            rows.append(r)
            idx.append(b)
            toks[sid].append(tok)
            kv[sid] = (torch.cat([kv[sid][0], k_new[b:b + 1]]),
                       torch.cat([kv[sid][1], v_new[b:b + 1]]))
        hp.kv_append(k_new.to(DEV), v_new.to(DEV), torch.as_tensor(rows, dtype=torch.int32,
                     device=DEV), kp, vp, lens_dev, torch.as_tensor(idx, dtype=torch.int32,
                                                                    device=DEV))
        if ts is None or changed_any:
            o2, l2, descs = P.context()
            assert np.array_equal(o2, order)
            ts = hp.TreeStep(torch.empty(len(order), Hq, d, dtype=dt, device=DEV), Hkv, descs,
                             2, num_chunks * 64)
        torch.cuda.synchronize()
        assert lens_dev.cpu().tolist() == [len(toks[s]) for s in order.tolist()]
        q = torch.randn(len(order), Hq, d, generator=g).to(dt)
        o, l = ts(q.to(DEV), kp, vp, lens_dev)
        torch.cuda.synchronize()
        segs = [[kv[s]] for s in order.tolist()]
        ro, rl = oracle.attention(q, segs, Hkv, workloads.scale_for(d))
        say(f"  step {step_i}: B={len(order)} segs={ts.plan.num_segs} "
            f"private rows={ts.plan.num_tok_rows}")
        compare(o, l, ro, rl, dtype, f"pakv step {step_i}")
        if step_i == 9:
            P.remove(order.tolist()[0])
            del toks[order.tolist()[0]], kv[order.tolist()[0]]
            ts = None
    st = P.stats()
    say(f"  chunks used {st.chunks_used} free {st.chunks_free} stored {st.tokens_stored} "
        f"logical {st.tokens_logical}")
    assert st.tokens_stored < st.tokens_logical
