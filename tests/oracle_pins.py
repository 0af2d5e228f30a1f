"""Pins of the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load(path)``)
and raises AssertionError when that build disagrees with:
  * a high-precision brute force of the plain definition (mpmath, 60 digits,
    no max shift), on tiny inputs in every storage type;
  * closed forms (one key, two keys, uniform scores);
  * invariances the mathematics fixes (key permutation, value shift and
    scale, query/scale trade, a constant added to every score);
  * the split/merge identity of the Hydragen page ("Attention Decomposition
    Across Subsequences", Eq. 5), at the size and magnitude the "Shared Prefix
    KV Caching, in depth" page reports for its own float64 check (golden
    fixture ``golden/split_merge_fp64.json``);
  * which keys a sequence of a generated step attends, rebuilt from the
    config's node ranges alone (a node (len, i, j) serves sequences i .. j-1:
    the ChunkAttention page's (C, i, j) descriptor, section "Context
    Generation and GPU-CPU Coordination"; every node on the sequence's path,
    root first: the Hydragen page, section "Hierarchical Sharing") and
    evaluated by a dense numpy softmax;
  * a subset of rows computed alone equals those rows of the full result.
Run against the real build by test_oracle_pins.py, and against builds with
planted mistakes by test_oracle_mutants.py.
"""
from __future__ import annotations

import json
import math
import os

import mpmath
import numpy as np
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
mpmath.mp.dps = 60


def _rand(shape, dtype, gen, mult=1.0):
    return (torch.randn(*shape, generator=gen, dtype=torch.float64) * mult).to(dtype)


def _brute(q, segs_per_seq, Hkv, scale):
    """Plain definition in 60-digit arithmetic: O = sum e^{s_j} v_j / sum e^{s_j},
    LSE = ln sum e^{s_j}, s_j = scale * q.k_j, KV head of query head h = h // (Hq/Hkv)."""
    B, Hq, d = q.shape
    G = Hq // Hkv
    qd = q.double()
    out_o = np.zeros((B * Hq, d))
    out_l = np.zeros(B * Hq)
    sc = mpmath.mpf(float(np.float32(scale)))
    for b in range(B):
        ks = [k.double() for (k, _) in segs_per_seq[b]]
        vs = [v.double() for (_, v) in segs_per_seq[b]]
        for h in range(Hq):
            g = h // G
            qv = [mpmath.mpf(float(x)) for x in qd[b, h]]
            num = [mpmath.mpf(0)] * d
            den = mpmath.mpf(0)
            for K, V in zip(ks, vs):
                for t in range(K.shape[0]):
                    s = sc * mpmath.fsum(qv[c] * mpmath.mpf(float(K[t, g, c])) for c in range(d))
                    e = mpmath.exp(s)
                    den += e
                    for c in range(d):
                        num[c] += e * mpmath.mpf(float(V[t, g, c]))
            r = b * Hq + h
            if den == 0:
                out_l[r] = -math.inf
                continue
            for c in range(d):
                out_o[r, c] = float(num[c] / den)
            out_l[r] = float(mpmath.log(den))
    return out_o, out_l


def _close(a, b, rel=1e-14, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: non-finite values differ"
    err = np.abs(a[fin] - b[fin]) / np.maximum(1.0, np.abs(b[fin]))
    assert err.size == 0 or err.max() <= rel, f"{what}: rel err {err.max():.3e} > {rel:.1e}"


def _tiny_problem(dtype, gen, d=8, Hq=4, Hkv=2, B=2, plen=5, mult=1.0, vmult=1.0):
    q = _rand((B, Hq, d), dtype, gen, mult)
    kp = _rand((plen, Hkv, d), dtype, gen)
    vp = _rand((plen, Hkv, d), dtype, gen, vmult)
    segs = []
    for b in range(B):
        n = b + 2
        ks = _rand((n, Hkv, d), dtype, gen)
        vs = _rand((n, Hkv, d), dtype, gen, vmult)
        segs.append([(kp, vp), (ks, vs)])
    return q, segs


def pin_brute_force(lib):
    """All storage types, GQA mapping, two segments per sequence, shared prefix."""
    gen = torch.Generator().manual_seed(11)
    for dtype in (torch.float32, torch.float16, torch.bfloat16):
        for d, Hq, Hkv in ((8, 4, 2), (3, 2, 1), (5, 3, 3)):
            q, segs = _tiny_problem(dtype, gen, d=d, Hq=Hq, Hkv=Hkv)
            scale = workloads.scale_for(d)
            o, l = oracle.attention(q, segs, Hkv, scale, lib=lib)
            bo, bl = _brute(q, segs, Hkv, scale)
            _close(o, bo, 1e-14, f"O {dtype} d={d}")
            _close(l, bl, 1e-14, f"LSE {dtype} d={d}")


def pin_brute_force_extreme_values(lib):
    """fp16 subnormal and large values, bf16 large exponents, and scores of several
    hundred (exp of them overflows double without a max shift)."""
    gen = torch.Generator().manual_seed(12)
    q, segs = _tiny_problem(torch.float16, gen, d=4, Hq=2, Hkv=1, vmult=1e-6)
    o, l = oracle.attention(q, segs, 1, 0.5, lib=lib)
    bo, bl = _brute(q, segs, 1, 0.5)
    _close(o, bo, 1e-14, "fp16 subnormal V")
    _close(l, bl, 1e-14, "fp16 subnormal V lse")
    q, segs = _tiny_problem(torch.float16, gen, d=4, Hq=2, Hkv=1, mult=3000.0)
    o, l = oracle.attention(q, segs, 1, 0.25, lib=lib)
    bo, bl = _brute(q, segs, 1, 0.25)
    _close(o, bo, 1e-14, "fp16 large Q")
    _close(l, bl, 1e-14, "fp16 large Q lse")
    assert np.abs(bl).max() > 720, "the case must reach scores that overflow exp in double"
    q, segs = _tiny_problem(torch.bfloat16, gen, d=4, Hq=2, Hkv=2, mult=1e3, vmult=1e20)
    o, l = oracle.attention(q, segs, 2, 0.5, lib=lib)
    bo, bl = _brute(q, segs, 2, 0.5)
    _close(o / 1e20, bo / 1e20, 1e-14, "bf16 wide range")
    _close(l, bl, 1e-14, "bf16 wide range lse")


def pin_closed_forms(lib):
    gen = torch.Generator().manual_seed(13)
    d = 16
    scale = workloads.scale_for(d)
    # one key: O = v exactly, LSE = s
    q = _rand((1, 1, d), torch.float32, gen)
    k = _rand((1, 1, d), torch.float32, gen)
    v = _rand((1, 1, d), torch.float32, gen)
    o, l = oracle.attention(q, [[(k, v)]], 1, scale, lib=lib)
    assert np.array_equal(o[0], v[0, 0].double().numpy()), "one key: O must equal v exactly"
    s = float(np.float32(scale)) * float(np.dot(q[0, 0].double().numpy(), k[0, 0].double().numpy()))
    _close(l, [s], 1e-14, "one key LSE")
    # two keys: O = sigma(s1-s2) v1 + sigma(s2-s1) v2, LSE = logaddexp(s1, s2)
    k = _rand((2, 1, d), torch.float32, gen)
    v = _rand((2, 1, d), torch.float32, gen)
    o, l = oracle.attention(q, [[(k, v)]], 1, scale, lib=lib)
    qq = q[0, 0].double().numpy()
    s1, s2 = [float(np.float32(scale)) * float(np.dot(qq, k[i, 0].double().numpy())) for i in (0, 1)]
    sig = 1.0 / (1.0 + math.exp(-(s1 - s2)))
    want = sig * v[0, 0].double().numpy() + (1.0 - sig) * v[1, 0].double().numpy()
    _close(o[0], want, 1e-14, "two keys O")
    _close(l, [np.logaddexp(s1, s2)], 1e-14, "two keys LSE")
    # zero query: uniform scores -> O = mean of V, LSE = ln n
    n = 37
    q0 = torch.zeros(1, 1, d)
    k = _rand((n, 1, d), torch.float32, gen)
    v = _rand((n, 1, d), torch.float32, gen)
    o, l = oracle.attention(q0, [[(k[:20], v[:20]), (k[20:], v[20:])]], 1, scale, lib=lib)
    _close(o[0], v[:, 0].double().mean(0).numpy(), 1e-14, "uniform O")
    _close(l, [math.log(n)], 1e-14, "uniform LSE")
    # no keys: O = 0, LSE = -inf
    o, l = oracle.attention(q0, [[]], 1, scale, lib=lib)
    assert np.array_equal(o, np.zeros((1, d))) and l[0] == -math.inf, "empty key list"


def pin_invariances(lib):
    gen = torch.Generator().manual_seed(14)
    d, Hq, Hkv, n = 32, 4, 2, 50
    scale = workloads.scale_for(d)
    q = _rand((1, Hq, d), torch.float32, gen)
    k = _rand((n, Hkv, d), torch.float32, gen)
    # values on a 2^-10 grid so that the shifted values below are stored exactly
    v = torch.round(_rand((n, Hkv, d), torch.float32, gen) * 1024) / 1024
    o, l = oracle.attention(q, [[(k, v)]], Hkv, scale, lib=lib)
    # key permutation, across a different segment split
    perm = torch.randperm(n, generator=gen)
    kp, vp = k[perm], v[perm]
    o2, l2 = oracle.attention(q, [[(kp[:7], vp[:7]), (kp[7:], vp[7:])]], Hkv, scale, lib=lib)
    _close(o2, o, 1e-14, "permutation O")
    _close(l2, l, 1e-14, "permutation LSE")
    # V + c -> O + c; 2V -> 2O exactly
    o3, _ = oracle.attention(q, [[(k, v + 0.75)]], Hkv, scale, lib=lib)
    _close(o3, o + 0.75, 1e-14, "value shift")
    o4, l4 = oracle.attention(q, [[(k, v * 2)]], Hkv, scale, lib=lib)
    assert np.array_equal(o4, 2 * o) and np.array_equal(l4, l), "value scale"
    # (2q, scale/2): identical scores
    o5, l5 = oracle.attention(q * 2, [[(k, v)]], Hkv, scale / 2, lib=lib)
    assert np.array_equal(o5, o) and np.array_equal(l5, l), "query/scale trade"
    # a constant added to every score: O unchanged, LSE shifted by it
    ke = torch.cat([k, torch.ones(n, Hkv, 1)], dim=2)
    ve = torch.cat([v, torch.zeros(n, Hkv, 1)], dim=2)
    c = 3.0
    qe = torch.cat([q, torch.full((1, Hq, 1), c)], dim=2)
    qz = torch.cat([q, torch.zeros(1, Hq, 1)], dim=2)
    oa, la = oracle.attention(qe, [[(ke, ve)]], Hkv, scale, lib=lib)
    ob, lb = oracle.attention(qz, [[(ke, ve)]], Hkv, scale, lib=lib)
    _close(oa, ob, 1e-13, "score shift O")
    _close(la - lb, np.full(Hq, float(np.float32(scale)) * c), 1e-13, "score shift LSE")


def pin_split_merge_identity(lib):
    """Eq. 5 of the Hydragen page: attention over prefix || suffix equals the merge of
    the two parts; fixture sizes and magnitude from the blog page's float64 check."""
    with open(os.path.join(GOLDEN, "split_merge_fp64.json")) as f:
        gold = json.load(f)
    d, P, B, S = gold["d"], gold["P"], gold["B"], gold["S"]
    gen = torch.Generator().manual_seed(15)
    q = _rand((B, 1, d), torch.float32, gen)
    kp, vp = _rand((P, 1, d), torch.float32, gen), _rand((P, 1, d), torch.float32, gen)
    ks, vs = _rand((B * S, 1, d), torch.float32, gen), _rand((B * S, 1, d), torch.float32, gen)
    scale = workloads.scale_for(d)
    suf = [(ks[b * S:(b + 1) * S], vs[b * S:(b + 1) * S]) for b in range(B)]
    o_all, l_all = oracle.attention(q, [[(kp, vp), suf[b]] for b in range(B)], 1, scale, lib=lib)
    o_a, l_a = oracle.attention(q, [[(kp, vp)] for b in range(B)], 1, scale, lib=lib)
    o_b, l_b = oracle.attention(q, [[suf[b]] for b in range(B)], 1, scale, lib=lib)
    o_m, l_m = oracle.merge([o_a, o_b], [l_a, l_b], lib=lib)
    err = np.abs(o_m - o_all).max()
    assert err <= gold["bound"], f"split/merge max-abs {err:.3e} > {gold['bound']}"
    assert np.abs(l_m - l_all).max() <= gold["bound"] * 10, "split/merge LSE"
    # three parts (global, group, suffix), any grouping
    o_c, l_c = oracle.attention(q, [[(kp[:200], vp[:200])] for b in range(B)], 1, scale, lib=lib)
    o_d, l_d = oracle.attention(q, [[(kp[200:], vp[200:])] for b in range(B)], 1, scale, lib=lib)
    o_3, l_3 = oracle.merge([o_c, o_d, o_b], [l_c, l_d, l_b], lib=lib)
    _close(o_3, o_all, 1e-14, "three-way merge O")
    _close(l_3, l_all, 1e-14, "three-way merge LSE")


def pin_merge_edges(lib):
    gen = torch.Generator().manual_seed(16)
    rows, d = 5, 8
    o1 = torch.randn(rows, d, generator=gen, dtype=torch.float64).numpy()
    l1 = torch.randn(rows, generator=gen, dtype=torch.float64).numpy()
    empty_o = np.zeros((rows, d))
    empty_l = np.full(rows, -math.inf)
    for parts in ([o1, empty_o], [empty_o, o1]):
        ls = [l1, empty_l] if parts[0] is o1 else [empty_l, l1]
        om, lm = oracle.merge(parts, ls, lib=lib)
        assert np.array_equal(om, o1) and np.array_equal(lm, l1), "merge with an empty part"
    om, lm = oracle.merge([empty_o, empty_o], [empty_l, empty_l], lib=lib)
    assert np.array_equal(om, empty_o) and np.all(lm == -math.inf), "merge of empty parts"
    # two equal parts: O unchanged, LSE + ln 2
    om, lm = oracle.merge([o1, o1], [l1, l1], lib=lib)
    _close(om, o1, 1e-15, "equal parts O")
    _close(lm, l1 + math.log(2.0), 1e-15, "equal parts LSE")


def pin_workload_step(lib):
    """Oracle over a generated step reads the logical arrays: its whole-step result equals
    the merge of its prefix-only and suffix-only results (two-level tree included)."""
    cfg = workloads.custom("pin_tree", B=6, Hq=4, Hkv=2, d=16, dtype="bf16",
                           levels=(((40, 0, 6),), ((9, 0, 2), (13, 3, 6))),
                           suffix_lo=1, suffix_hi=20)
    step = workloads.generate(cfg, seed=3)
    o, l = oracle.step_attention(step, "all", lib=lib)
    parts = [oracle.step_attention(step, ("level", 0), lib=lib),
             oracle.step_attention(step, ("level", 1), lib=lib),
             oracle.step_attention(step, "suffix", lib=lib)]
    om, lm = oracle.merge([p[0] for p in parts], [p[1] for p in parts], lib=lib)
    _close(om, o, 1e-14, "tree merge O")
    _close(lm, l, 1e-14, "tree merge LSE")
    bo, bl = _brute(step.q, oracle.step_segments(step, "all"), cfg.Hkv, step.scale)
    _close(o, bo, 1e-14, "tree brute O")
    _close(l, bl, 1e-14, "tree brute LSE")


def _dense_rows(q, keys_per_seq, Hkv, scale):
    """Softmax attention of every (b, h) row by whole-array numpy fp64 operations
    (scores as one matrix-vector product, logsumexp by numpy), a second
    implementation of the definition independent of oracle.c."""
    B, Hq, d = q.shape
    G = Hq // Hkv
    o = np.zeros((B * Hq, d))
    l = np.full(B * Hq, -math.inf)
    sc = float(np.float32(scale))
    for b in range(B):
        if not keys_per_seq[b]:
            continue
        K = np.concatenate([k.double().numpy() for (k, _) in keys_per_seq[b]], axis=0)
        V = np.concatenate([v.double().numpy() for (_, v) in keys_per_seq[b]], axis=0)
        for h in range(Hq):
            s = sc * (K[:, h // G, :] @ q[b, h].double().numpy())
            w = np.exp(s - s.max())
            o[b * Hq + h] = (w @ V[:, h // G, :]) / w.sum()
            l[b * Hq + h] = np.logaddexp.reduce(s)
    return o, l


def pin_workload_keys(lib):
    """The keys a generated step's sequence attends, rebuilt from the config alone:
    node (len, i, j) of a level serves sequences i .. j-1 (half-open, the (C, i, j)
    descriptor of the ChunkAttention page), root level first, then the sequence's
    own suffix.  The tree has sequences at both ends of a group's range and one
    sequence under no group node, so a node range read one past either end, or a
    level skipped, changes some row."""
    cfg = workloads.custom("pin_keys", B=7, Hq=4, Hkv=2, d=16, dtype="f32",
                           levels=(((30, 0, 7),), ((11, 0, 2), (9, 3, 5), (14, 5, 7))),
                           suffix_lo=1, suffix_hi=12)
    step = workloads.generate(cfg, seed=5)
    keys = [[] for _ in range(cfg.B)]
    for li, level in enumerate(cfg.levels):
        for ni, (ln, i, j) in enumerate(level):
            node = step.levels[li][ni]
            assert node.k.shape[0] == ln, "generated node length differs from the config"
            for b in range(i, j):
                keys[b].append((node.k, node.v))
    for b in range(cfg.B):
        keys[b].append(step.suffix(b))
    assert sum(1 for b in range(cfg.B) if len(keys[b]) == 2) == 1, "one sequence under no group"
    want_o, want_l = _dense_rows(step.q, keys, cfg.Hkv, step.scale)
    o, l = oracle.step_attention(step, "all", lib=lib)
    _close(o, want_o, 1e-12, "step keys O")
    _close(l, want_l, 1e-12, "step keys LSE")
    # the prefix-only view attends the same nodes and nothing else
    pre = [ks[:-1] for ks in keys]
    want_o, want_l = _dense_rows(step.q, pre, cfg.Hkv, step.scale)
    o, l = oracle.step_attention(step, "prefix", lib=lib)
    _close(o, want_o, 1e-12, "prefix keys O")
    _close(l, want_l, 1e-12, "prefix keys LSE")


def pin_rows_subset(lib):
    """Rows computed on their own (the rows= path, in any order, repeats allowed)
    are bit-identical to the same rows of the full result."""
    gen = torch.Generator().manual_seed(17)
    q, segs = _tiny_problem(torch.bfloat16, gen, d=8, Hq=4, Hkv=2, B=5, plen=9)
    scale = workloads.scale_for(8)
    o, l = oracle.attention(q, segs, 2, scale, lib=lib)
    rows = [17, 3, 3, 0, 11, 19, 8]
    os_, ls_ = oracle.attention(q, segs, 2, scale, rows=rows, lib=lib)
    assert os_.shape == (len(rows), 8) and ls_.shape == (len(rows),), "subset shapes"
    for i, r in enumerate(rows):
        assert np.array_equal(os_[i], o[r]) and ls_[i] == l[r], f"subset row {i} (row {r})"


ALL_PINS = [pin_brute_force, pin_brute_force_extreme_values, pin_closed_forms, pin_invariances,
            pin_split_merge_identity, pin_merge_edges, pin_workload_step, pin_workload_keys,
            pin_rows_subset]
