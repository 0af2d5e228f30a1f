"""Helpers for the GPU parity tests: device copies of generated steps and the
tolerance checks stated for this path."""
from __future__ import annotations

import sys

import numpy as np
import torch

import decode_attention_shared_amd as hp
import workloads

DEV = "cuda:0"

# fp32 inputs: max-abs 1e-5 on O (and on LSE).  16-bit inputs: max-abs 1e-2 and
# mean-abs 1e-3 on O, max-abs 1e-3 on LSE.
TOL = {"f32": dict(max_abs=1e-5, mean_abs=1e-5, lse=1e-5),
       "f16": dict(max_abs=1e-2, mean_abs=1e-3, lse=1e-3),
       "bf16": dict(max_abs=1e-2, mean_abs=1e-3, lse=1e-3)}


# Every compare() appends (what, dtype, max-abs, mean-abs, LSE max-abs, rel-L2); the
# test session prints them at its end (conftest.py), so the margins against the
# tolerances stay in the output of a quiet run.
MARGINS = []


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_step(step, dev=DEV, kv_layout="NHD"):
    """Copy a workloads.Step to the GPU: q, tree levels, paged pool (in kv_layout)."""
    levels = [[(n.k.to(dev), n.v.to(dev), n.seq_begin, n.seq_end) for n in lvl]
              for lvl in step.levels]
    return dict(q=step.q.to(dev), levels=levels,
                k_pool=workloads.pool_in_layout(step.k_pool, kv_layout).to(dev),
                v_pool=workloads.pool_in_layout(step.v_pool, kv_layout).to(dev),
                block_table=step.block_table.to(dev), seq_lens=step.seq_lens.to(dev),
                kv_layout=kv_layout)


def cascade(ds, scale, levels=None, paged=True, share_min=0):
    """share_min 0: the library's batching policy picks the nodes the prefix pass reads
    (the rest are read by each sequence in the suffix pass); 1: every node batched."""
    lv = ds["levels"] if levels is None else levels
    if paged:
        return hp.cascade_step(ds["q"], lv, ds["k_pool"], ds["v_pool"], ds["block_table"],
                               ds["seq_lens"], scale, share_min=share_min,
                               kv_layout=ds["kv_layout"])
    return hp.cascade_step(ds["q"], lv, scale=scale, share_min=share_min)


def compare(got_o, got_l, ref_o, ref_l, dtype: str, what: str, rows=None):
    """got_*: torch (any shape, rows-major) ; ref_*: numpy [n][d] / [n]."""
    go = got_o.detach().double().cpu().numpy().reshape(-1, ref_o.shape[-1])
    gl = got_l.detach().double().cpu().numpy().reshape(-1)
    if rows is not None:
        go = go[rows]
        gl = gl[rows]
    assert go.shape == ref_o.shape, (go.shape, ref_o.shape)
    tol = TOL[dtype]
    assert np.isfinite(go).all(), f"{what}: non-finite output"
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(gl), fin), f"{what}: LSE finiteness differs"
    assert np.array_equal(gl[~fin], ref_l[~fin]), f"{what}: LSE of empty rows differs"
    err = np.abs(go - ref_o)
    lerr = np.abs(gl[fin] - ref_l[fin]) if fin.any() else np.zeros(1)
    rel_l2 = float(np.linalg.norm(go - ref_o) / max(1e-300, np.linalg.norm(ref_o)))
    say(f"  {what}: max-abs {err.max():.3e} mean-abs {err.mean():.3e} "
        f"lse-max {lerr.max():.3e} rel-l2 {rel_l2:.3e}")
    MARGINS.append((what, dtype, float(err.max()), float(err.mean()), float(lerr.max()), rel_l2,
                    go.shape[0]))
    assert err.max() <= tol["max_abs"], f"{what}: max-abs {err.max():.3e} > {tol['max_abs']}"
    assert err.mean() <= tol["mean_abs"], f"{what}: mean-abs {err.mean():.3e} > {tol['mean_abs']}"
    assert lerr.max() <= tol["lse"], f"{what}: LSE max-abs {lerr.max():.3e} > {tol['lse']}"
    return err.max(), lerr.max()


def sample_rows(B: int, Hq: int, n: int, seed: int = 0) -> np.ndarray:
    """n distinct rows b*Hq + h spread over the batch, always including the first and
    last sequence and head."""
    rng = np.random.default_rng(seed)
    total = B * Hq
    pick = set([0, total - 1, Hq - 1, (B - 1) * Hq])
    while len(pick) < min(n, total):
        pick.add(int(rng.integers(0, total)))
    return np.array(sorted(pick), dtype=np.int64)
