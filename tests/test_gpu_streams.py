"""GPU parity of shared-context stream decode (hp_stream_decode) against the fp64 oracle.

Each query is one stream of a request; it attends its document (prefix nodes) and the
positions of its request's KV row whose stream id is -1 or its own ("Read Once, Answer
Many: Parallel Prompting for Shared-Context LLM Inference", section "Parallel
Prompting", Eq. 2).  Tolerances as for the cascade (gpu_util.TOL); the gather of
visible rows is checked bit-exactly with needles.
"""
import numpy as np
import pytest
import torch

import decode_attention_shared_amd as hp
import oracle
import workloads
from gpu_util import DEV, compare, say

pytestmark = pytest.mark.gpu

NEG = -16384.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X (no GPU visible)")
    hp.lib()


def dev(step):
    levels = [[(n.k.to(DEV), n.v.to(DEV), n.seq_begin, n.seq_end) for n in lvl]
              for lvl in step.levels]
    return dict(q=step.q.to(DEV), levels=levels, k_pool=step.k_pool.to(DEV),
                v_pool=step.v_pool.to(DEV), row_slots=step.row_slots.to(DEV),
                slot_sid=step.row_sid.to(DEV), row_len=step.row_len.to(DEV),
                q_req=step.q_req.to(DEV), q_sid=step.q_sid.to(DEV))


def call_of(ds, scale, levels=None, overlap=1):
    return hp.StreamCall(ds["q"], ds["levels"] if levels is None else levels, ds["k_pool"],
                         ds["v_pool"], ds["row_slots"], ds["slot_sid"], ds["row_len"],
                         ds["q_req"], ds["q_sid"], scale, overlap=overlap)


# 0: the serial step (document partials merged in the stream pass's epilogue); 2: the
# stream pass on a second stream beside the document's prefix pass, then one merge
MODES = [0, 2]


CASES = [
    # name, dtype, d, B, Hq, Hkv, doc levels, own lo..hi, P, answer, shared
    ("mha_bf16", "bf16", 128, 20, 8, 8, (((300, 0, 20),),), 3, 90, 6, 3, 2),
    ("gqa_f16", "f16", 128, 17, 32, 8, (((1000, 0, 17),),), 1, 260, 4, 1, 0),
    ("d64_f32", "f32", 64, 9, 2, 1, (((129, 0, 9),),), 0, 40, 3, 0, 1),
    ("one_stream_per_request", "bf16", 64, 7, 4, 2, (((65, 0, 7),),), 2, 33, 1, 2, 0),
    ("two_docs", "bf16", 128, 24, 8, 2, (((200, 0, 12), (150, 12, 24)),), 4, 70, 8, 4, 1),
    ("long_rows", "bf16", 128, 12, 4, 4, (((64, 0, 12),),), 300, 520, 12, 16, 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("mode", MODES)
def test_stream_decode_reduced(case, seed, mode):
    name, dtype, d, B, Hq, Hkv, levels, lo, hi, P, ans, shared = case
    say(f"streams {name} seed {seed} mode {mode}")
    cfg = workloads.custom(name, B=B, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, levels=levels,
                           suffix_lo=lo, suffix_hi=hi)
    step = workloads.stream_step(cfg, P=P, seed=seed, answer_len=ans, shared_len=shared)
    ds = dev(step)
    call = call_of(ds, step.scale, overlap=mode)
    assert call.concurrent == (mode == 2)
    out, lse = call()
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.stream_attention(step)
    compare(out, lse, ref_o, ref_l, dtype, name)


def test_stream_decode_without_document_and_empty_streams():
    cfg = workloads.custom("nodoc", B=10, Hq=4, Hkv=2, d=128, dtype="bf16",
                           levels=(((1, 0, 10),),), suffix_lo=0, suffix_hi=9)
    step = workloads.stream_step(cfg, P=5, seed=3, answer_len=0, shared_len=0)
    step.levels = []                       # no document: only the row tokens
    ds = dev(step)
    call = call_of(ds, step.scale, levels=[], overlap=2)
    assert not call.concurrent  # no document: nothing runs beside the stream pass
    out, lse = call()
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.stream_attention(step)
    compare(out, lse, ref_o, ref_l, "bf16", "no document")
    empty = [b for b in range(cfg.B) if int(step.own_lens[b]) == 0]
    for b in empty:
        assert torch.all(out[b] == 0) and torch.all(lse[b] == -float("inf"))


@pytest.mark.parametrize("mode", MODES)
def test_stream_decode_bad_metadata_gives_nan_rows_only(mode):
    cfg = workloads.custom("bad", B=16, Hq=8, Hkv=2, d=128, dtype="f16",
                           levels=(((100, 0, 16),),), suffix_lo=2, suffix_hi=30)
    step = workloads.stream_step(cfg, P=4, seed=4, answer_len=2)
    ds = dev(step)
    ds["q_req"][1] = step.R                     # request out of range
    ds["q_req"][2] = -1
    ds["row_len"][3] = step.row_cap + 1         # request 3 (queries 12..15): longer than its row
    r0 = int(step.q_req[5])
    vis = oracle.visible_positions(step.row_sid[r0, :int(step.row_len[r0])].tolist(),
                                   int(step.q_sid[5]))
    ds["row_slots"][r0, int(vis[-1])] = step.k_pool.shape[0]   # a visible slot past the pool
    out, lse = call_of(ds, step.scale, overlap=mode)()
    torch.cuda.synchronize()
    bad = [1, 2, 5, 12, 13, 14, 15]
    assert torch.isnan(out[bad]).all() and torch.isnan(lse[bad]).all()
    good = [b for b in range(cfg.B) if b not in bad]
    rows = np.array([b * cfg.Hq + h for b in good for h in range(cfg.Hq)])
    ref_o, ref_l = oracle.stream_attention(step, rows=rows)
    compare(out, lse, ref_o, ref_l, "f16", "good rows", rows=rows)


def test_stream_needles_every_visible_position():
    """Every visible key of every stream, one at a time: O must be that key's value row
    exactly (a wrong gather, order or mask picks another row)."""
    cfg = workloads.custom("needle_streams", B=12, Hq=4, Hkv=2, d=128, dtype="bf16",
                           levels=(((90, 0, 12),),), suffix_lo=2, suffix_hi=40)
    step = workloads.stream_step(cfg, P=4, seed=5, answer_len=2, shared_len=3)
    ds = dev(step)
    ds["q"].zero_()
    ds["q"][:, :, 0] = 1.0
    for lvl in ds["levels"]:
        for (k, v, _, _) in lvl:
            k[:, :, 0] = NEG
    ds["k_pool"][:, :, 0] = NEG
    call = call_of(ds, step.scale)
    vis = []
    for b in range(cfg.B):
        r = int(step.q_req[b])
        vis.append(oracle.visible_positions(step.row_sid[r, :int(step.row_len[r])].tolist(),
                                            int(step.q_sid[b])))
    runs = max(len(v) for v in vis)
    G = cfg.G
    for run in range(runs):
        # one needle per (request, KV head): streams of a request share their shared
        # positions, so only the first stream of each request places its needle there
        slots, heads, want = [], [], torch.zeros(cfg.B, cfg.Hq, cfg.d)
        placed = {}
        for b in range(cfg.B):
            r = int(step.q_req[b])
            for g in range(cfg.Hkv):
                pos = int(vis[b][(run + g) % len(vis[b])])
                key = (r, pos, g)
                slot = int(step.row_slots[r, pos])
                if key not in placed:
                    placed[key] = slot
                    slots.append(slot)
                    heads.append(g)
        idx = (torch.tensor(slots, device=DEV), torch.tensor(heads, device=DEV))
        ds["k_pool"][idx + (0,)] = 0.0
        out, lse = call()
        got = out.cpu()
        for b in range(cfg.B):
            r = int(step.q_req[b])
            for h in range(cfg.Hq):
                g = h // G
                # the stream's visible needles of head g: its own pick, plus any shared
                # position another stream of the request picked in this run
                hits = [p for p in vis[b].tolist() if (r, p, g) in placed]
                if len(hits) == 1:
                    assert torch.equal(got[b, h], step.row_v[r][hits[0], g].float()), \
                        f"run {run} stream {b} head {h}: wrong key"
                    assert float(lse[b, h]) == 0.0
                else:   # several needles visible: exact equal-weight mean, LSE = ln n
                    want = torch.stack([step.row_v[r][p, g].double() for p in hits]).mean(0)
                    assert torch.allclose(got[b, h].double(), want, atol=1e-2)
        ds["k_pool"][idx + (0,)] = NEG
    say(f"  stream needles: {runs} runs cover every visible position of every stream")


@pytest.mark.parametrize("mode", MODES)
def test_stream_decode_deterministic_and_graph_replay(mode):
    """Eager calls agree bit for bit; every replay of a captured step equals them, with
    eager work (a fill) between replays."""
    cfg = workloads.custom("graph", B=16, Hq=8, Hkv=8, d=128, dtype="bf16",
                           levels=(((500, 0, 16),),), suffix_lo=8, suffix_hi=100)
    step = workloads.stream_step(cfg, P=8, seed=6, answer_len=4)
    ds = dev(step)
    call = call_of(ds, step.scale, overlap=mode)
    assert call.concurrent == (mode == 2)
    o1, l1 = [t.clone() for t in call()]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call(stream=s)
        torch.cuda.synchronize()
        g.capture_begin()
        call(stream=s)
        g.capture_end()
    for _ in range(3):
        call.out.fill_(5.0)
        call.lse.fill_(5.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.out, o1) and torch.equal(call.lse, l1)
    ref_o, ref_l = oracle.stream_attention(step)
    compare(call.out, call.lse, ref_o, ref_l, "bf16", f"graph replay, mode {mode}")


def test_stream_decode_full_size_every_row():
    """The full-size step (16K-token document, 256 streams in requests of 32) in both of
    the plans the default policy can pick, serial and side by side (the one bench.py
    times): every row against one oracle pass."""
    cfg = workloads.docqa_streams(32)
    say(f"full {cfg.name}: generating")
    step = workloads.stream_step(cfg, P=32, seed=0)
    ds = dev(step)
    outs = {}
    for mode in (0, 1):
        call = call_of(ds, step.scale, overlap=mode)
        assert call.concurrent == (mode == 1)
        out, lse = call()
        torch.cuda.synchronize()
        outs[mode] = (out.clone(), lse.clone())
    say(f"full {cfg.name}: oracle over {cfg.B * cfg.Hq} rows")
    ref_o, ref_l = oracle.stream_attention(step)
    for mode, (out, lse) in outs.items():
        compare(out, lse, ref_o, ref_l, cfg.dtype, f"{cfg.name} mode {mode} (all rows)")
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()


def _small_stream_step(seed):
    cfg = workloads.custom("side", B=24, Hq=8, Hkv=4, d=128, dtype="bf16",
                           levels=(((700, 0, 24),),), suffix_lo=8, suffix_hi=120)
    return cfg, workloads.stream_step(cfg, P=6, seed=seed, answer_len=3)


def test_stream_side_by_side_orders_with_caller_stream():
    """Side by side: a change of q enqueued on the caller's stream right before the step
    is seen by both passes, and a copy enqueued right after it sees the merged result."""
    cfg, step = _small_stream_step(31)
    ds = dev(step)
    call = call_of(ds, step.scale, overlap=2)
    assert call.concurrent
    s = torch.cuda.Stream()
    q0 = step.q.clone()
    with torch.cuda.stream(s):
        for rep in range(3):
            q_rep = (q0.float() * (1.0 + 0.5 * rep)).to(q0.dtype)
            ds["q"].copy_(q_rep.to(DEV), non_blocking=True)
            call(stream=s)
            got_o, got_l = call.out.clone(), call.lse.clone()  # ordered after the merge on s
            call.out.fill_(5.0)                                 # and before the next step
            s.synchronize()
            step.q = q_rep
            ref_o, ref_l = oracle.stream_attention(step)
            compare(got_o, got_l, ref_o, ref_l, "bf16", f"stream ordered step {rep}")
    step.q = q0


def test_stream_side_by_side_first_call_captured():
    """The very first call of a side-by-side stream step may be the one captured into a
    graph: every replay equals a separate eager step on the same inputs."""
    cfg, step = _small_stream_step(33)
    ds = dev(step)
    ref_call = call_of(ds, step.scale, overlap=2)
    eager_o, eager_l = [t.clone() for t in ref_call()]
    torch.cuda.synchronize()
    call = call_of(ds, step.scale, overlap=2)
    assert call.concurrent
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        g.capture_begin()
        call(stream=s)
        g.capture_end()
    for rep in range(4):
        call.out.fill_(3.0)
        call.lse.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.out, eager_o) and torch.equal(call.lse, eager_l), f"replay {rep}"
        ref_call()  # eager work between replays
        torch.cuda.synchronize()
    ref_o, ref_l = oracle.stream_attention(step)
    compare(call.out, call.lse, ref_o, ref_l, "bf16", "stream first call captured")
