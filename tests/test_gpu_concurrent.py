"""GPU parity of the cascade step when its suffix pass runs beside its prefix pass
(hp_cascade_step_overlap: on a second stream that the caller owns, forked from and
joined to the caller's stream with the caller's events), forced on (mode 2) for shapes
the automatic policy would run serially: results against the fp64 oracle (tolerances
in gpu_util.TOL), NaN rows for bad metadata, ordering with work the caller enqueues just
before and after the step, graph capture (also of a step's very first call), and the
timed entry point.  The full-size MHA and document steps, which the automatic policy
runs this way, are covered by test_cascade_full_size_every_row."""
import ctypes

import numpy as np
import pytest
import torch

import decode_attention_shared_amd as hp
import oracle
import workloads
from gpu_util import DEV, compare, dev_step, say
from test_gpu_parity import REDUCED

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X (no GPU visible)")


def _call(ds, scale, share_min=1):
    call = hp.CascadeCall(ds["q"], ds["levels"], ds["k_pool"], ds["v_pool"], ds["block_table"],
                          ds["seq_lens"], scale, overlap=2, share_min=share_min)
    assert call.concurrent, "forced mode must run the passes side by side"
    return call


@pytest.mark.parametrize("cfg", REDUCED, ids=lambda c: c.name)
def test_concurrent_matches_oracle(cfg):
    say(f"concurrent cascade {cfg.name}")
    step = workloads.generate(cfg, seed=3)
    ds = dev_step(step)
    out, lse = _call(ds, step.scale)()
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.step_attention(step, "all")
    compare(out, lse, ref_o, ref_l, cfg.dtype, f"concurrent {cfg.name}")


def test_concurrent_with_private_nodes():
    """The batching policy on the two-level shape: the root (700 tokens, 24 sequences) is
    batched, the group nodes (300 tokens, 8 sequences each) are read by each sequence in
    the suffix pass, which runs beside the prefix pass."""
    cfg = REDUCED[4]
    assert cfg.name == "two_level_small"
    step = workloads.generate(cfg, seed=4)
    ds = dev_step(step)
    call = _call(ds, step.scale, share_min=0)
    batched = _call(ds, step.scale, share_min=1)
    assert call.workspace_bytes < batched.workspace_bytes, "the group nodes need no partials"
    out, lse = call()
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.step_attention(step, "all")
    compare(out, lse, ref_o, ref_l, cfg.dtype, "concurrent, private group nodes")


def test_concurrent_bad_metadata_gives_nan_rows_only():
    cfg = REDUCED[1]
    step = workloads.generate(cfg, seed=8)
    ds = dev_step(step)
    ds["block_table"][3, 0] = step.num_blocks
    ds["block_table"][5, 0] = -1
    ds["seq_lens"][9] = cfg.max_blocks * 16 + 1
    out, lse = _call(ds, step.scale)()
    torch.cuda.synchronize()
    bad = [3, 5, 9]
    assert torch.isnan(out[bad]).all() and torch.isnan(lse[bad]).all()
    good = [b for b in range(cfg.B) if b not in bad]
    rows = np.array([b * cfg.Hq + h for b in good for h in range(cfg.Hq)])
    ref_o, ref_l = oracle.step_attention(step, "all", rows=rows)
    compare(out, lse, ref_o, ref_l, cfg.dtype, "concurrent good rows", rows=rows)


def test_concurrent_orders_with_caller_stream():
    """Work enqueued on the caller's stream right before the step (a change of q) is seen
    by both passes, and a read enqueued right after it sees the merged result."""
    cfg = REDUCED[2]
    step = workloads.generate(cfg, seed=13)
    ds = dev_step(step)
    call = _call(ds, step.scale)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for rep in range(3):
            ds["q"].copy_((step.q * (1.0 + 0.5 * rep)).to(DEV), non_blocking=True)
            call(stream=s)
            got_o, got_l = call.out.clone(), call.lse.clone()  # ordered after the merge on s
            call.out.fill_(5.0)                                 # and before the next step
            s.synchronize()
            q_rep = (step.q.float() * (1.0 + 0.5 * rep)).to(step.q.dtype)
            segs = [[(nd.k, nd.v) for nd in step.nodes_of(b)] + [step.suffix(b)]
                    for b in range(cfg.B)]
            ref_o, ref_l = oracle.attention(q_rep, segs, cfg.Hkv, step.scale)
            compare(got_o, got_l, ref_o, ref_l, cfg.dtype, f"ordered step {rep}")


def test_concurrent_graph_replay_matches_eager():
    cfg = REDUCED[4]
    step = workloads.generate(cfg, seed=11)
    ds = dev_step(step)
    call = _call(ds, step.scale)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(stream=s)
        torch.cuda.synchronize()
        eager_o, eager_l = call.out.clone(), call.lse.clone()
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
        call()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(call.out, eager_o), f"eager after replay {rep}"


def test_concurrent_first_call_captured():
    """The very first call of a side-by-side step may be the one captured into a graph:
    nothing is created on first use (the second stream and the events exist before the
    call), and every replay equals a separate eager step on the same inputs."""
    cfg = REDUCED[3]
    step = workloads.generate(cfg, seed=17)
    ds = dev_step(step)
    ref_call = _call(ds, step.scale)
    eager_o, eager_l = [t.clone() for t in ref_call()]
    torch.cuda.synchronize()
    call = _call(ds, step.scale)
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
    ref_o, ref_l = oracle.step_attention(step, "all")
    compare(call.out, call.lse, ref_o, ref_l, cfg.dtype, "first call captured")


def test_concurrent_timed_records_events():
    """events[2] and events[4] are recorded on the second stream: the passes
    end between events[0] and events[3], the suffix pass lies between events[4] and
    events[2], and the result equals the untimed call."""
    cfg = REDUCED[2]
    step = workloads.generate(cfg, seed=12)
    ds = dev_step(step)
    call = _call(ds, step.scale)
    o1, l1 = [t.clone() for t in call()]
    torch.cuda.synchronize()
    rt = ctypes.CDLL("libamdhip64.so")
    raw = []
    for _ in range(5):
        h = ctypes.c_void_p()
        assert rt.hipEventCreate(ctypes.byref(h)) == 0
        raw.append(h.value)
    o2, l2 = call.timed(raw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)

    def ms(a, b):
        t = ctypes.c_float()
        assert rt.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return t.value
    total = ms(raw[0], raw[3])
    assert 0 < ms(raw[0], raw[1]) <= total and 0 < ms(raw[0], raw[2]) <= total
    # events[4]: on the second stream, right before the suffix pass (events[0] is
    # right before the prefix pass, so the two may come in either order)
    assert 0 < ms(raw[4], raw[2]) < ms(raw[4], raw[3])
    for h in raw:
        rt.hipEventDestroy(ctypes.c_void_p(h))
    ref_o, ref_l = oracle.step_attention(step, "all")
    compare(o2, l2, ref_o, ref_l, cfg.dtype, "concurrent timed")


def test_concurrent_from_two_host_threads():
    """Two host threads, each with its own stream, inputs, workspace, second stream and
    events, step side by side many times: each thread's results equal its
    single-threaded ones (the library shares nothing between the calls)."""
    import threading
    cfgs = [REDUCED[2], REDUCED[3]]
    setups = []
    for i, cfg in enumerate(cfgs):
        step = workloads.generate(cfg, seed=20 + i)
        ds = dev_step(step)
        call = _call(ds, step.scale)
        o, l = [t.clone() for t in call()]
        torch.cuda.synchronize()
        setups.append((call, o, l))
    errors = []

    def run(i):
        call, o_ref, l_ref = setups[i]
        s = torch.cuda.Stream()
        try:
            with torch.cuda.stream(s):
                for rep in range(20):
                    call.out.fill_(9.0)
                    call(stream=s)
                    got_o, got_l = call.out.clone(), call.lse.clone()
                    s.synchronize()
                    if not (torch.equal(got_o, o_ref) and torch.equal(got_l, l_ref)):
                        errors.append((i, rep))
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
