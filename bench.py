#!/usr/bin/env python3
"""Benchmark of one shared-prefix decode step on one MI355X.

Workload (default): a CodeLlama-13B-shaped attention layer -- 40 query heads =
40 KV heads, head dim 128, fp16 -- with B=256 sequences sharing a 16384-token
prefix and each owning a paged suffix of U[1,128] tokens (block size 16,
shuffled block tables).  Inputs are synthetic N(0,1), drawn from a seeded
generator and resident in HBM before timing starts.

A "step" is one hp_cascade_step: the prefix pass, the suffix pass and the
merge, for every (sequence, query head) row (for long prefixes the library
runs the suffix pass beside the prefix pass on a second, caller-owned stream;
`passes_concurrent` says when).

Timing protocol.  The step is captured once into a HIP graph.  Each timed step
is one graph replay preceded by a read of 1 GiB (four times the 256 MB
Infinity Cache), so no step starts with its inputs cached; HIP events on the
replay stream bracket the replay alone, and the headline is the median over
the timed steps.  Beside it: the hot time (back-to-back eager steps, and
back-to-back replays); the per-pass split of eager steps (HIP events recorded
by the library on the streams its kernels run on), hot, and flushed with the
passes one after the other, where each kernel has the GPU to itself: the
longest of those gives the dominant kernel's roofline (`--profile-only` runs
just that loop, for rocprofv3); and the same protocol for a prefix-length
sweep (1K..16K) and every other workload shape.  Prints ONE JSON line; the fp64 CPU oracle is
timed over the whole step on the host's cores beside it.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense fp16/bf16 matrix peak
MFMA_F32_PEAK_TFLOPS = 157.3
METRIC = "decode attention steps/s + effective HBM GB/s (% roofline) at B=256, 16K prefix"
KERNEL_SOURCES = ["prefix_kernel.hip", "suffix_kernel.hip", "merge_kernel.hip", "api.cpp", "host.hpp",
                  "common.hpp", "fat_suffix.hpp"]


class HipEvents:
    """hipEvent_t handles through the HIP runtime (timing of the library's own launches)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(h.value)
        self.made += out
        return out

    def ms(self, a, b) -> float:
        self.rt.hipEventSynchronize(b)
        t = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(t), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(t.value)

    def close(self):
        for h in self.made:
            self.rt.hipEventDestroy(h)
        self.made = []


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_shared_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def workload(name: str):
    import workloads
    if name.startswith("codellama13b_mha_p"):
        rest = name[len("codellama13b_mha_p"):]
        if "_share" in rest:
            prefix, ways = rest.split("_share")
            return workloads.codellama13b_mha_share(int(ways), int(prefix))
        return workloads.codellama13b_mha(int(rest))
    for c in workloads.all_configs():
        if c.name == name:
            return c
    raise SystemExit(f"unknown workload {name}")


# Paged suffix blocks as head-major [Hkv][16][d] (each (sequence, KV head) reads
# 16 contiguous rows per block; measured faster than token-major [16][Hkv][d]).
KV_LAYOUT = "HND"


def prepare(cfg, seed: int, overlap: int = 1, kv_layout: str = KV_LAYOUT):
    """Draw the step's inputs, copy them to the GPU and prepare the cascade call."""
    import workloads
    step = workloads.generate(cfg, seed=seed)
    dev = "cuda:0"
    levels = [[(n.k.to(dev), n.v.to(dev), n.seq_begin, n.seq_end) for n in lvl]
              for lvl in step.levels]
    inputs = (step.q.to(dev), levels, workloads.pool_in_layout(step.k_pool, kv_layout).to(dev),
              workloads.pool_in_layout(step.v_pool, kv_layout).to(dev),
              step.block_table.to(dev), step.seq_lens.to(dev), step.scale)
    return step, make_call(inputs, overlap, kv_layout)


def make_call(inputs, overlap: int, kv_layout: str = KV_LAYOUT):
    """A CascadeCall over device inputs (q, levels, pools, table, lengths, scale)."""
    import torch
    import decode_attention_shared_amd as hp
    call = hp.CascadeCall(*inputs, overlap=overlap, kv_layout=kv_layout)
    call.inputs = inputs
    call.kv_layout = kv_layout
    torch.cuda.synchronize()
    return call


EVENT_EVERY = 10  # steps between event-instrumented steps inside the timed region


# Untimed steps before each sweep point and other shape: as many as before the
# headline run, so that every line is timed after the same ramp of clocks and
# queues.
SWEEP_WARMUP = 20


def time_steps(call, ev: HipEvents, steps: int, warmup: int):
    """Returns wall seconds for `steps` back-to-back steps and per-pass event times (ms).

    Every EVENT_EVERY-th step records HIP events around its passes (on the library's
    stream); the others run plain.  An event record costs a few microseconds on this
    runtime, so instrumenting every step would inflate the step time it measures."""
    import torch
    for _ in range(warmup):
        call()
    timed_at = set(range(0, steps, EVENT_EVERY))
    evs = {k: ev.create(5) for k in sorted(timed_at)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        if k in timed_at:
            call.timed(evs[k])
        else:
            call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    passes = {"prefix": [], "suffix": [], "merge": [], "step": []}
    # events[4] is recorded right before the suffix launch on its own stream (the
    # library's second stream when the passes run side by side), so the suffix
    # pass is timed from its start; the merge starts when the later pass ends.
    for e in evs.values():
        t1, t2, t3 = ev.ms(e[0], e[1]), ev.ms(e[0], e[2]), ev.ms(e[0], e[3])
        passes["prefix"].append(t1)
        passes["suffix"].append(ev.ms(e[4], e[2]))
        passes["merge"].append(t3 - max(t1, t2))
        passes["step"].append(t3)
    ev.close()
    return wall, passes


FLUSH_BYTES = 1 << 30  # read between timed steps: four times the 256 MB Infinity Cache


class Flusher:
    """Reads FLUSH_BYTES (a sum over a 1 GiB buffer) on the current stream.  A read,
    not a write: a written flush leaves the caches full of dirty lines whose
    write-back then competes with the step's own reads."""

    def __init__(self):
        import torch
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
        self.sink = torch.zeros((), dtype=torch.float32, device="cuda:0")

    def __call__(self):
        self.sink += self.buf.sum()


def capture(call, warmup: int):
    """The step captured into a HIP graph (on a side stream, as capture requires), after
    `warmup` eager steps; then `warmup` untimed replays."""
    import torch
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    return g


def time_flushed(g, flush: Flusher, steps: int):
    """Per-step times (ms, sorted) of `steps` graph replays, each after a cache flush,
    each bracketed by HIP events on the replay stream; and the wall seconds of the
    whole region (flushes included), synchronised on both sides."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        flush()
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return sorted(e0.elapsed_time(e1) for e0, e1 in evs), wall


def time_passes_flushed(call, ev: HipEvents, flush: Flusher, steps: int, warmup: int):
    """Per-pass times (ms) of `steps` eager steps, each after a cache flush, from the
    HIP events the library records around its passes on the streams they run on."""
    import torch
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        flush()
        e = ev.create(5)
        call.timed(e)
        evs.append(e)
    torch.cuda.synchronize()
    passes = {"prefix": [], "suffix": [], "merge": [], "step": []}
    for e in evs:
        t1, t2, t3 = ev.ms(e[0], e[1]), ev.ms(e[0], e[2]), ev.ms(e[0], e[3])
        passes["prefix"].append(t1)
        passes["suffix"].append(ev.ms(e[4], e[2]))
        passes["merge"].append(t3 - max(t1, t2))
        passes["step"].append(t3)
    ev.close()
    return passes


def copy_gbps(mib: int = 1024, reps: int = 10) -> float:
    """Bytes moved (read + written) per second by a plain device-to-device copy of `mib`
    MiB: the streaming rate this GPU reaches in the same run, beside the 8 TB/s spec."""
    import torch
    src = torch.ones((mib << 20) // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = time_hot(lambda: dst.copy_(src), reps)
    del src, dst
    return 2.0 * (mib << 20) / (ms * 1e-3) / 1e9


def stream_read_gbps(mib: int = 4096, reps: int = 5) -> float:
    """Bytes per second that the library's streaming-read probe (one pass of 16-byte
    non-temporal loads, nothing written but one word per workgroup) pulls from a
    `mib` MiB buffer, sixteen times the Infinity Cache (long enough that the launch's
    ramp does not count): the read ceiling of this GPU in the same run, beside the
    8 TB/s spec."""
    import torch
    import decode_attention_shared_amd as hp
    buf = torch.ones((mib << 20) // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.empty(hp.HP_READ_PROBE_WGS, dtype=torch.int32, device="cuda:0")
    hp.read_probe(buf, sink)
    ms = time_hot(lambda: hp.read_probe(buf, sink), reps)
    del buf, sink
    return (mib << 20) / (ms * 1e-3) / 1e9


def time_hot(fn, steps: int) -> float:
    """Mean ms of `steps` back-to-back calls of fn, between two HIP events."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) / steps


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def measure(cfg, step, call, ev, flush, steps: int, warmup: int) -> dict:
    """The protocol above for one prepared workload: flushed graph replays (headline),
    hot eager and hot graph steps, and the per-pass split of eager steps."""
    import workloads
    g = capture(call, warmup)
    times, wall = time_flushed(g, flush, steps)
    hot_graph = time_hot(g.replay, steps)
    eager_wall, passes = time_steps(call, ev, steps, warmup)
    del g
    b = workloads.algorithmic_bytes(cfg, step.seq_lens.tolist())
    med = median(times)
    return {"cold_ms_median": med, "cold_ms_mean": mean(times), "cold_ms_min": times[0],
            "cold_ms_max": times[-1],
            "region_wall_s": wall, "hot_graph_ms": hot_graph,
            "hot_eager_ms": eager_wall / steps * 1e3, "passes": passes, "bytes": b,
            "concurrent": bool(getattr(call, "concurrent", False))}


def summary(cfg, m: dict) -> dict:
    """One workload's line: steps/s and effective GB/s from the flushed median."""
    b = m["bytes"]["total"]
    med = m["cold_ms_median"]
    return {"workload": cfg.name, "steps_per_s": round(1e3 / med, 1),
            "ms_per_step": round(med, 4), "ms_per_step_mean": round(m["cold_ms_mean"], 4),
            "algorithmic_bytes": b,
            "effective_gbps": round(b / (med * 1e-3) / 1e9, 1),
            "hbm_roofline_frac": round(b / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "hot_eager_ms": round(m["hot_eager_ms"], 4),
            "hot_graph_ms": round(m["hot_graph_ms"], 4),
            "pass_ms_eager": {k: round(mean(m["passes"][k]), 4)
                              for k in ("prefix", "suffix", "merge")},
            "passes_concurrent": m["concurrent"]}


def mean(xs):
    return sum(xs) / max(1, len(xs))


def cpu_model() -> str:
    """The host CPU's model name (lscpu when present, else /proc/cpuinfo)."""
    import shutil
    import subprocess
    if shutil.which("lscpu"):
        try:
            out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
            for line in out.splitlines():
                if line.strip().startswith("Model name"):
                    return line.split(":", 1)[1].strip()
        except (OSError, subprocess.SubprocessError):
            pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    return max(1, threads)


def oracle_pass(step, threads: int, budget_s: float):
    """Seconds of the fp64 oracle, as it stands, over every row of the step; when a probe
    of 64 rows projects more than budget_s, over the rows that fit in about half of it
    (scaled to the whole step).  Returns (seconds per step, rows timed)."""
    import numpy as np
    import oracle
    cfg = step.cfg
    total = cfg.B * cfg.Hq
    rng = np.random.default_rng(0)
    probe = np.sort(rng.choice(total, size=min(total, 64), replace=False))
    t0 = time.perf_counter()
    oracle.step_attention(step, "all", rows=probe, nthreads=threads)
    per_row = (time.perf_counter() - t0) / len(probe)
    if per_row * total <= budget_s:
        t0 = time.perf_counter()
        oracle.step_attention(step, "all", nthreads=threads)
        return time.perf_counter() - t0, total
    n = max(len(probe), int(0.5 * budget_s / max(per_row, 1e-9)))
    rows = np.sort(rng.choice(total, size=min(total, n), replace=False))
    t0 = time.perf_counter()
    oracle.step_attention(step, "all", rows=rows, nthreads=threads)
    return (time.perf_counter() - t0) * total / len(rows), len(rows)


def cpu_baseline(step, budget_s: float):
    """The fp64 oracle over the whole step on this host's cores (a baseline only)."""
    threads = host_threads()
    sec, rows = oracle_pass(step, threads, budget_s)
    total = step.cfg.B * step.cfg.Hq
    what = (f"the whole step: all {total} (sequence, query head) rows" if rows == total else
            f"{rows} of {total} (sequence, query head) rows, scaled to the step")
    return {"value": round(1.0 / sec, 5), "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}, seed {step.seed}; {sec:.1f} s of fp64 work per step",
            "cpu_model": cpu_model()}


SHARE_SEQS = (2, 4, 8, 16, 32, 64, 128, 256)
SHARE_TOKENS = (64, 128, 256, 512, 1024, 2048, 4096, 16384)
SHARE_PRIVATE = 64  # private tokens per sequence beside the shared run


def share_sweep(dtype: str = "bf16", d: int = 128, reps: int = 20):
    """Batched vs private reading of one shared run of keys, through the chunk-tree step:
    the run's descriptors cover sequences [0, nseq); each sequence also owns SHARE_PRIVATE
    private rows.  share_min = 2 batches the run (prefix pass + merge), share_min =
    nseq + 1 makes every descriptor private (each sequence reads the run itself)."""
    import torch
    import decode_attention_shared_amd as hp
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    out = []
    dev = "cuda:0"
    for (Hq, Hkv) in ((32, 32), (32, 8)):
        B = max(SHARE_SEQS)
        rows = max(SHARE_TOKENS) + B * SHARE_PRIVATE
        g = torch.Generator(device=dev).manual_seed(0)
        kp = torch.randn(rows, Hkv, d, generator=g, device=dev).to(tdt)
        vp = torch.randn(rows, Hkv, d, generator=g, device=dev).to(tdt)
        for nseq in SHARE_SEQS:
            q = torch.randn(nseq, Hq, d, generator=g, device=dev).to(tdt)
            for tok in SHARE_TOKENS:
                descs = [(r, min(64, tok - r), 0, nseq) for r in range(0, tok, 64)]
                base = max(SHARE_TOKENS)
                descs += [(base + b * SHARE_PRIVATE + r, 64, b, b + 1)
                          for b in range(nseq) for r in range(0, SHARE_PRIVATE, 64)]
                res = {"Hq": Hq, "Hkv": Hkv, "nseq": nseq, "tokens": tok}
                for mode, smin in (("batched", 2), ("private", nseq + 1)):
                    ts = hp.TreeStep(q, Hkv, descs, smin, rows, 1.0 / d ** 0.5)
                    o, l = ts(q, kp, vp)
                    for _ in range(5):
                        ts(q, kp, vp, out=o, lse=l)
                    torch.cuda.synchronize()
                    times = []
                    for _ in range(reps):
                        a = torch.cuda.Event(enable_timing=True)
                        e = torch.cuda.Event(enable_timing=True)
                        a.record()
                        ts(q, kp, vp, out=o, lse=l)
                        e.record()
                        e.synchronize()
                        times.append(a.elapsed_time(e) * 1e3)
                    times.sort()
                    res[mode + "_us"] = round(times[len(times) // 2], 2)
                res["batched_wins"] = res["batched_us"] < res["private_us"]
                out.append(res)
                print(f"[share] {dtype} d {d} Hq {Hq} Hkv {Hkv} nseq {nseq:3d} tokens {tok:5d}: batched "
                      f"{res['batched_us']:8.1f} us  private {res['private_us']:8.1f} us",
                      file=sys.stderr, flush=True)
    return {"share_sweep": out, "private_tokens_per_seq": SHARE_PRIVATE, "dtype": dtype,
            "d": d}


def other_configs(ev, flush, seed: int, steps: int, cpu_budget_s: float):
    """Every other workload shape (cascade step; one 8-way head share of the headline
    shape) and the shared-document workload laid out as Parallel Prompting requests
    (stream decode), each under the same protocol as the headline, with the fp64 oracle
    over the same step beside it (cpu_budget_s <= 0: no oracle)."""
    import torch
    import workloads
    import decode_attention_shared_amd as hp
    out = []
    threads = host_threads()
    for cfg in (workloads.tiny_f32(), workloads.llama3_8b_gqa(), workloads.docqa_codellama7b(),
                workloads.two_level_gqa(), workloads.codellama13b_mha_share(8)):
        print(f"[bench] config {cfg.name}", file=sys.stderr, flush=True)
        st, cl = prepare(cfg, seed)
        line = summary(cfg, measure(cfg, st, cl, ev, flush, steps, SWEEP_WARMUP))
        line["path"] = "cascade"
        del cl
        torch.cuda.empty_cache()
        if cpu_budget_s > 0:
            sec, rows = oracle_pass(st, threads, cpu_budget_s)
            line["cpu_oracle"] = {"s_per_step": round(sec, 3), "cores": threads,
                                  "rows_timed": rows}
            if cfg.name in ("tiny_f32", "llama3_8b_gqa"):
                sec1, rows1 = oracle_pass(st, 1, cpu_budget_s)
                line["cpu_oracle"].update({"s_per_step_1core": round(sec1, 3),
                                           "rows_timed_1core": rows1})
        out.append(line)
        del st
    cfg = workloads.docqa_streams(32)
    print(f"[bench] config {cfg.name}", file=sys.stderr, flush=True)
    st = workloads.stream_step(cfg, P=32, seed=seed)
    dev = "cuda:0"
    levels = [[(n.k.to(dev), n.v.to(dev), n.seq_begin, n.seq_end) for n in lvl]
              for lvl in st.levels]
    call = hp.StreamCall(st.q.to(dev), levels, st.k_pool.to(dev), st.v_pool.to(dev),
                         st.row_slots.to(dev), st.row_sid.to(dev), st.row_len.to(dev),
                         st.q_req.to(dev), st.q_sid.to(dev), st.scale)
    g = capture(call, SWEEP_WARMUP)
    times, _ = time_flushed(g, flush, steps)
    hot_graph = time_hot(g.replay, steps)
    hot_eager = time_hot(call, steps)
    del g
    b = workloads.stream_bytes(st)["total"]
    med = median(times)
    out.append({"workload": cfg.name, "path": "stream_decode",
                "steps_per_s": round(1e3 / med, 1), "ms_per_step": round(med, 4),
                "algorithmic_bytes": b, "effective_gbps": round(b / (med * 1e-3) / 1e9, 1),
                "hbm_roofline_frac": round(b / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "hot_eager_ms": round(hot_eager, 4), "hot_graph_ms": round(hot_graph, 4),
                "requests": st.R, "streams_per_request": 32,
                "row_positions": int(st.row_len.sum())})
    del call, st
    torch.cuda.empty_cache()
    return out


def load_traffic(name: str, khash: str):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(name)
    if not ent or ent.get("kernel_hash") != khash:
        return None
    return ent


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="codellama13b_mha_p16384")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--overlap", type=int, default=1, choices=(0, 1, 2),
                    help="hp_cascade_step_overlap mode of the headline step: 0 the passes one "
                         "after the other, 1 (default) side by side when the library's plan "
                         "expects a gain, 2 side by side whenever possible")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=60.0,
                    help="the oracle runs over every row of a step when a probe projects at "
                         "most this many seconds, else over a sample of about half of it")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workload shapes and the stream-decode workload")
    ap.add_argument("--sweep-steps", type=int, default=200)
    ap.add_argument("--profile-only", action="store_true",
                    help="only warmup + timed eager steps (for rocprofv3); no graph, sweep, "
                         "other shapes or CPU leg")
    ap.add_argument("--share-sweep", action="store_true",
                    help="instead of the step, time one shared run of keys read once for all its "
                         "sequences (batched) against each sequence reading it (private), over a "
                         "grid of sequence counts and run lengths (the data the batching policy "
                         "is fitted to)")
    ap.add_argument("--share-dtype", default="bf16", choices=("bf16", "f16", "f32"),
                    help="storage type of the --share-sweep keys, values and queries")
    ap.add_argument("--share-d", type=int, default=128, choices=(64, 128),
                    help="head dimension of the --share-sweep")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the step, run --steps device-to-device copies of MIB MiB "
                         "(a plain copy of known size, to calibrate HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (a step "
              "would shard by KV head with no exchange between GPUs). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")

    if args.share_sweep:
        print(json.dumps(share_sweep(args.share_dtype, args.share_d)), flush=True)
        return

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        print(json.dumps({"copy_probe_bytes": n, "copies": args.steps,
                          "gbps_read_plus_write": round(2 * n * args.steps / el / 1e9, 1)}))
        return

    cfg = workload(args.workload)
    print(f"[bench] generating {cfg.name} seed {args.seed}", file=sys.stderr, flush=True)
    step, call = prepare(cfg, args.seed, overlap=args.overlap)
    ev = HipEvents()
    lens = step.seq_lens.tolist()
    ab = workloads.algorithmic_bytes(cfg, lens)
    flops = workloads.prefix_flops(cfg)
    pass_bytes = {"prefix": ab["prefix"] + ab["q"], "suffix": ab["suffix"] + ab["q"],
                  "merge": ab["out"]}
    khash = kernel_hash()
    mfma_peak = MFMA_F32_PEAK_TFLOPS if cfg.dtype == "f32" else MFMA_F16_PEAK_TFLOPS

    def roofline(pass_ms):
        # the pass that takes longest when each runs on the whole GPU by itself
        dom = max(pass_ms, key=pass_ms.get)
        achieved = pass_bytes[dom] / (pass_ms[dom] * 1e-3) / 1e9
        traffic = load_traffic(f"{cfg.name}:{dom}", khash)
        return {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": (traffic or {}).get("bytes_per_launch"),
                "algorithmic_bytes_per_launch": pass_bytes[dom],
                "launch_ms": round(pass_ms[dom], 4), "kernel_hash": khash}

    config = {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "d": cfg.d,
              "prefix_tokens": [n[0] for lvl in cfg.levels for n in lvl],
              "suffix": f"U[{cfg.suffix_lo},{cfg.suffix_hi}] paged, block 16, {KV_LAYOUT} blocks",
              "seed": args.seed, "parallelism": "single GPU"}
    common = {"unit": "steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": cfg.dtype, "data": "synthetic N(0,1), seeded; inputs resident in HBM",
              "config": config}

    flush = Flusher()
    if args.profile_only:
        # the roofline's measurement alone, for rocprofv3 (kernel trace or counters):
        # eager steps, each after a cache flush, passes timed by the library's events
        print(f"[bench] {args.steps} flushed eager steps after {args.warmup} warmup",
              file=sys.stderr, flush=True)
        passes = time_passes_flushed(call, ev, flush, args.steps, args.warmup)
        pass_ms = {k: mean(passes[k]) for k in ("prefix", "suffix", "merge")}
        ms = median(passes["step"])
        print(json.dumps({"metric": METRIC + " (profiling run: flushed eager steps)",
                          "value": round(1e3 / ms, 2), "ms_per_step": round(ms, 4), **common,
                          "pass_ms": {k: round(v, 4) for k, v in pass_ms.items()},
                          "passes_concurrent": bool(call.concurrent),
                          "roofline": roofline(pass_ms)}), flush=True)
        return

    print(f"[bench] {args.steps} flushed graph replays after {args.warmup} warmup",
          file=sys.stderr, flush=True)
    m = measure(cfg, step, call, ev, flush, args.steps, args.warmup)
    med = m["cold_ms_median"]
    pass_ms = {k: mean(m["passes"][k]) for k in ("prefix", "suffix", "merge")}
    # Each kernel by itself: the passes one after the other on one stream (in the
    # side-by-side plan a pass's duration includes sharing the GPU with the other),
    # each step after a cache flush like the headline's.
    print("[bench] serial plan, flushed: each pass on the whole GPU", file=sys.stderr,
          flush=True)
    scall = make_call(call.inputs, 0, call.kv_layout) if m["concurrent"] else call
    sp = time_passes_flushed(scall, ev, flush, args.steps, args.warmup)
    del scall
    alone_ms = {k: mean(sp[k]) for k in ("prefix", "suffix", "merge")}
    prefix_tflops = flops / (alone_ms["prefix"] * 1e-3) / 1e12
    eff = ab["total"] / (med * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(1e3 / med, 2),
        "ms_per_step": round(med, 4),
        **common,
        "timing": (f"median of {args.steps} HIP-graph replays of the step, each after a "
                   f"{FLUSH_BYTES >> 30} GiB read that evicts the Infinity Cache; HIP events "
                   "around each replay on its stream"),
        "cold_ms_mean": round(m["cold_ms_mean"], 4),
        "cold_ms_min": round(m["cold_ms_min"], 4),
        "cold_ms_max": round(m["cold_ms_max"], 4),
        "timed_region_wall_s": round(m["region_wall_s"], 4),
        "hot_eager_ms": round(m["hot_eager_ms"], 4),
        "hot_graph_ms": round(m["hot_graph_ms"], 4),
        "query_tokens_per_s": round(1e3 / med * cfg.B, 1),
        "effective_gbps": round(eff, 1),
        "hbm_roofline_frac": round(eff / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes": ab,
        "pass_ms_eager": {k: round(v, 4) for k, v in pass_ms.items()},
        "passes_concurrent": m["concurrent"],
        "pass_ms_alone": {k: round(v, 4) for k, v in alone_ms.items()},
        "prefix_mfma_frac": round(prefix_tflops / mfma_peak, 4),
        "prefix_tflops": round(prefix_tflops, 1),
        "roofline": roofline(alone_ms),
        "device_copy_gbps": None,
    }
    del call
    torch.cuda.empty_cache()
    cg = copy_gbps()
    result["device_copy_gbps"] = round(cg, 1)
    result["hbm_frac_of_device_copy"] = round(eff / cg, 4)
    rg = stream_read_gbps()
    result["device_stream_read_gbps"] = round(rg, 1)
    result["hbm_frac_of_stream_read"] = round(eff / rg, 4)
    if not args.no_sweep and cfg.name.startswith("codellama13b"):
        sweep = []
        for P in workloads.CODELLAMA13B_SWEEP:
            c = workloads.codellama13b_mha(P)
            print(f"[bench] sweep prefix {P}", file=sys.stderr, flush=True)
            st, cl = prepare(c, args.seed)
            line = summary(c, measure(c, st, cl, ev, flush, args.sweep_steps, SWEEP_WARMUP))
            line["prefix"] = P
            # bytes relative to the 16K step: the steps/s a bandwidth-bound step would show
            line["bytes_vs_headline"] = round(line["algorithmic_bytes"] / ab["total"], 4)
            sweep.append(line)
            del cl, st
            torch.cuda.empty_cache()
        result["prefix_sweep"] = sweep
    if not args.no_configs:
        result["configs"] = other_configs(ev, flush, args.seed, args.sweep_steps,
                                          0.0 if args.no_cpu_baseline else args.cpu_seconds)
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(step, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
