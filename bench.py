#!/usr/bin/env python3
"""Benchmark of one shared-prefix decode step on one MI355X.

Workload (default): a CodeLlama-13B-shaped attention layer -- 40 query heads =
40 KV heads, head dim 128, fp16 -- with B=256 sequences sharing a 16384-token
prefix and each owning a paged suffix of U[1,128] tokens (block size 16,
shuffled block tables).  Inputs are synthetic N(0,1), drawn from a seeded
generator and resident in HBM before timing starts.

A "step" is one hp_cascade_step: the prefix pass, the suffix pass and the
merge, for every (sequence, query head) row (for long prefixes the library
runs the suffix pass beside the prefix pass on a second stream of its own;
`passes_concurrent` says when).  Prints ONE JSON line with
steps/s (the metric), query-tokens/s, effective HBM GB/s of the whole step
against 8 TB/s, the roofline of the dominant kernel (timed with HIP events on
the stream it runs on), the prefix pass's MFMA fraction, a prefix-length sweep
(1K..16K), and the fp64 CPU oracle timed on a bounded sample of the same rows.
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
                  "common.hpp"]


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
        return workloads.codellama13b_mha(int(name.rsplit("p", 1)[1]))
    for c in workloads.all_configs():
        if c.name == name:
            return c
    raise SystemExit(f"unknown workload {name}")


def prepare(cfg, seed: int, overlap: int = 1):
    import torch
    import workloads
    import decode_attention_shared_amd as hp
    step = workloads.generate(cfg, seed=seed)
    dev = "cuda:0"
    levels = [[(n.k.to(dev), n.v.to(dev), n.seq_begin, n.seq_end) for n in lvl]
              for lvl in step.levels]
    call = hp.CascadeCall(step.q.to(dev), levels, step.k_pool.to(dev), step.v_pool.to(dev),
                          step.block_table.to(dev), step.seq_lens.to(dev), step.scale,
                          overlap=overlap)
    torch.cuda.synchronize()
    return step, call


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


def time_cold(call, ev: HipEvents, steps: int) -> float:
    """Median step time (ms) with 1 GiB read between steps (more than 2x the 256 MB
    Infinity Cache), so no step starts with its inputs cached.  The flush reads rather
    than writes: a written flush leaves the caches full of dirty lines whose write-back
    then competes with the step's own reads, which measures the flush, not the step."""
    import torch
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    sink = torch.zeros((), dtype=torch.float32, device="cuda:0")
    times = []
    for _ in range(steps):
        sink += flush.sum()
        e = ev.create(4)
        call.timed(e)
        times.append(ev.ms(e[0], e[3]))
    ev.close()
    del flush
    times.sort()
    return times[len(times) // 2]


def mean(xs):
    return sum(xs) / max(1, len(xs))


def cpu_baseline(step, target_s: float):
    """The fp64 oracle, as it stands, on a bounded sample of the same rows."""
    import numpy as np
    import oracle
    cfg = step.cfg
    total = cfg.B * cfg.Hq
    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    rng = np.random.default_rng(0)
    probe = np.sort(rng.choice(total, size=min(total, max(4 * threads, 64)), replace=False))
    t0 = time.perf_counter()
    oracle.step_attention(step, "all", rows=probe, nthreads=threads)
    per_row = (time.perf_counter() - t0) / len(probe)
    n = int(min(total, max(len(probe), target_s / max(per_row, 1e-9))))
    rows = np.sort(rng.choice(total, size=n, replace=False))
    t0 = time.perf_counter()
    oracle.step_attention(step, "all", rows=rows, nthreads=threads)
    el = time.perf_counter() - t0
    steps_per_s = (n / total) / el
    return {"value": steps_per_s, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {total} (sequence, query head) rows of the same step, seed 0, "
                      f"{el:.1f} s of fp64 work; steps/s scaled by rows"}


SHARE_SEQS = (2, 4, 8, 16, 32, 64, 128, 256)
SHARE_TOKENS = (64, 128, 256, 512, 1024, 2048, 4096, 16384)
SHARE_PRIVATE = 64  # private tokens per sequence beside the shared run


def share_sweep(reps: int = 20):
    """Batched vs private reading of one shared run of keys, through the chunk-tree step:
    the run's descriptors cover sequences [0, nseq); each sequence also owns SHARE_PRIVATE
    private rows.  share_min = 2 batches the run (prefix pass + merge), share_min =
    nseq + 1 makes every descriptor private (each sequence reads the run itself)."""
    import torch
    import decode_attention_shared_amd as hp
    out = []
    dev = "cuda:0"
    for (Hq, Hkv) in ((32, 32), (32, 8)):
        d = 128
        B = max(SHARE_SEQS)
        rows = max(SHARE_TOKENS) + B * SHARE_PRIVATE
        g = torch.Generator(device=dev).manual_seed(0)
        kp = torch.randn(rows, Hkv, d, generator=g, device=dev).to(torch.bfloat16)
        vp = torch.randn(rows, Hkv, d, generator=g, device=dev).to(torch.bfloat16)
        for nseq in SHARE_SEQS:
            q = torch.randn(nseq, Hq, d, generator=g, device=dev).to(torch.bfloat16)
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
                print(f"[share] Hq {Hq} Hkv {Hkv} nseq {nseq:3d} tokens {tok:5d}: batched "
                      f"{res['batched_us']:8.1f} us  private {res['private_us']:8.1f} us",
                      file=sys.stderr, flush=True)
    return {"share_sweep": out, "private_tokens_per_seq": SHARE_PRIVATE, "dtype": "bf16",
            "d": 128}


def other_configs(ev, seed: int, steps: int):
    """Step time of every other workload shape (cascade) and of the shared-document
    workload laid out as Parallel Prompting requests (stream decode), hot, inputs
    resident in HBM.  Effective GB/s = algorithmic bytes / wall time per step."""
    import torch
    import workloads
    import decode_attention_shared_amd as hp
    out = []
    for cfg in (workloads.tiny_f32(), workloads.llama3_8b_gqa(), workloads.docqa_codellama7b(),
                workloads.two_level_gqa()):
        print(f"[bench] config {cfg.name}", file=sys.stderr, flush=True)
        st, cl = prepare(cfg, seed)
        w, ps = time_steps(cl, ev, steps, SWEEP_WARMUP)
        b = workloads.algorithmic_bytes(cfg, st.seq_lens.tolist())["total"]
        wms = w / steps * 1e3
        out.append({"workload": cfg.name, "path": "cascade", "steps_per_s": round(steps / w, 1),
                    "ms_per_step": round(wms, 4), "algorithmic_bytes": b,
                    "effective_gbps": round(b / (wms * 1e-3) / 1e9, 1),
                    "hbm_roofline_frac": round(b / (wms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                    "pass_ms": {k: round(mean(ps[k]), 4) for k in ("prefix", "suffix", "merge")},
                    "passes_concurrent": bool(getattr(cl, "concurrent", False))})
        del cl, st
        torch.cuda.empty_cache()
    cfg = workloads.docqa_streams(32)
    print(f"[bench] config {cfg.name}", file=sys.stderr, flush=True)
    st = workloads.stream_step(cfg, P=32, seed=seed)
    dev = "cuda:0"
    levels = [[(n.k.to(dev), n.v.to(dev), n.seq_begin, n.seq_end) for n in lvl]
              for lvl in st.levels]
    call = hp.StreamCall(st.q.to(dev), levels, st.k_pool.to(dev), st.v_pool.to(dev),
                         st.row_slots.to(dev), st.row_sid.to(dev), st.row_len.to(dev),
                         st.q_req.to(dev), st.q_sid.to(dev), st.scale)
    for _ in range(SWEEP_WARMUP):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    w = time.perf_counter() - t0
    b = workloads.stream_bytes(st)["total"]
    wms = w / steps * 1e3
    out.append({"workload": cfg.name, "path": "stream_decode", "steps_per_s": round(steps / w, 1),
                "ms_per_step": round(wms, 4), "algorithmic_bytes": b,
                "effective_gbps": round(b / (wms * 1e-3) / 1e9, 1),
                "hbm_roofline_frac": round(b / (wms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workload shapes and the stream-decode workload")
    ap.add_argument("--sweep-steps", type=int, default=200)
    ap.add_argument("--profile-only", action="store_true",
                    help="only run warmup + timed steps (for rocprofv3); no sweep or CPU leg")
    ap.add_argument("--share-sweep", action="store_true",
                    help="instead of the step, time one shared run of keys read once for all its "
                         "sequences (batched) against each sequence reading it (private), over a "
                         "grid of sequence counts and run lengths (the data the batching policy "
                         "is fitted to)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the step, run --steps device-to-device copies of MIB MiB "
                         "(a plain copy of known size, to calibrate HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (it would "
              "shard by KV head with no exchange; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")

    if args.share_sweep:
        print(json.dumps(share_sweep()), flush=True)
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
    step, call = prepare(cfg, args.seed)
    ev = HipEvents()
    print(f"[bench] timing {args.steps} steps after {args.warmup} warmup", file=sys.stderr,
          flush=True)
    wall, passes = time_steps(call, ev, args.steps, args.warmup)
    lens = step.seq_lens.tolist()
    ab = workloads.algorithmic_bytes(cfg, lens)
    flops = workloads.prefix_flops(cfg)
    step_ms = mean(passes["step"])
    ms_per_step = wall / args.steps * 1e3
    steps_per_s = args.steps / wall
    pass_bytes = {"prefix": ab["prefix"] + ab["q"], "suffix": ab["suffix"] + ab["q"],
                  "merge": ab["out"]}
    pass_ms = {k: mean(passes[k]) for k in ("prefix", "suffix", "merge")}
    dom = max(pass_ms, key=pass_ms.get)
    achieved = pass_bytes[dom] / (pass_ms[dom] * 1e-3) / 1e9
    khash = kernel_hash()
    traffic = load_traffic(f"{cfg.name}:{dom}", khash)
    mfma_peak = MFMA_F32_PEAK_TFLOPS if cfg.dtype == "f32" else MFMA_F16_PEAK_TFLOPS
    prefix_tflops = flops / (pass_ms["prefix"] * 1e-3) / 1e12
    # whole-step effective bandwidth from the wall-clock step time (the event-timed
    # steps carry a few microseconds of event overhead)
    eff = ab["total"] / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if cfg.dtype == "f16" else cfg.dtype,
        "data": "synthetic N(0,1), seeded; inputs resident in HBM",
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "d": cfg.d,
                   "prefix_tokens": [n[0] for lvl in cfg.levels for n in lvl],
                   "suffix": f"U[{cfg.suffix_lo},{cfg.suffix_hi}] paged, block 16",
                   "seed": args.seed, "parallelism": "single GPU"},
        "query_tokens_per_s": round(steps_per_s * cfg.B, 1),
        "step_ms_events": round(step_ms, 4),
        "effective_gbps": round(eff, 1),
        "hbm_roofline_frac": round(eff / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes": ab,
        "pass_ms": {k: round(v, 4) for k, v in pass_ms.items()},
        "passes_concurrent": bool(getattr(call, "concurrent", False)),
        "prefix_mfma_frac": round(prefix_tflops / mfma_peak, 4),
        "prefix_tflops": round(prefix_tflops, 1),
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": (traffic or {}).get("bytes_per_launch"),
                     "algorithmic_bytes_per_launch": pass_bytes[dom],
                     "kernel_hash": khash},
    }
    if not args.profile_only:
        print("[bench] cold (cache-flushed) steps", file=sys.stderr, flush=True)
        result["cold_step_ms_median"] = round(time_cold(call, ev, 20), 4)
    del call
    torch.cuda.empty_cache()
    if not args.profile_only and not args.no_sweep and cfg.name.startswith("codellama13b"):
        sweep = []
        for P in workloads.CODELLAMA13B_SWEEP:
            c = workloads.codellama13b_mha(P)
            print(f"[bench] sweep prefix {P}", file=sys.stderr, flush=True)
            st, cl = prepare(c, args.seed)
            w, ps = time_steps(cl, ev, args.sweep_steps, SWEEP_WARMUP)
            sm = mean(ps["step"])
            b = workloads.algorithmic_bytes(c, st.seq_lens.tolist())["total"]
            wms = w / args.sweep_steps * 1e3
            sweep.append({"prefix": P, "steps_per_s": round(args.sweep_steps / w, 1),
                          "step_ms_events": round(sm, 4),
                          "effective_gbps": round(b / (wms * 1e-3) / 1e9, 1),
                          "hbm_roofline_frac": round(b / (wms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                          "pass_ms": {k: round(mean(ps[k]), 4) for k in ("prefix", "suffix",
                                                                         "merge")},
                          "passes_concurrent": bool(getattr(cl, "concurrent", False))})
            del cl, st
            torch.cuda.empty_cache()
        result["prefix_sweep"] = sweep
    if not args.profile_only and not args.no_configs:
        result["configs"] = other_configs(ev, args.seed, args.sweep_steps)
    if not args.profile_only and not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(step, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
