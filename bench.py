#!/usr/bin/env python3
"""Benchmark: MLA decode attention on one MI355X.

One step = one mla_decode call (split kernel: plan and attention over each
key range; combine kernel: merge of the sequences split across ranges) over
the whole batch, inputs already resident in HBM.  The default workload
is batch 16, 16 heads, one query token, 65536 cached keys per sequence
(KV cache 1,207,959,552 B, larger than the 256 MB last-level cache, so every
step streams it from HBM).  Prints one JSON line.

  value      KV-cache bytes of a step / step time, GB/s (whole job)
  roofline   the split kernel: algorithmic KV bytes per launch / its mean
             launch time from HIP events on the stream it runs on, against
             MI355X's 8 TB/s; traffic from committed rocprofv3 counters when
             they were taken on the current kernel source, else null
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload on
             the host cores (a reported baseline, not a target)

Other modes: --workload NAME (any of workloads.WORKLOADS), --calibrate-copy
(a plain 1 GiB device copy, the reference for the HBM byte counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV HBM GB/s (% of peak) + µs/call, MLA decode bs16 ctx64K 16 heads"
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ("decode_attention_mla_amd/csrc/mla_kernels.hip", "decode_attention_mla_amd/csrc/context.h",
                  "decode_attention_mla_amd/csrc/plan.h", "include/mla_decode.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload: str):
    """HBM bytes per split-kernel launch from committed counter runs, if they
    were taken on this exact kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_mla_split_{workload}.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None, rec
    return rec.get("bytes_per_launch"), rec


def cpu_threads() -> int:
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def calibrate_copy(steps: int) -> None:
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"mode": "calibrate-copy", "bytes_read": n, "bytes_written": n,
                      "ms_per_copy": dt * 1e3, "GBps_read_plus_write": 2 * n / dt / 1e9}))


def sweep(args) -> int:
    """The pages' sweep grid on one GPU: KV GB/s against context length at
    batch 16 and 32 (16 heads), and against the per-GPU head count (16, 32,
    64, 128) at batch 16 x 64K.  One JSON line per point.  Inputs are seeded
    N(0,1) bf16 drawn on the device (a timing curve: parity is the tests'
    job); workloads under 1 GiB rotate over copies so every step streams
    from HBM."""
    import numpy as np
    import torch

    import decode_attention_mla_amd as mla

    gen = torch.Generator(device="cuda")
    points = [(b, 1, 16, L) for b in (16, 32) for L in (512, 1024, 2048, 4096, 8192, 16384, 32768, 65536)]
    points += [(16, 1, h, 65536) for h in (32, 64, 128)]
    if args.sweep_points:
        keep = {tuple(int(x) for x in p.split("x")) for p in args.sweep_points.split(",")}
        points = [pt for pt in points if (pt[0], pt[2], pt[3]) in keep] or \
                 [(b, 1, h, L) for b, h, L in sorted(keep)]
    ctx = mla.Context()
    ctx.set_option(mla.MLA_OPT_NUM_SPLITS, args.splits)
    ctx.set_option(mla.MLA_OPT_MIN_CHUNK, args.min_chunk)
    scale = 1.0 / 24.0
    for B, s_q, H, L in points:
        gen.manual_seed(7000 + B * 131 + H * 17 + L)
        q = torch.randn((B, s_q, H, 576), generator=gen, device="cuda").to(torch.bfloat16)
        kv = torch.randn((B, L, 576), generator=gen, device="cuda").to(torch.bfloat16)
        lens_h = np.full(B, L, dtype=np.int32)
        lens = torch.from_numpy(lens_h).cuda()
        kv_bytes = B * L * 576 * 2
        copies = [kv]
        while kv_bytes * len(copies) < (1 << 30) and len(copies) < 16:
            copies.append(kv.clone())
        out = torch.empty((B, s_q, H, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, s_q, H), dtype=torch.float32, device="cuda")
        ctx.reserve(s_q, H)

        def step(i):
            mla.mla_decode(ctx, q, copies[i % len(copies)], None, lens, scale, out=out, lse=lse,
                           seqlens_host=lens_h)

        s0 = time.perf_counter()
        while time.perf_counter() - s0 < args.settle_s:
            for i in range(10):
                step(i)
            torch.cuda.synchronize()
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / args.steps
        ctx.kernel_times()
        ctx.set_option(mla.MLA_OPT_KERNEL_TIMING, 1)
        for i in range(args.steps):
            step(i)
        split_ms, n_split, comb_ms, n_comb = ctx.kernel_times()
        ctx.set_option(mla.MLA_OPT_KERNEL_TIMING, 0)
        split_us = split_ms * 1e3 / max(1, n_split)
        print(json.dumps({"mode": "sweep", "batch": B, "s_q": s_q, "heads": H, "kv_len": L,
                          "min_chunk": args.min_chunk or "default",
                          "kv_bytes": kv_bytes, "us_per_call": round(us, 2),
                          "GBps": round(kv_bytes / us / 1e3, 1),
                          "split_us": round(split_us, 2),
                          "split_GBps": round(kv_bytes / split_us / 1e3, 1),
                          "split_frac_of_8TBps": round(kv_bytes / split_us / 1e3 / PEAK_HBM_GBS, 4),
                          "combine_us": round(comb_ms * 1e3 / n_comb, 2) if n_comb else 0.0}), flush=True)
        del q, kv, copies, out, lse
        torch.cuda.empty_cache()
    ctx.close()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="untimed steps for this long before the warmup steps (clock ramp)")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="GB/s against context length (bs16, bs32) and head count; one line per point")
    ap.add_argument("--sweep-points", default="",
                    help="restrict the sweep to BxHxL points, comma-separated (e.g. 16x16x512)")
    ap.add_argument("--splits", type=int, default=0, help="key ranges per launch (0: library default)")
    ap.add_argument("--min-chunk", type=int, default=0, help="smallest key range (0: library default)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build runs on a single MI355X "
              "(no collectives); use --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import decode_attention_mla_amd as mla
    import workloads as wl

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(max(1, args.steps))
        return 0
    if args.sweep:
        return sweep(args)

    name = args.workload or wl.HEADLINE
    w = wl.WORKLOADS[name]
    print(f"[bench] generating {name}", file=sys.stderr, flush=True)
    inp = wl.make_inputs(w)
    kv_bytes = inp.kv_bytes
    q, kv, bt, lens = wl.to_torch(inp, "cuda:0")
    # Workloads that fit in the last-level cache rotate over enough copies of
    # the cache to stream from HBM on every step.
    copies = [kv]
    dev_bytes = kv.numel() * 2
    while dev_bytes * len(copies) < (1 << 30) and len(copies) < 16:
        copies.append(kv.clone())
    out = torch.empty((w.batch, w.s_q, w.heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, w.s_q, w.heads), dtype=torch.float32, device="cuda")
    ctx = mla.Context()
    ctx.set_option(mla.MLA_OPT_NUM_SPLITS, args.splits)
    ctx.set_option(mla.MLA_OPT_MIN_CHUNK, args.min_chunk)
    ctx.reserve(w.s_q, w.heads)

    def step(i):
        mla.mla_decode(ctx, q, copies[i % len(copies)], bt, lens, inp.scale, out=out, lse=lse,
                       seqlens_host=inp.seqlens)

    # The GPU's clocks reach their steady state only after some milliseconds
    # of load (input generation leaves it idle for seconds).  Untimed steps
    # run for --settle-s seconds first, then the W warmup steps, so that the
    # K timed steps see the clocks a serving loop runs at.
    settle_steps, s0 = 0, time.perf_counter()
    while time.perf_counter() - s0 < args.settle_s:
        for i in range(10):
            step(i)
        torch.cuda.synchronize()
        settle_steps += 10
    print(f"[bench] settle {settle_steps} steps, warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` calls between two synchronizations.
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    print(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step", file=sys.stderr,
          flush=True)

    # Per-kernel time of the same steps, HIP events on the library's stream.
    ctx.kernel_times()
    ctx.set_option(mla.MLA_OPT_KERNEL_TIMING, 1)
    for i in range(args.steps):
        step(i)
    split_ms, n_split, comb_ms, n_comb = ctx.kernel_times()
    ctx.set_option(mla.MLA_OPT_KERNEL_TIMING, 0)
    split_avg_ms = split_ms / max(1, n_split)
    achieved = kv_bytes / (split_avg_ms * 1e-3) / 1e9
    traffic, traffic_rec = stored_traffic(name)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) bf16, seeded",
        "config": {"workload": name, "batch": w.batch, "s_q": w.s_q, "heads": w.heads,
                   "kv_len": w.seqlen if isinstance(w.seqlen, int) else list(w.seqlen),
                   "layout": "paged%d" % w.page_size if w.page_size else "contiguous",
                   "kv_bytes": kv_bytes, "cache_copies_rotated": len(copies),
                   "splits": args.splits or "default", "min_chunk": args.min_chunk or "default"},
        "roofline": {
            "bound": "hbm",
            "kernel": "mla_split_kernel",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes,
            "split_us_mean": round(split_avg_ms * 1e3, 2),
            "combine_us_mean": round(comb_ms / n_comb * 1e3, 2) if n_comb else 0.0,
            "launches_timed": n_split,
        },
    }
    if traffic_rec is not None and traffic is None:
        res["roofline"]["traffic_note"] = "counters were taken on another kernel source"

    if not args.no_cpu_baseline:
        import oracle

        threads = cpu_threads()
        # The oracle over the whole workload, repeated until about 10 s of
        # CPU time has passed (at least once; bounded by --cpu-seconds).
        print(f"[bench] cpu baseline on {threads} threads", file=sys.stderr, flush=True)
        runs, c0 = 0, time.perf_counter()
        while True:
            ro, rl = oracle.mla_decode(inp.q, inp.kv, inp.block_table, inp.seqlens, inp.scale,
                                       threads=threads)
            runs += 1
            elapsed = time.perf_counter() - c0
            if elapsed >= args.cpu_seconds or elapsed / runs * (runs + 1) > 3 * args.cpu_seconds:
                break
        res["cpu_baseline"] = {
            "value": round(kv_bytes * runs / elapsed / 1e9, 4),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"the whole {name} workload ({kv_bytes} KV bytes, {w.batch * w.s_q * w.heads} "
                      f"rows), fp64, {runs} pass(es) in {elapsed:.2f} s",
        }
        o = out.cpu().numpy().astype(np.float64)
        l = lse.cpu().numpy().astype(np.float64)
        res["parity"] = {
            "against": "fp64 oracle, every output row",
            "o_rmse": float(np.sqrt(np.mean((o - ro) ** 2))),
            "o_maxabs": float(np.max(np.abs(o - ro))),
            "lse_maxabs": float(np.max(np.abs(l - rl))),
        }
    ctx.close()
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
