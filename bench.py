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
(a plain 1 GiB device copy, the reference for the HBM byte counters),
--sweep (context length and head count grid), --mla-steps (the absorbed
query, output projection and cache append around the attention, and a
whole decode step).
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
    """sha256 of the split kernel's sources with comments and blank space
    removed: a change to the code invalidates stored counters, a change to
    a comment does not."""
    import re

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
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


def mla_steps(args) -> int:
    """The MLA steps around the attention at decode sizes, one JSON line
    each: absorbed query, output up-projection, latent-cache append, then
    one whole decode step (absorb, append, attend, project) on the default
    workload.  The projections read each head's weights once per call; the
    weights rotate over copies totalling >= 1 GiB per matrix, as the layers
    of a model would, so every call streams them from HBM.  Algorithmic
    bytes: every input byte read once plus every output byte written once.

    ``us_per_call`` is GPU time: N calls captured in a HIP graph, replayed,
    timed with events on the graph's stream (launch gaps inside the graph
    included, the Python binding's host time excluded).
    ``us_per_call_eager`` times the same calls made one by one from Python,
    where the host side of each call can be the longer part."""
    import torch

    import decode_attention_mla_amd as mla
    import workloads as wl

    B, s_q, H = (int(x) for x in args.step_shape.split(","))
    dn, dv = wl.D_NOPE, wl.D_VHEAD
    rows = B * s_q
    dev = "cuda:0"
    si = wl.make_step_inputs(9000, B, s_q, H)
    ctx = mla.Context()
    stream = torch.cuda.Stream()
    gctx = mla.Context(stream=stream)

    def copies_of(t, limit=2048):
        n = max(1, min(limit, (1 << 30) // (t.numel() * t.element_size())))
        return [t] + [t.clone() for _ in range(n - 1)]

    def settle(fn):
        s0 = time.perf_counter()
        while time.perf_counter() - s0 < args.settle_s:
            for i in range(50):
                fn(ctx, i)
            torch.cuda.synchronize()
        for i in range(args.warmup):
            fn(ctx, i)
        torch.cuda.synchronize()

    def eager(fn, k):
        settle(fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(k):
            fn(ctx, i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / k

    def graphed(fn, n, reps):
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            fn(gctx, 0)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(gctx, i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            s0 = time.perf_counter()  # replays until the clocks settle, as for eager calls
            while True:
                g.replay()
                stream.synchronize()
                if time.perf_counter() - s0 >= args.settle_s:
                    break
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e3 / (n * reps)

    def report(step, us, us_eager, nbytes, extra=None):
        line = {"mode": "mla-steps", "step": step, "batch": B, "s_q": s_q, "heads": H,
                "d_nope": dn, "d_v": dv, "us_per_call": round(us, 3),
                "us_per_call_eager": round(us_eager, 3),
                "algorithmic_bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1),
                "frac_of_8TBps": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}
        line.update(extra or {})
        print(json.dumps(line), flush=True)

    k = max(args.steps, 200)
    qn, qr = wl.bf16_tensor(si.q_nope), wl.bf16_tensor(si.q_rope)
    w_uk = copies_of(wl.bf16_tensor(si.w_uk))
    q_out = torch.empty((rows, H, 576), dtype=torch.bfloat16, device=dev)

    def absorb(c, i):
        mla.mla_absorb_q(c, qn, qr, w_uk[i % len(w_uk)], q_out=q_out)

    us_e = eager(absorb, k)
    report("absorb_q", graphed(absorb, 256, 4), us_e, H * 512 * dn * 2 + rows * H * (dn + 64 + 576) * 2,
           {"weight_copies": len(w_uk)})
    del w_uk

    o = torch.from_numpy(si.o).to(dev)
    w_uv = copies_of(wl.bf16_tensor(si.w_uv))
    out = torch.empty((rows, H, dv), dtype=torch.float32, device=dev)

    def project(c, i):
        mla.mla_project_out(c, o, w_uv[i % len(w_uv)], out=out)

    us_e = eager(project, k)
    report("project_out", graphed(project, 256, 4), us_e, H * dv * 512 * 2 + rows * H * (512 + dv) * 4,
           {"weight_copies": len(w_uv)})
    del w_uv

    # The append and the whole step run on the default workload's cache;
    # its lengths already count the new token, so the append writes the last
    # key of each sequence and the attention reads it.  Device lengths only
    # (as a captured serving loop would pass them).
    w = wl.WORKLOADS[args.workload or wl.HEADLINE]
    assert (w.batch, w.s_q) == (B, s_q) and w.page_size == 0, "step shape must match the workload"
    inp = wl.make_inputs(w)
    q, kv, bt, lens = wl.to_torch(inp, dev)
    new_rows = wl.bf16_tensor(si.new_rows)

    def append(c, i):
        mla.mla_append_kv(c, new_rows, kv, bt, lens)

    us_e = eager(append, k)
    report("append_kv", graphed(append, 256, 4), us_e, 2 * rows * 576 * 2 + B * 4)

    o_lat = torch.empty((B, s_q, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, s_q, H), dtype=torch.float32, device=dev)
    w_uk = copies_of(wl.bf16_tensor(si.w_uk), 64)
    w_uv = copies_of(wl.bf16_tensor(si.w_uv), 64)
    qn4, qr4 = qn.view(B, s_q, H, dn), qr.view(B, s_q, H, 64)
    q_abs = torch.empty((B, s_q, H, 576), dtype=torch.bfloat16, device=dev)
    out4 = out.view(B, s_q, H, dv)
    ctx.reserve(s_q, H)
    gctx.reserve(s_q, H)

    def decode_only(c, i):
        mla.mla_decode(c, q_abs, kv, bt, lens, inp.scale, out=o_lat, lse=lse)

    def whole(c, i):
        mla.mla_absorb_q(c, qn4, qr4, w_uk[i % len(w_uk)], q_out=q_abs)
        mla.mla_append_kv(c, new_rows, kv, bt, lens)
        decode_only(c, i)
        mla.mla_project_out(c, o_lat, w_uv[i % len(w_uv)], out=out4)

    ks = max(args.steps, 20)
    us_dec_e = eager(decode_only, ks)
    us_all_e = eager(whole, ks)
    us_dec = graphed(decode_only, 16, 4)
    us_all = graphed(whole, 16, 4)
    # KV and weights once; per (row, head): q_nope and q_rope read, the
    # absorbed query written and read, the latent output written and read,
    # the projected output written; the appended rows read and written.
    step_bytes = inp.kv_bytes + H * 512 * (dn + dv) * 2 \
        + rows * H * (2 * dn + 2 * 64 + 2 * 576 * 2 + 4 * 512 * 2 + 4 * dv) + 2 * rows * 576 * 2
    report("decode_step", us_all, us_all_e, step_bytes,
           {"workload": w.name, "attention_only_us": round(us_dec, 3),
            "attention_only_us_eager": round(us_dec_e, 3),
            "steps_overhead_us": round(us_all - us_dec, 3)})
    gctx.close()
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
    ap.add_argument("--warm", action="store_true",
                    help="no rotation over cache copies: a cache that fits the 256 MB last-level cache "
                         "stays there between steps (the default streams every step from HBM)")
    ap.add_argument("--sweep", action="store_true",
                    help="GB/s against context length (bs16, bs32) and head count; one line per point")
    ap.add_argument("--sweep-points", default="",
                    help="restrict the sweep to BxHxL points, comma-separated (e.g. 16x16x512)")
    ap.add_argument("--mla-steps", action="store_true",
                    help="time the absorbed query, the output projection, the cache append and a "
                         "whole decode step; one line each")
    ap.add_argument("--step-shape", default="16,1,16", help="B,s_q,H of --mla-steps")
    ap.add_argument("--splits", type=int, default=0, help="key ranges per launch (0: library default)")
    ap.add_argument("--min-chunk", type=int, default=0, help="smallest key range (0: library default)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs on a single MI355X "
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
    if args.mla_steps:
        return mla_steps(args)

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
    while not args.warm and dev_bytes * len(copies) < (1 << 30) and len(copies) < 16:
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
                   "kv_bytes": kv_bytes, "cache_copies_rotated": len(copies), "warm": bool(args.warm),
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
