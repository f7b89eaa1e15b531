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
import os
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV HBM GB/s (% of peak) + µs/call, MLA decode bs16 ctx64K 16 heads"
PEAK_HBM_GBS = 8000.0
# The split and combine kernels and their launch configuration (the host side
# of the C ABI lives elsewhere and does not change what the counters see).
KERNEL_SOURCES = ("decode_attention_mla_amd/csrc/mla_kernels.hip", "decode_attention_mla_amd/csrc/plan.h",
                  "decode_attention_mla_amd/csrc/launch.h")


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
        # exactly the requested BxHxL points, in the order given
        points = [(b, 1, h, L) for b, h, L in
                  (tuple(int(x) for x in pt.split("x")) for pt in args.sweep_points.split(","))]
    ctx = mla.Context()
    ctx.set_option(mla.MLA_OPT_NUM_SPLITS, args.splits)
    ctx.set_option(mla.MLA_OPT_MIN_CHUNK, args.min_chunk)
    ctx.set_option(mla.MLA_OPT_P_BF16, int(args.p_bf16))
    scale = 1.0 / 24.0
    results = []
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
        res = {"mode": "sweep", "batch": B, "s_q": s_q, "heads": H, "kv_len": L,
               "min_chunk": args.min_chunk or "default",
               "kv_bytes": kv_bytes, "us_per_call": round(us, 2),
               "GBps": round(kv_bytes / us / 1e3, 1),
               "split_us": round(split_us, 2),
               "split_GBps": round(kv_bytes / split_us / 1e3, 1),
               "split_frac_of_8TBps": round(kv_bytes / split_us / 1e3 / PEAK_HBM_GBS, 4),
               "combine_us": round(comb_ms * 1e3 / n_comb, 2) if n_comb else 0.0}
        results.append(res)
        print(json.dumps(res), flush=True)
        del q, kv, copies, out, lse
        torch.cuda.empty_cache()
    ctx.close()
    if not args.sweep_points:
        write_sweep_summary(args, results)
    return 0


def write_sweep_summary(args, results) -> None:
    """profiles/sweep_mla_decode.md from a whole-grid sweep."""
    lines = ["# Sweep: KV bandwidth against context length and head count", "",
             f"Kernel source sha256 {kernel_source_hash()[:16]}..., MI355X (gfx950).  Command:",
             "", "```", f"python3 bench.py --sweep --steps {args.steps} --warmup {args.warmup}"
             + (" --p-bf16" if args.p_bf16 else ""), "```", "",
             "One point = batch x heads x context, one query token, contiguous cache, seeded N(0,1) bf16 inputs "
             f"drawn on the device.  Each point: clocks settled for {args.settle_s:g} s, {args.warmup} warmup steps, "
             f"{args.steps} timed steps (wall clock, `us/call`), then {args.steps} more with HIP events around the "
             "split kernel.  Points under 1 GiB of KV rotate over copies so every step streams from HBM.", "",
             "| batch | heads | context | KV MB | us/call | GB/s (call) | split us | split GB/s | split % of 8 TB/s |",
             "|---|---|---|---|---|---|---|---|---|"]
    for r in results:
        lines.append(f"| {r['batch']} | {r['heads']} | {r['kv_len']} | {r['kv_bytes'] / 1e6:,.1f} | "
                     f"{r['us_per_call']:.2f} | {r['GBps']:,.0f} | {r['split_us']:.2f} | {r['split_GBps']:,.0f} | "
                     f"{100 * r['split_frac_of_8TBps']:.1f}% |")
    os.makedirs(args.profiles_out, exist_ok=True)
    with open(os.path.join(args.profiles_out, "sweep_mla_decode.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


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


# ----------------------------------------------------------- counter passes

SQ_COUNTERS = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES",
               "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE")
# A second pass of eight more (at most eight SQ counters fit in one pass).
SQ_COUNTERS_2 = ("SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                 "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM", "SQ_LDS_ADDR_CONFLICT")
SIMDS = 1024  # 256 CUs x 4 SIMDs
# Raw L2-to-memory read requests, all, 32-byte, 128-byte ("bubble") and
# those sent on to DRAM: FETCH_SIZE is computed from the first three.
TCC_READ_REQUESTS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum", "TCC_EA0_RDREQ_DRAM_sum")


def _rocprof_pass(counters, bench_args, out_dir, timeout_s, reuse=False):
    """One rocprofv3 counter pass over a child bench.py run; returns
    {kernel name: {counter: mean per dispatch}} and the command line.  With
    `reuse`, the raw output already in out_dir is read instead."""
    import csv
    import subprocess

    cmd = ["rocprofv3", "--pmc", *counters, "-f", "csv", "-d", out_dir, "-o", "run", "--",
           sys.executable, os.path.join(ROOT, "bench.py"), *bench_args]
    if not reuse:
        os.makedirs(out_dir, exist_ok=True)
        env = dict(os.environ, TMPDIR="/tmp")
        print(f"[counters] {' '.join(cmd)}", file=sys.stderr, flush=True)
        r = subprocess.run(["timeout", "-s", "KILL", str(timeout_s), *cmd], cwd="/tmp", env=env,
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"counter pass failed ({r.returncode}): {r.stderr[-2000:]}")
    sums, counts = {}, {}
    for root, _, files in os.walk(out_dir):
        for fn in files:
            if not fn.endswith("counter_collection.csv"):
                continue
            with open(os.path.join(root, fn)) as f:
                for row in csv.DictReader(f):
                    k = row["Kernel_Name"]
                    c = row["Counter_Name"]
                    key = (k, c, row.get("Dispatch_Id", ""))
                    sums[key] = sums.get(key, 0.0) + float(row["Counter_Value"])
    per = {}
    for (k, c, _), v in sums.items():
        per.setdefault(k, {}).setdefault(c, []).append(v)
    res = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in per.items()}
    shown = " ".join(cmd).replace(out_dir, "<out>").replace(sys.executable, "python3").replace(ROOT, "/root/repo")
    return res, f"cd /tmp && {shown}"


def _kernel_entry(res, prefix):
    for k, v in res.items():
        if k.lstrip().startswith(prefix) or prefix in k:
            return k, v
    return None, {}


def collect_counters(args) -> int:
    """Counter passes for the split kernel of each named workload, each in a
    run of its own (FETCH_SIZE, WRITE_SIZE, then the SQ counters), plus the
    plain 1 GiB copy that calibrates the byte counters.  Writes
    profiles/traffic_mla_split_<workload>.{json,md} and
    profiles/counters_mla_split_<workload>.json, keyed by the kernel source
    hash so that bench.py uses them only while the kernels are unchanged."""
    import subprocess

    rev = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                         text=True).stdout.strip() or "unknown"
    sha = kernel_source_hash()
    base = os.path.join(args.counters_dir, "pass")
    n_pass = [0]

    def run(counters, bench_args):
        n_pass[0] += 1
        return _rocprof_pass(counters, bench_args, f"{base}{n_pass[0]}", args.counters_timeout,
                             reuse=args.counters_reuse)

    cal_f, cmd_cf = run(["FETCH_SIZE"], ["--calibrate-copy", "--steps", "5"])
    cal_w, cmd_cw = run(["WRITE_SIZE"], ["--calibrate-copy", "--steps", "5"])
    cal_r, cmd_cr = run(list(TCC_READ_REQUESTS), ["--calibrate-copy", "--steps", "5"])
    _, cf = _kernel_entry(cal_f, "copyBuffer")
    _, cw = _kernel_entry(cal_w, "copyBuffer")
    _, cr = _kernel_entry(cal_r, "copyBuffer")
    copy_bytes = 1 << 30
    fetch_factor = copy_bytes / (cf["FETCH_SIZE"] * 1024)
    write_factor = copy_bytes / (cw["WRITE_SIZE"] * 1024)
    # Bytes per read request, measured on the copy (all its requests are of
    # one kind): the size that FETCH_SIZE's expression should have used.
    copy_req = cr.get("TCC_EA0_RDREQ_sum", 0.0)
    req_size = copy_bytes / copy_req if copy_req else None
    counter_recs = []
    for name in args.collect_counters.split(","):
        import workloads as wl

        w = wl.WORKLOADS[name]
        kv_bytes = int(wl.draw_seqlens(w).astype("int64").sum()) * wl.D_QK * 2
        wargs = ["--workload", name, "--settle-s", "0", "--steps", "5", "--warmup", "2", "--no-cpu-baseline"]
        rf, cmd_f = run(["FETCH_SIZE"], wargs)
        rw, cmd_w = run(["WRITE_SIZE"], wargs)
        rs, cmd_s = run(list(SQ_COUNTERS), wargs)
        rr, cmd_r = run(list(TCC_READ_REQUESTS), wargs)
        rs2, cmd_s2 = run(list(SQ_COUNTERS_2), wargs)
        ks, f = _kernel_entry(rf, "mla_split_kernel")
        _, rq = _kernel_entry(rr, "mla_split_kernel")
        _, wv = _kernel_entry(rw, "mla_split_kernel")
        _, sq = _kernel_entry(rs, "mla_split_kernel")
        _, sq2 = _kernel_entry(rs2, "mla_split_kernel")
        kc, fc = _kernel_entry(rf, "mla_combine_kernel")
        _, wc = _kernel_entry(rw, "mla_combine_kernel")
        fetch_b = int(round(f["FETCH_SIZE"] * 1024 * fetch_factor))
        write_b = int(round(wv["WRITE_SIZE"] * 1024 * write_factor))
        cmds = [cmd_f, cmd_cf, cmd_w, cmd_cw]
        rec = {"kernel": "mla_split_kernel", "workload": name, "kernel_source_sha256": sha, "revision": rev,
               "fetch_kib_per_dispatch": f["FETCH_SIZE"], "write_kib_per_dispatch": wv["WRITE_SIZE"],
               "copy_calibration": {"bytes_read": copy_bytes, "bytes_written": copy_bytes,
                                    "fetch_kib": cf["FETCH_SIZE"], "write_kib": cw["WRITE_SIZE"],
                                    "fetch_factor": fetch_factor, "write_factor": write_factor},
               "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
               "bytes_per_launch": fetch_b + write_b, "algorithmic_kv_bytes": kv_bytes,
               "fetch_over_algorithmic": fetch_b / kv_bytes, "commands": cmds}
        if req_size:
            n_req = rq.get("TCC_EA0_RDREQ_sum", 0.0)
            rec["read_requests"] = {
                "counters_per_dispatch": rq, "copy_counters_per_dispatch": cr,
                "bytes_per_request_from_copy": req_size,
                "request_bytes_per_launch": int(round(n_req * req_size)),
                "request_bytes_over_algorithmic": n_req * req_size / kv_bytes,
                "commands": [cmd_r, cmd_cr]}
        if kc:
            rec["combine_kernel"] = {"fetch_bytes": int(round(fc.get("FETCH_SIZE", 0) * 1024 * fetch_factor)),
                                     "write_bytes": int(round(wc.get("WRITE_SIZE", 0) * 1024 * write_factor))}
        prof = args.profiles_out
        os.makedirs(prof, exist_ok=True)
        with open(os.path.join(prof, f"traffic_mla_split_{name}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        busy_cycles = sq.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        gui = sq.get("GRBM_GUI_ACTIVE", 0.0)
        mfma_busy = 100.0 * busy_cycles / (SIMDS * gui / 8) if gui else None
        crec = {"kernel": "mla_split_kernel", "workload": name, "kernel_source_sha256": sha, "revision": rev,
                "counters_per_dispatch": sq, "mfma_busy_pct": mfma_busy,
                "mfma_busy_definition": "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8)",
                "command": cmd_s, "counters_per_dispatch_2": sq2, "command_2": cmd_s2,
                "derived": derived_counters(w, {**sq2, **sq}, mfma_busy)}
        counter_recs.append(crec)
        with open(os.path.join(prof, f"counters_mla_split_{name}.json"), "w") as fh:
            json.dump(crec, fh, indent=1)
            fh.write("\n")
        lines = [f"# HBM traffic: mla_split_kernel, {name}", "",
                 f"Source revision {rev} (kernel source sha256 {sha[:16]}...). Counters in their own runs "
                 "(one counter group per run), written by `bench.py --collect-counters`:", "", "```",
                 *cmds, "```", "",
                 f"Calibration: a plain 1 GiB device copy (`bench.py --calibrate-copy`) reads FETCH_SIZE = "
                 f"{cf['FETCH_SIZE']:,.1f} KiB and WRITE_SIZE = {cw['WRITE_SIZE']:,.1f} KiB per dispatch for "
                 f"1,048,576 KiB moved each way: factors {fetch_factor:.4f} (fetch) and {write_factor:.4f} (write).",
                 "", "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch bytes (calibrated) | write bytes (calibrated) |",
                 "|---|---|---|---|---|",
                 f"| mla_split_kernel | {f['FETCH_SIZE']:,.1f} | {wv['WRITE_SIZE']:,.1f} | {fetch_b:,} | {write_b:,} |"]
        if kc:
            lines.append(f"| mla_combine_kernel | {fc.get('FETCH_SIZE', 0):,.1f} | {wc.get('WRITE_SIZE', 0):,.1f} | "
                         f"{rec['combine_kernel']['fetch_bytes']:,} | {rec['combine_kernel']['write_bytes']:,} |")
        lines += ["", f"Algorithmic KV bytes per split launch: {kv_bytes:,}; fetched / algorithmic = "
                  f"{fetch_b / kv_bytes:.4f}.", ""]
        if "read_requests" in rec:
            rr_ = rec["read_requests"]
            lines += ["Check of the fetch factor with the raw L2-to-memory read requests (one more pass each):", "",
                      "```", cmd_r, cmd_cr, "```", "",
                      "| counter (per dispatch) | mla_split_kernel | 1 GiB copy |", "|---|---|---|"]
            lines += [f"| {c} | {rq.get(c, 0.0):,.0f} | {cr.get(c, 0.0):,.0f} |" for c in TCC_READ_REQUESTS]
            lines += ["", f"The copy reads 1 GiB in {copy_req:,.0f} requests: {req_size:.2f} B per request. "
                      "FETCH_SIZE's expression counts 32 B for a 32-byte request, 128 B for a bubble and 64 B for "
                      f"any other. At {req_size:.2f} B per request the split kernel's requests come to "
                      f"{rr_['request_bytes_per_launch']:,} B per launch, "
                      f"{rr_['request_bytes_over_algorithmic']:.4f} of the algorithmic bytes.", ""]
        lines += ["SQ counters of the split kernel, mean per dispatch (two passes):", "", "```", cmd_s, cmd_s2,
                  "```", "", "| counter | value |", "|---|---|"]
        lines += [f"| {c} | {v:,.0f} |" for c, v in sorted({**sq2, **sq}.items())]
        if mfma_busy is not None:
            lines += ["", f"MFMA busy: {mfma_busy:.2f}% of SIMD time "
                      "(SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8))."]
        with open(os.path.join(prof, f"traffic_mla_split_{name}.md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(json.dumps({"mode": "collect-counters", "workload": name, "fetch_over_algorithmic":
                          round(fetch_b / kv_bytes, 4), "write_bytes": write_b, "mfma_busy_pct":
                          None if mfma_busy is None else round(mfma_busy, 2)}), flush=True)
    write_counter_summary(args, counter_recs, rev, sha)
    return 0


def derived_counters(w, c, mfma_busy):
    """Per-unit figures from one workload's SQ counters (means per dispatch).
    A block is 16 keys of one sequence; a row block is 16 query rows (one
    token, 16 heads), so every block is computed once per row block.  SQ
    wave-cycle counters share one unit, so their ratios are fractions of the
    waves' lifetime."""
    import workloads as wl

    blocks = float(wl.draw_seqlens(w).astype("int64").sum()) / 16
    n_rb = w.s_q * w.heads // 16
    wave = c.get("SQ_WAVE_CYCLES", 0.0)

    def ratio(a, b, scale=1.0):
        return scale * a / b if b else None

    return {
        "blocks_of_16_keys": blocks, "row_blocks": n_rb,
        "mfma_per_block_per_row_block": ratio(c.get("SQ_INSTS_MFMA", 0.0), blocks * n_rb),
        "lds_insts_per_block_per_row_block": ratio(c.get("SQ_INSTS_LDS", 0.0), blocks * n_rb),
        "valu_insts_per_block_per_row_block": ratio(c.get("SQ_INSTS_VALU", 0.0), blocks * n_rb),
        "mfma_busy_cycles_per_mfma": ratio(c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), c.get("SQ_INSTS_MFMA", 0.0)),
        "lds_bank_conflict_cycles_per_block": ratio(c.get("SQ_LDS_BANK_CONFLICT", 0.0), blocks),
        "mfma_busy_pct": mfma_busy,
        "wait_any_pct_of_wave_cycles": ratio(c.get("SQ_WAIT_ANY", 0.0), wave, 100.0),
        "wait_inst_any_pct_of_wave_cycles": ratio(c.get("SQ_WAIT_INST_ANY", 0.0), wave, 100.0),
        "wait_inst_lds_pct_of_wave_cycles": ratio(c.get("SQ_WAIT_INST_LDS", 0.0), wave, 100.0),
        "active_lds_pct_of_wave_cycles": ratio(c.get("SQ_ACTIVE_INST_LDS", 0.0), wave, 100.0),
        "kernel_us_from_grbm_at_2_4_ghz": ratio(c.get("GRBM_GUI_ACTIVE", 0.0), 8 * 2400.0),
    }


DERIVED_ROWS = (
    ("mfma_per_block_per_row_block", "MFMA instructions per 16-key block per row block", "{:.2f}"),
    ("lds_insts_per_block_per_row_block", "LDS instructions per block per row block", "{:.2f}"),
    ("valu_insts_per_block_per_row_block", "VALU instructions per block per row block", "{:.1f}"),
    ("mfma_busy_cycles_per_mfma", "MFMA busy cycles per MFMA", "{:.2f}"),
    ("lds_bank_conflict_cycles_per_block", "LDS bank-conflict cycles per block", "{:.2f}"),
    ("mfma_busy_pct", "MFMA busy, % of SIMD time", "{:.2f}"),
    ("wait_any_pct_of_wave_cycles", "waves waiting on counters (SQ_WAIT_ANY), % of wave cycles", "{:.2f}"),
    ("wait_inst_any_pct_of_wave_cycles", "waves waiting to issue (SQ_WAIT_INST_ANY), % of wave cycles", "{:.2f}"),
    ("wait_inst_lds_pct_of_wave_cycles", "waves waiting to issue LDS (SQ_WAIT_INST_LDS), % of wave cycles",
     "{:.2f}"),
    ("active_lds_pct_of_wave_cycles", "LDS instructions active (SQ_ACTIVE_INST_LDS), % of wave cycles", "{:.2f}"),
    ("kernel_us_from_grbm_at_2_4_ghz", "kernel time from GRBM_GUI_ACTIVE / 8 at 2.4 GHz, us", "{:.2f}"),
)


def write_counter_summary(args, recs, rev, sha) -> None:
    """profiles/counters_mla_split.md: the SQ counters of every workload of
    one --collect-counters run side by side, with per-unit figures."""
    if not recs:
        return
    names = [r["workload"] for r in recs]
    counters = sorted({c for r in recs for c in (*r["counters_per_dispatch"], *r["counters_per_dispatch_2"])})
    lines = ["# SQ counters of mla_split_kernel, by workload", "",
             f"Source revision {rev} (kernel source sha256 {sha[:16]}...), MI355X (gfx950), ROCm 7.2. Written by "
             "`bench.py --collect-counters`; two SQ passes per workload, each in a run of its own:", "", "```"]
    for r in recs:
        lines += [r["command"], r["command_2"]]
    lines += ["```", "", "Mean per dispatch. SQ wave and busy counters tick once per 4 cycles; GRBM_GUI_ACTIVE is "
              "summed over the 8 XCDs.", "", "| counter | " + " | ".join(names) + " |",
              "|---|" + "---|" * len(names)]
    for c in counters:
        vals = []
        for r in recs:
            v = r["counters_per_dispatch"].get(c, r["counters_per_dispatch_2"].get(c))
            vals.append("" if v is None else f"{v:,.0f}")
        lines.append(f"| {c} | " + " | ".join(vals) + " |")
    lines += ["", "Derived (a block is 16 keys; a row block is 16 query rows, so each block is computed once per "
              "row block):", "", "| quantity | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    for key, label, fmt in DERIVED_ROWS:
        vals = [r["derived"].get(key) for r in recs]
        lines.append(f"| {label} | " + " | ".join("" if v is None else fmt.format(v) for v in vals) + " |")
    os.makedirs(args.profiles_out, exist_ok=True)
    with open(os.path.join(args.profiles_out, "counters_mla_split.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def trace_summary(args) -> int:
    """A rocprofv3 kernel trace of bench.py's timed run of each named
    workload (a child run), summarized per kernel into
    profiles/mla_split_<workload>_kernel_trace.md."""
    import csv
    import subprocess

    import workloads as wl

    rev = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                         text=True).stdout.strip() or "unknown"
    sha = kernel_source_hash()
    for name in args.trace_summary.split(","):
        w = wl.WORKLOADS[name]
        kv_bytes = int(wl.draw_seqlens(w).astype("int64").sum()) * wl.D_QK * 2
        # With --p-bf16 the traced run uses MLA_OPT_P_BF16 and the summary
        # is filed under its own name.
        tag = f"{name}_p_bf16" if args.p_bf16 else name
        out_dir = os.path.join(args.counters_dir, f"trace_{tag}")
        cmd = ["rocprofv3", "--kernel-trace", "--stats", "-f", "csv", "-d", out_dir, "-o", "run", "--",
               sys.executable, os.path.join(ROOT, "bench.py"), "--workload", name, "--steps", "20",
               "--warmup", "5", "--no-cpu-baseline", *(["--p-bf16"] if args.p_bf16 else [])]
        if not args.counters_reuse:
            os.makedirs(out_dir, exist_ok=True)
            print(f"[trace] {' '.join(cmd)}", file=sys.stderr, flush=True)
            r = subprocess.run(["timeout", "-s", "KILL", str(args.counters_timeout), *cmd], cwd="/tmp",
                               env=dict(os.environ, TMPDIR="/tmp"), capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"trace run failed ({r.returncode}): {r.stderr[-2000:]}")
        rows = []
        for root, _, files in os.walk(out_dir):
            for fn in files:
                if fn.endswith("kernel_stats.csv"):
                    with open(os.path.join(root, fn)) as f:
                        rows += list(csv.DictReader(f))
        rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
        total = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
        shown = " ".join(cmd).replace(out_dir, "<out>").replace(sys.executable, "python3").replace(ROOT, "/root/repo")
        lines = [f"# Kernel trace: {name}" + (" with MLA_OPT_P_BF16" if args.p_bf16 else ""), "",
                 f"Source revision: {rev} (kernel source sha256 {sha[:16]}...), MI355X (gfx950), ROCm 7.2.", "",
                 "Command:", "", "```", f"cd /tmp && {shown}", "```", "",
                 "Every dispatch of the run is counted: the clock-settling steps (about one second), the warmup, "
                 "the timed steps and the event-timed repeat.", "",
                 "`mla_split_kernel<mode, p_bf16>`: mode 0 one row block per workgroup, 1 two key groups, "
                 "2 one key group of three or four row blocks, 3 one row block that sends the next segment's "
                 "first block before the merge; p_bf16 is MLA_OPT_P_BF16.", "",
                 "| kernel | calls | mean us | min us | max us | share |", "|---|---|---|---|---|---|"]
        split_rows = []
        for r in rows:
            mean = float(r["AverageNs"]) / 1e3
            lines.append(f"| {r['Name']} | {int(r['Calls'])} | {mean:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                         f"{float(r['MaxNs']) / 1e3:.2f} | {100 * float(r['TotalDurationNs']) / total:.1f}% |")
            if "mla_split_kernel" in r["Name"]:
                split_rows.append(mean)
        # One split launch per step covers all the keys once (every workload
        # here launches one instantiation once per step): bytes / its mean.
        if len(split_rows) == 1:
            mean = split_rows[0]
            lines += ["", f"KV bytes per launch (sum of L_b x 1152 B): {kv_bytes:,}; split kernel mean "
                      f"{mean:.2f} us -> {kv_bytes / mean / 1e3:.1f} GB/s "
                      f"({kv_bytes / mean / 1e3 / PEAK_HBM_GBS * 100:.1f}% of 8 TB/s)."]
        os.makedirs(args.profiles_out, exist_ok=True)
        with open(os.path.join(args.profiles_out, f"mla_split_{tag}_kernel_trace.md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(json.dumps({"mode": "trace-summary", "workload": name, "kernels": len(rows)}), flush=True)
    return 0


def stored_mfma_busy(workload: str):
    """MFMA busy % of the split kernel from committed SQ counters taken on
    this exact kernel source, else None."""
    path = os.path.join(ROOT, "profiles", f"counters_mla_split_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("mfma_busy_pct")


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
    ap.add_argument("--p-bf16", action="store_true",
                    help="MLA_OPT_P_BF16: P as one bf16 value in the kernels whose row blocks share key steps "
                         "(faster, each P term within 2^-8 of itself; off by default)")
    ap.add_argument("--collect-counters", default="",
                    help="comma-separated workloads: run the rocprofv3 counter passes of their split kernel "
                         "(each pass a child run) and write profiles/traffic_* and profiles/counters_*")
    ap.add_argument("--counters-dir", default=os.path.join(tempfile.gettempdir(), "mla_decode_counters"),
                    help="where the counter passes write their raw output")
    ap.add_argument("--counters-timeout", type=int, default=300, help="seconds per counter pass")
    ap.add_argument("--counters-reuse", action="store_true",
                    help="read the raw output of earlier counter passes in --counters-dir instead of running them")
    ap.add_argument("--profiles-out", default=os.path.join(ROOT, "profiles"),
                    help="where --collect-counters and --trace-summary write their summaries")
    ap.add_argument("--trace-summary", default="",
                    help="comma-separated workloads: a rocprofv3 kernel trace of each one's bench run "
                         "(a child run), summarized into profiles/mla_split_<workload>_kernel_trace.md")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs on a single MI355X "
              "(no collectives); use --gpus 1.", file=sys.stderr)
        return 2

    # the counter and trace runs are children started in /tmp
    args.counters_dir = os.path.abspath(args.counters_dir)
    args.profiles_out = os.path.abspath(args.profiles_out)
    if args.collect_counters:
        return collect_counters(args)  # before this process touches the GPU
    if args.trace_summary:
        return trace_summary(args)

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
    ctx.set_option(mla.MLA_OPT_P_BF16, int(args.p_bf16))
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
                   "splits": args.splits or "default", "min_chunk": args.min_chunk or "default",
                   "p_bf16": bool(args.p_bf16)},
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
    if traffic is not None and "read_requests" in traffic_rec:
        # the same reads counted as raw requests at the copy's bytes per request
        rq = traffic_rec["read_requests"]
        res["roofline"]["fetch_check"] = {
            "request_bytes_per_launch": rq["request_bytes_per_launch"],
            "bytes_per_request_from_copy": round(rq["bytes_per_request_from_copy"], 2),
            "fetch_bytes_per_launch": traffic_rec["fetch_bytes_per_launch"]}
    busy = stored_mfma_busy(name)
    res["roofline"]["mfma_busy_pct"] = None if busy is None else round(busy, 2)

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
