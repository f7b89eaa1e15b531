"""CPU checks of bench.py's command line and of the key its stored counters
are filed under (no GPU needed: these paths return before touching one)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_modes():
    r = run_bench("--help")
    assert r.returncode == 0
    for flag in ("--workload", "--sweep", "--mla-steps", "--warm", "--calibrate-copy", "--steps", "--warmup"):
        assert flag in r.stdout


def test_counter_key_ignores_comments(tmp_path, monkeypatch):
    import bench

    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; } // one\n/* block\n comment */ int g;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ("k.hip",))
    a = bench.kernel_source_hash()
    src.write_text("int f() {\n  return 1;  // changed comment\n}\n/* other */ int g;\n")
    assert bench.kernel_source_hash() == a
    src.write_text("int f() { return 2; }\nint g;\n")
    assert bench.kernel_source_hash() != a


def test_stored_traffic_matches_the_current_kernels():
    """The committed counter summaries were taken on the kernel code as it
    stands (else bench.py reports traffic as null)."""
    import bench

    traffic, rec = bench.stored_traffic("mla_bs16_ctx65536")
    assert rec is not None and traffic is not None, "profiles/traffic_* are stale: re-take the counters"


def _counter_csv(path, rows):
    path.mkdir(parents=True, exist_ok=True)
    lines = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    lines += [f"{d},{k},{c},{v}" for d, k, c, v in rows]
    (path / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")


def test_counter_summary_from_raw_output(tmp_path):
    """--collect-counters on stored raw output (no GPU): the copy calibrates
    both byte counters and the bytes per read request, and the split
    kernel's request count is turned into bytes at that size."""
    import json

    copy, split = "__amd_rocclr_copyBuffer", "void mla::mla_split_kernel<0>(mla::Params)"
    gib_kib = 1 << 20
    d = tmp_path / "raw"
    # the passes in the order bench.py runs them: the copy's three, then the workload's five
    _counter_csv(d / "pass1", [(1, copy, "FETCH_SIZE", gib_kib / 2)])
    _counter_csv(d / "pass2", [(1, copy, "WRITE_SIZE", gib_kib)])
    _counter_csv(d / "pass3", [(1, copy, "TCC_EA0_RDREQ_sum", (1 << 30) // 128),
                               (1, copy, "TCC_EA0_RDREQ_32B_sum", 0), (1, copy, "TCC_BUBBLE_sum", 0),
                               (1, copy, "TCC_EA0_RDREQ_DRAM_sum", (1 << 30) // 128)])
    kv = 512 * 1152  # the bs1 ctx512 workload's KV bytes
    # two dispatches of the split kernel: the summary takes their mean
    _counter_csv(d / "pass4", [(1, split, "FETCH_SIZE", kv / 2 / 1024), (2, split, "FETCH_SIZE", kv / 2 / 1024)])
    _counter_csv(d / "pass5", [(1, split, "WRITE_SIZE", 256.0)])
    # 512 keys = 32 blocks of 16 keys, one row block: 50 MFMAs of 16 busy cycles per block
    _counter_csv(d / "pass6", [(1, split, "SQ_INSTS_MFMA", 1600.0), (1, split, "SQ_VALU_MFMA_BUSY_CYCLES", 25600.0),
                               (1, split, "SQ_WAVE_CYCLES", 10000.0), (1, split, "GRBM_GUI_ACTIVE", 8000.0)])
    _counter_csv(d / "pass7", [(1, split, "TCC_EA0_RDREQ_sum", kv // 128 + 10), (1, split, "TCC_EA0_RDREQ_32B_sum", 0),
                               (1, split, "TCC_BUBBLE_sum", 0), (1, split, "TCC_EA0_RDREQ_DRAM_sum", kv // 128)])
    _counter_csv(d / "pass8", [(1, split, "SQ_WAIT_ANY", 2500.0), (1, split, "SQ_INSTS_VALU", 6400.0)])
    prof = tmp_path / "prof"
    r = run_bench("--collect-counters", "mla_bs1_ctx512", "--counters-reuse", "--counters-dir", str(d),
                  "--profiles-out", str(prof))
    assert r.returncode == 0, r.stderr
    rec = json.loads((prof / "traffic_mla_split_mla_bs1_ctx512.json").read_text())
    assert rec["copy_calibration"]["fetch_factor"] == 2.0 and rec["copy_calibration"]["write_factor"] == 1.0
    assert rec["fetch_bytes_per_launch"] == kv and rec["write_bytes_per_launch"] == 256 * 1024
    rq = rec["read_requests"]
    assert rq["bytes_per_request_from_copy"] == 128.0
    assert rq["request_bytes_per_launch"] == kv + 10 * 128
    counters = json.loads((prof / "counters_mla_split_mla_bs1_ctx512.json").read_text())
    assert counters["mfma_busy_pct"] == 100.0 * 25600 / (1024 * 8000 / 8)
    der = counters["derived"]
    assert der["mfma_per_block_per_row_block"] == 50.0 and der["mfma_busy_cycles_per_mfma"] == 16.0
    assert der["valu_insts_per_block_per_row_block"] == 200.0 and der["wait_any_pct_of_wave_cycles"] == 25.0
    md = (prof / "traffic_mla_split_mla_bs1_ctx512.md").read_text()
    assert "128.00 B per request" in md and "TCC_BUBBLE_sum" in md and "SQ_WAIT_ANY" in md
    summary = (prof / "counters_mla_split.md").read_text()
    assert "| MFMA instructions per 16-key block per row block | 50.00 |" in summary
    assert "| waves waiting on counters (SQ_WAIT_ANY), % of wave cycles | 25.00 |" in summary
    assert "| SQ_WAIT_ANY | 2,500 |" in summary


def test_trace_summary_from_raw_output(tmp_path):
    """--trace-summary on a stored kernel_stats.csv (no GPU): one table row
    per kernel and the split kernel's bandwidth from its mean duration."""
    d = tmp_path / "raw" / "trace_mla_bs1_ctx512"
    d.mkdir(parents=True)
    (d / "run_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void mla::mla_split_kernel<0>(mla::Params)",10,100000,10000.0,90.9,9000,12000,100\n'
        '"mla::mla_combine_kernel(mla::Params)",10,10000,1000.0,9.1,900,1200,10\n')
    prof = tmp_path / "prof"
    r = run_bench("--trace-summary", "mla_bs1_ctx512", "--counters-reuse", "--counters-dir",
                  str(tmp_path / "raw"), "--profiles-out", str(prof))
    assert r.returncode == 0, r.stderr
    md = (prof / "mla_split_mla_bs1_ctx512_kernel_trace.md").read_text()
    assert "| void mla::mla_split_kernel<0>(mla::Params) | 10 | 10.00 | 9.00 | 12.00 | 90.9% |" in md
    # 589,824 B in 10 us
    assert "split kernel mean 10.00 us -> 59.0 GB/s" in md


def test_committed_bench_line_is_consistent():
    """The stored default bench line keeps the JSON contract and its own
    arithmetic: value from bytes and step time, the split kernel's achieved
    bandwidth from its bytes and mean time, frac = achieved / peak, and the
    traffic of the counters stored for the current kernels."""
    import json

    import bench

    with open(os.path.join(ROOT, "profiles", "bench_mla_bs16_ctx65536.json")) as f:
        d = json.load(f)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["unit"] == "GB/s" and d["higher_is_better"] is True
    assert d["config"]["workload"] == "mla_bs16_ctx65536"
    kv = d["config"]["kv_bytes"]
    assert abs(d["value"] - kv / (d["ms_per_step"] * 1e3) / 1e3) <= 0.01 * d["value"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert r["algorithmic_bytes_per_launch"] == kv
    assert abs(r["achieved"] - kv / r["split_us_mean"] / 1e3) <= 0.001 * r["achieved"]
    assert abs(r["frac"] - r["achieved"] / r["peak"]) <= 1e-4
    traffic, rec = bench.stored_traffic("mla_bs16_ctx65536")
    assert traffic is not None and r["traffic"] == traffic
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "GB/s" and c["cores"] >= 1 and c["value"] > 0


def test_profile_summaries_name_the_current_kernels():
    """Every stored summary of the attention kernels (traffic, counters,
    kernel traces, sweep) was taken on the kernel source as it stands: the
    source hash each one records matches."""
    import glob
    import re

    import bench

    sha = bench.kernel_source_hash()
    found = 0
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            m = re.search(r"[Kk]ernel source sha256 ([0-9a-f]{16})", f.read())
        if m:
            found += 1
            assert sha.startswith(m.group(1)), f"{os.path.basename(path)} is stale: re-take it"
    assert found >= 16
