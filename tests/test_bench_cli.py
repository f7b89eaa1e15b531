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
