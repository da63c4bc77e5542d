"""bench.py's command-line contract, checked on the host (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = run_bench("--gpus", n)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_help_lists_the_contract_flags():
    r = run_bench("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_and_clocks_only_for_the_sources_they_were_taken_on(tmp_path):
    """The counter figures are reported only while the GEMM sources hash to the value
    recorded with them; a changed source, a missing summary or a missing field gives
    None (bench.py then prints null)."""
    bench = _bench_module()
    good = bench.gemm_source_hash()
    traffic = tmp_path / "pmc.txt"
    clocks = tmp_path / "mfma.txt"
    bench.TRAFFIC_SUMMARY, bench.CLOCK_SUMMARY = str(traffic), str(clocks)
    assert bench.recorded_traffic() is None and bench.recorded_clocks() is None  # no summaries

    traffic.write_text(f"# header = ignored\nkernel_source_sha256 = {good}\ntraffic_bytes_per_launch = 1234.5\n")
    clocks.write_text(f"kernel_source_sha256 = {good}\ngate_up_clock_ghz = 1.8\ndown_clock_ghz = 2.0\n")
    assert bench.recorded_traffic() == 1234.5
    assert bench.recorded_clocks() == (1.8, 2.0)

    stale = "0" * 64
    traffic.write_text(f"kernel_source_sha256 = {stale}\ntraffic_bytes_per_launch = 1234.5\n")
    clocks.write_text(f"kernel_source_sha256 = {stale}\ngate_up_clock_ghz = 1.8\ndown_clock_ghz = 2.0\n")
    assert bench.recorded_traffic() is None and bench.recorded_clocks() is None

    traffic.write_text(f"kernel_source_sha256 = {good}\n")
    clocks.write_text(f"kernel_source_sha256 = {good}\ngate_up_clock_ghz = 1.8\n")
    assert bench.recorded_traffic() is None and bench.recorded_clocks() is None


def test_source_hash_covers_every_gemm_source(tmp_path):
    """Changing any file the GEMM kernels are built from changes the hash (on copies
    of the sources in a scratch tree)."""
    import shutil
    bench = _bench_module()
    assert "mixture_experts_ffn_08_amd/csrc/grouped_gemm.hip" in bench.GEMM_SOURCES
    for rel in bench.GEMM_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copyfile(os.path.join(ROOT, rel), dst)
    base = bench.gemm_source_hash()
    bench.ROOT = str(tmp_path)
    assert bench.gemm_source_hash() == base
    for rel in bench.GEMM_SOURCES:
        f = tmp_path / rel
        original = f.read_bytes()
        f.write_bytes(original + b"\n")
        assert bench.gemm_source_hash() != base, rel
        f.write_bytes(original)
    assert bench.gemm_source_hash() == base
