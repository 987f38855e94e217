"""The bench's command-line contract and the counter summary it reads, on
the CPU: more than one GPU is refused with a message, and the measured
traffic is taken from the committed counter summary only while that summary
was made on the current GEMM source (otherwise the bench reports none)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--no-clocks"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_traffic_needs_the_current_gemm_source(tmp_path):
    b = _bench()
    summary = open(b.PROFILE_COUNTERS).read()
    current = tmp_path / "current.txt"      # the committed summary, as if taken on this source
    import re
    current.write_text(re.sub(r"kernel_source_sha256_16:\s*\w+",
                              f"kernel_source_sha256_16: {b.source_hash(b.GEMM_SOURCE)}", summary))
    b.PROFILE_COUNTERS = str(current)
    t = b.measured_traffic(2.476e9)
    assert t is not None and t > 2.476e9
    # a summary of another source, and a missing one, give no figure
    stale = tmp_path / "counters.txt"
    stale.write_text(current.read_text().replace(b.source_hash(b.GEMM_SOURCE), "0000000000000000"))
    b.PROFILE_COUNTERS = str(stale)
    assert b.measured_traffic(2.476e9) is None
    b.PROFILE_COUNTERS = str(tmp_path / "missing.txt")
    assert b.measured_traffic(2.476e9) is None
