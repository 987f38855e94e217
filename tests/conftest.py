import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="session")
def gemm_kernels_asm(tmp_path_factory):
    """{kernel symbol: [instruction text]} of nvfp4_gemm.hip compiled for
    gfx950 with the library's flags (skipped without hipcc)."""
    hipcc = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
    if hipcc is None:
        pytest.skip("hipcc not available")
    src = os.path.join(ROOT, "nvfp4_w4a4_quantized_05_amd", "csrc", "nvfp4_gemm.hip")
    out = tmp_path_factory.mktemp("asm") / "gemm.s"
    cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-mllvm", "-pragma-unroll-threshold=1000000", "-I", os.path.join(ROOT, "include"),
           "--cuda-device-only", "-S", "-o", str(out), src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kern, kernels = None, {}
    for line in out.read_text().splitlines():
        s = line.strip()
        m = re.match(r"^(_Z\S*):", s)
        if m:
            kern = m.group(1)
            kernels[kern] = []
            continue
        if kern is None or not s or s.startswith((".", ";", "//")) or s.endswith(":"):
            continue
        kernels[kern].append(s.split(";")[0].strip())
    return kernels
