"""The host-only build's launcher stubs stay in step with the library's
launchers: moe_prefill.cpp and tests/sanitize/host_stubs.cpp link into a
shared library with no undefined symbol. A stub whose signature drifted from
its declaration in internal.h leaves that launcher undefined, and the
sanitizer build of the host side (tests/sanitize/run_host_sanitizers.py)
would then fail to load."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_stubs_link_without_undefined_symbols(tmp_path):
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are not available")
    out = tmp_path / "libmoe_prefill_host.so"
    cmd = ["g++", "-O0", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(ROOT, "quantized_moe_expert_scatter_amd", "csrc", "moe_prefill.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"),
           "-o", str(out), "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
