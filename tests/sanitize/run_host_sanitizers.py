"""Host-side sanitizer run, on the CPU only.

Builds, with gcc/g++ and -fsanitize=address,undefined (no GPU code is
compiled here):
  * the C oracle (oracle/moe_oracle.c), and
  * the host side of the library (csrc/moe_prefill.cpp: argument checks, host
    plans, plan queries, the ABI's exports) linked with host_stubs.cpp in place
    of the device launchers,
into a temporary directory, then runs the CPU tests that exercise them (the
oracle's pins and the host ABI tests) with the sanitizer runtime preloaded and
MOE_ORACLE_LIB / MOE_PREFILL_LIB pointing the loaders at the instrumented
builds.  Any sanitizer report aborts the test process (halt_on_error, no
recovery from undefined behaviour).

    python tests/sanitize/run_host_sanitizers.py
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
TESTS = ["tests/test_oracle_q8_1.py", "tests/test_oracle_weights.py", "tests/test_oracle_products.py",
         "tests/test_oracle_swiglu_plan.py", "tests/test_oracle_combine.py", "tests/test_abi_host.py"]


def main() -> int:
    out = tempfile.mkdtemp(prefix="moe_san_")
    oracle = os.path.join(out, "libmoe_oracle_san.so")
    host = os.path.join(out, "libmoe_prefill_san.so")
    subprocess.check_call(["gcc", "-O1", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", *SAN,
                           os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", oracle, "-lm"])
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__",
                           "-I/opt/rocm/include",
                           os.path.join(ROOT, "quantized_moe_expert_scatter_amd", "csrc", "moe_prefill.cpp"),
                           os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"),
                           "-o", host, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    for lib in (oracle, host):                     # both builds are instrumented
        syms = subprocess.check_output(["nm", "-D", lib], text=True)
        assert "__asan_report_load" in syms and "__ubsan_handle" in syms, lib
    libasan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    libubsan = subprocess.check_output(["gcc", "-print-file-name=libubsan.so"], text=True).strip()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": f"{libasan}:{libubsan}",
        # python itself is not instrumented: its own allocations at exit are not ours
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "MOE_ORACLE_LIB": oracle,
        "MOE_PREFILL_LIB": host,
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *TESTS]
    print(" ".join(cmd), flush=True)
    return subprocess.call(cmd, cwd=ROOT, env=env)


if __name__ == "__main__":
    sys.exit(main())
