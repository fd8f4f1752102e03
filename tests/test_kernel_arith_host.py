"""Host checks of arithmetic the kernels rely on (CPU only).

* q8_1 rounding in the fused gate/up epilogue: truncating y + 0.49999997
  (the binary32 below 1/2, with y's sign) rounded to binary32 is y rounded
  half away from zero, for every binary32 y in [-127, 127].
* swiglu.cuh: the device functions' own text, compiled for the host, gives
  E = e^-g rounded to the nearest binary32 for every binary32 g (against the
  C library's binary64 exponential and the 80-bit one), and silu_div equals
  the binary32 division g / (1 + E).
"""
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SWIGLU = os.path.join(HERE, "..", "quantized_moe_expert_scatter_amd", "csrc", "swiglu.cuh")


def test_round_half_away_by_binary32_add():
    c = np.nextafter(np.float32(0.5), np.float32(0.0))
    assert c == np.float32(0.49999997)
    top = int(np.float32(127.0).view(np.uint32))
    step = 1 << 24
    for start in range(0, top + 1, step):
        y = np.arange(start, min(start + step, top + 1), dtype=np.uint32).view(np.float32)
        got = np.trunc((y + c).astype(np.float32))          # binary32 add, nearest even
        ref = np.floor(y.astype(np.float64) + 0.5)          # exact in binary64
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, (y[bad[:5]], got[bad[:5]], ref[bad[:5]])
    # adding 1/2 itself is wrong just below 1/2, which is why the constant is below it
    assert np.trunc(np.float32(c) + np.float32(0.5)) == 1.0


def _device_functions() -> str:
    text = open(SWIGLU).read()
    start = text.index("__device__ __forceinline__ float exp_neg_rn32")
    end = text.rindex("}  // namespace moe")
    return text[start:end]


@pytest.fixture(scope="module")
def harness():
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tempfile.mkdtemp(prefix="swiglu_host_")
    with open(os.path.join(d, "swiglu_host.inc"), "w") as f:
        f.write(_device_functions())
    exe = os.path.join(d, "swiglu_arith")
    subprocess.check_call(["g++", "-O2", "-std=c++20", "-ffp-contract=off", "-fopenmp", "-I", d,
                           os.path.join(HERE, "host_checks", "swiglu_arith.cpp"), "-o", exe])
    yield exe
    shutil.rmtree(d, ignore_errors=True)


def test_exp_neg_rn32_every_binary32(harness):
    out = subprocess.run([harness, "exp"], capture_output=True, text=True, timeout=600)
    print(out.stdout)
    assert out.returncode == 0, out.stdout + out.stderr
    n = int(re.search(r"inputs (\d+)", out.stdout).group(1))
    assert n > 2_200_000_000


def test_silu_div_is_the_binary32_division(harness):
    out = subprocess.run([harness, "silu"], capture_output=True, text=True, timeout=600)
    print(out.stdout)
    assert out.returncode == 0, out.stdout + out.stderr
