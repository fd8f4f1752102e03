"""Build the HIP library (gfx950) in-tree: libmoe_prefill.so next to this file."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_prefill.so")
SOURCES = ["moe_prefill.cpp", "quant_kernels.hip", "expert_kernels.hip", "weight_pack.hip",
           "combine_kernels.hip", "plan_kernels.hip", "expert_small_kernels.hip", "plan_scratch.hip"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # the bytes of q8_1 and the epilogue's bits depend on IEEE division and on
    # no implicit contraction: every fused multiply-add is written as fmaf
    "-ffp-contract=off",
    "-fno-fast-math",
    # no packed fp32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    # a launcher declared but not built fails here, not at load time
    "-Wl,--no-undefined",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", *HIPCC_FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
