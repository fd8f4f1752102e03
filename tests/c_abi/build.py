"""Build tests/c_abi/abi_chain: the routed-expert chain driven from plain C
through include/moe_prefill.h and checked against the C oracle.  Test code:
gcc links the library, the oracle and the HIP runtime (host code only)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "abi_chain")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", os.path.join(HERE, "abi_chain.c"), "-o", BIN,
           "-L" + os.path.join(ROOT, "quantized_moe_expert_scatter_amd"), "-lmoe_prefill",
           "-L" + os.path.join(ROOT, "oracle"), "-lmoe_oracle", f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../quantized_moe_expert_scatter_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", f"-Wl,-rpath,{ROCM}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    return BIN


if __name__ == "__main__":
    print(build(verbose=True))
