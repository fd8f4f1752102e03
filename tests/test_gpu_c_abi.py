"""The chain driven from plain C through include/moe_prefill.h (no Python or
torch on the path: hipMalloc'd buffers, the default stream), checked against
the C oracle by tests/c_abi/abi_chain.c; built by __graft_entry__.build()."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_chain")


def test_chain_from_c():
    assert os.path.exists(BIN), "tests/c_abi/abi_chain is not built (run __graft_entry__.build())"
    print("case: 64 tokens, hidden 256, n_ff 128, 8 experts, top-2, from C", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("OK")
