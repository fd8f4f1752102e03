"""The C ABI on the host (no GPU): exported symbols, size queries, the plan's
host logic against the oracle's plan, and every validation error that can be
forced before any HIP call."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

from oracle import oracle
from quantized_moe_expert_scatter_amd import _lib
from quantized_moe_expert_scatter_amd import workloads as wl
from tests.test_oracle_swiglu_plan import check_plan_invariants

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_prefill.h")
FAKE_BASE = 1 << 20          # an aligned stand-in address: host-only plans never touch it


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_every_declared_symbol_is_exported():
    L = _lib.lib()
    decl = declared_functions()
    assert len(decl) >= 13
    for name in decl:
        assert hasattr(L, name), name
    assert sorted(decl) == sorted(_lib.EXPORTS)


def test_size_queries():
    assert _lib.moe_q8_1_bytes(3, 64) == 3 * 80
    assert _lib.moe_q8_1_bytes(163840, 2560) == 163840 * 3200
    assert _lib.moe_q8_1_bytes(2, 48) == 0
    assert _lib.moe_weight_bytes(1, 1280, 2560) == 921600
    assert _lib.moe_weight_bytes(2, 2560, 640) == 921600
    assert _lib.moe_weight_bytes(1, 2560, 640) == 460800
    assert _lib.moe_weight_bytes(1, 64, 96) == 0
    assert _lib.moe_weight_bytes(3, 64, 64) == 0
    assert _lib.moe_weight_bytes(1 | _lib.MOE_W_TILED, 1280, 2560) == 921600
    assert _lib.moe_plan_device_bytes(64, 2, 8, 64) > 0
    assert _lib.moe_plan_device_bytes(64, 2, 8, 128) > 0
    assert _lib.moe_plan_device_bytes(64, 2, 8, 129) == 0
    assert _lib.moe_plan_device_bytes(-1, 2, 8, 64) == 0
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert _lib.status_string(s)


def _weights(cfg, base=FAKE_BASE, shuffle=False, down_type=None, tiled=True):
    F, H, E = cfg.n_ff, cfg.hidden, cfg.n_expert
    dt = cfg.down_type if down_type is None else down_type
    gu_per = _lib.moe_weight_bytes(1, 2 * F, H)
    dn_per = _lib.moe_weight_bytes(dt, H, F)
    gu_off = np.arange(E, dtype=np.uint64) * np.uint64(gu_per)
    dn_off = np.arange(E, dtype=np.uint64) * np.uint64(dn_per)
    if shuffle:
        gu_off = gu_off[::-1].copy()
    flag = _lib.MOE_W_TILED if tiled else 0
    w_gu = _lib.Weights(1 | flag, 2 * F, H, E, base, gu_per * E, gu_off)
    cb = wl.nl4_codebook(1) if dt == 2 else None
    w_dn = _lib.Weights(dt | flag, H, F, E, base, dn_per * E, dn_off, cb)
    return w_gu, w_dn


@pytest.mark.parametrize("kind,T,E,K,C", [("uniform", 64, 8, 2, 64), ("lognormal", 700, 64, 6, 16),
                                          ("uniform", 33, 16, 4, 1), ("lognormal", 2048, 512, 10, 64)])
def test_host_plan_matches_oracle(kind, T, E, K, C):
    ids = (wl.routing_uniform(T, E, K, seed=T) if kind == "uniform"
           else wl.routing_lognormal(T, E, K, 1.0, seed=T))
    cfg = wl.small_config("p", T, 128, 64, E, K)
    w_gu, w_dn = _weights(cfg)
    plan = _lib.moe_prefill_plan(ids, E, C, w_gu, w_dn, workspace=None)
    counts, offsets, perm, chunks = plan.query()
    ref = oracle.plan(ids, E, C)
    assert np.array_equal(counts, ref.counts)
    assert np.array_equal(offsets, ref.offsets)
    assert np.array_equal(perm, ref.perm)
    assert np.array_equal(chunks, ref.chunks)
    check_plan_invariants(ids, E, C, counts, offsets, perm, chunks)
    plan.close()


def test_empty_plan():
    cfg = wl.small_config("p", 1, 128, 64, 4, 2)
    w_gu, w_dn = _weights(cfg)
    plan = _lib.moe_prefill_plan(np.zeros((0, 2), np.int32), 4, 64, w_gu, w_dn)
    counts, offsets, perm, chunks = plan.query()
    assert counts.tolist() == [0, 0, 0, 0] and perm.size == 0 and chunks.size == 0


def _plan_status(ids, E, C, w_gu, w_dn, ws_ptr=None, ws_bytes=0):
    L = _lib.lib()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    h = ctypes.c_void_p()
    st = L.moe_prefill_plan(ids.ctypes.data, ids.shape[0], ids.shape[1], E, C,
                            ctypes.byref(w_gu.struct), ctypes.byref(w_dn.struct),
                            ws_ptr, ws_bytes, None, ctypes.byref(h))
    if st == 0:
        L.moe_plan_destroy(h.value)
    else:
        assert h.value is None
    return st


def test_validation_errors():
    cfg = wl.small_config("v", 8, 128, 64, 4, 2)
    ids = wl.routing_uniform(8, 4, 2, seed=1)
    good = _weights(cfg)
    assert _plan_status(ids, 4, 64, *good) == 0
    # routing
    assert _plan_status(np.array([[0, 4]]), 4, 64, *good) == -1
    assert _plan_status(np.array([[0, -1]]), 4, 64, *good) == -1
    assert _plan_status(ids, 4, 0, *good) == -1
    assert _plan_status(ids, 4, 129, *good) == -1
    assert _plan_status(ids, 4, 128, *good) == 0
    # weights
    w_gu, w_dn = _weights(cfg)
    w_gu.struct.base = FAKE_BASE + 8
    assert _plan_status(ids, 4, 64, w_gu, w_dn) == -2
    w_gu, w_dn = _weights(cfg)
    w_gu.offsets[1] += 8
    assert _plan_status(ids, 4, 64, w_gu, w_dn) == -2
    w_gu, w_dn = _weights(cfg)
    w_gu.struct.base_bytes -= 16
    assert _plan_status(ids, 4, 64, w_gu, w_dn) == -4
    w_gu, w_dn = _weights(cfg)
    w_gu.struct.type = 3
    assert _plan_status(ids, 4, 64, w_gu, w_dn) == -3
    for which in (0, 1):                       # the kernels read only the tiled layout
        ws = list(_weights(cfg))
        ws[which].struct.type &= ~_lib.MOE_W_TILED
        assert _plan_status(ids, 4, 64, *ws) == -3
    ws = list(_weights(cfg))                   # alternating gate/up rows must be packed first
    ws[0].struct.type |= _lib.MOE_W_GU_INTERLEAVED
    assert _plan_status(ids, 4, 64, *ws) == -3
    w_gu, w_dn = _weights(cfg)
    w_gu.struct.type = 2 | _lib.MOE_W_TILED    # NL4 gate/up needs its codebook
    assert _plan_status(ids, 4, 64, w_gu, w_dn) == -1
    w_gu.codebook = wl.nl4_codebook(5)
    w_gu.struct.codebook = w_gu.codebook.ctypes.data
    assert _plan_status(ids, 4, 64, w_gu, w_dn) == -4   # NL4 matrices are twice as large
    w_gu.struct.base_bytes *= 2
    assert _plan_status(ids, 4, 64, w_gu, w_dn) == 0
    w_gu, w_dn = _weights(cfg)
    w_gu.struct.cols = 96                      # not a multiple of 64 for Q2_0
    w_dn.struct.rows = 96
    assert _plan_status(ids, 4, 64, w_gu, w_dn) == -3
    w_gu, w_dn = _weights(cfg)
    w_dn.struct.rows = 64                      # down rows must equal hidden
    assert _plan_status(ids, 4, 64, w_gu, w_dn) == -1
    w_gu, w_dn = _weights(cfg, down_type=2)
    assert _plan_status(ids, 4, 64, w_gu, w_dn) == 0
    w_dn.struct.codebook = None
    assert _plan_status(ids, 4, 64, w_gu, w_dn) == -1
    w_gu, w_dn = _weights(cfg)
    w_gu.struct.n_expert = 5
    assert _plan_status(ids, 4, 64, w_gu, w_dn) == -1
    w_gu, w_dn = _weights(cfg)
    w_gu.struct.base = None
    assert _plan_status(ids, 4, 64, w_gu, w_dn) == -1
    # device workspace: misaligned, too small (rejected before any HIP call)
    need = _lib.moe_plan_device_bytes(8, 2, 4, 64)
    assert _plan_status(ids, 4, 64, *good, ws_ptr=FAKE_BASE + 4, ws_bytes=need) == -2
    assert _plan_status(ids, 4, 64, *good, ws_ptr=FAKE_BASE, ws_bytes=need - 16) == -4


def test_host_only_plan_refuses_kernels():
    cfg = wl.small_config("v", 8, 128, 64, 4, 2)
    ids = wl.routing_uniform(8, 4, 2, seed=1)
    plan = _lib.moe_prefill_plan(ids, 4, 64, *_weights(cfg))
    L = _lib.lib()
    for f in (L.quantize_scatter, L.expert_gate_up, L.swiglu_q8, L.expert_gate_up_swiglu_q8,
              L.expert_down):
        assert f(plan.handle, FAKE_BASE, FAKE_BASE, None) == -6
        assert f(None, FAKE_BASE, FAKE_BASE, None) == -1
    assert L.moe_combine(plan.handle, FAKE_BASE, FAKE_BASE, FAKE_BASE, None) == -6
    assert L.moe_combine(None, FAKE_BASE, FAKE_BASE, FAKE_BASE, None) == -1
    assert L.moe_debug_block_dots(plan.handle, 0, FAKE_BASE, 0, 1, FAKE_BASE, None) == -6
    assert L.quantize_scatter(None, FAKE_BASE, FAKE_BASE, None) == -1
    with pytest.raises(_lib.MoeError):
        _lib.expert_gate_up(plan, None, None, stream=0)


def _pack_status(w, dst, dst_bytes):
    return _lib.lib().moe_weights_pack(ctypes.byref(w.struct) if w is not None else None, dst,
                                       dst_bytes, None)


def test_pack_validation_errors():
    """moe_weights_pack refuses, before any HIP call, every descriptor and
    destination it cannot pack."""
    cfg = wl.small_config("v", 8, 128, 64, 4, 2)
    DST = 1 << 36                                # another stand-in, far from FAKE_BASE
    w_gu, w_dn = _weights(cfg, tiled=False)
    size = w_gu.struct.base_bytes
    assert _pack_status(None, DST, size) == -1
    assert _pack_status(w_gu, None, size) == -1
    assert _pack_status(w_gu, DST + 8, size) == -2
    assert _pack_status(w_gu, DST, size - 16) == -4
    assert _pack_status(w_gu, FAKE_BASE + 64, size) == -1      # overlaps the source
    t_gu, _ = _weights(cfg, tiled=True)
    assert _pack_status(t_gu, DST, size) == -3                  # already tiled
    w_gu.struct.type = 3
    assert _pack_status(w_gu, DST, size) == -3
    w_gu, _ = _weights(cfg, tiled=False)
    w_gu.struct.rows = 96                                       # not a multiple of 64
    assert _pack_status(w_gu, DST, size) == -3
    w_gu, _ = _weights(cfg, tiled=False)
    w_gu.offsets[1] = w_gu.offsets[0] + np.uint64(16)           # experts overlap partly
    assert _pack_status(w_gu, DST, size) == -1
    w_gu, _ = _weights(cfg, tiled=False)
    w_gu.offsets[1] += np.uint64(8)
    assert _pack_status(w_gu, DST, size) == -2
    _, w_dn = _weights(cfg, tiled=False, down_type=2)
    w_dn.struct.codebook = None
    assert _pack_status(w_dn, DST, w_dn.struct.base_bytes) == -1
    # one expert's matrix must stay below 2^31 bytes (32-bit offsets inside an
    # expert); just below, the descriptor passes and the small destination is
    # what is refused
    for cols, want in ((131072, -1), (114688, -4)):
        per = _lib.moe_weight_bytes(1, 65536, cols)
        assert (per >= 1 << 31) == (want == -1)
        big = _lib.Weights(1, 65536, cols, 1, FAKE_BASE, per, np.zeros(1, dtype=np.uint64))
        assert _pack_status(big, DST, 16) == want


def test_device_plan_validation_errors():
    """moe_prefill_plan_device refuses, before any HIP call, what it can check
    on the host (its routing ids are device memory, checked on the device)."""
    L = _lib.lib()
    cfg = wl.small_config("v", 8, 128, 64, 4, 2)
    w_gu, w_dn = _weights(cfg)
    need = _lib.moe_plan_device_bytes(8, 2, 4, 64)
    DEV_IDS = 1 << 32

    def st(ids=DEV_IDS, T=8, K=2, E=4, C=64, gu=w_gu, dn=w_dn, ws=FAKE_BASE, nb=need):
        h = ctypes.c_void_p()
        r = L.moe_prefill_plan_device(ids, T, K, E, C, ctypes.byref(gu.struct), ctypes.byref(dn.struct),
                                      ws, nb, None, ctypes.byref(h))
        assert h.value is None
        return r

    assert st(ws=None) == -1                      # the device workspace is required
    assert st(ids=None) == -1
    assert st(ids=DEV_IDS + 4) == -2
    assert st(ws=FAKE_BASE + 8) == -2
    assert st(nb=need - 16) == -4
    assert st(C=0) == -1 and st(C=129) == -1 and st(K=0) == -1
    u_gu, _ = _weights(cfg, tiled=False)
    assert st(gu=u_gu) == -3
    assert L.moe_prefill_plan_device(DEV_IDS, 8, 2, 4, 64, ctypes.byref(w_gu.struct),
                                     ctypes.byref(w_dn.struct), FAKE_BASE, need, None, None) == -1
    # the stated limits, each against its neighbour inside the limit, which
    # passes that check and is refused by the later size check (16 bytes):
    # fewer than 2^29 rows (an XCD's rows and index share 32 bits) ...
    assert st(T=(1 << 28), K=2, nb=16) == -1
    assert st(T=(1 << 28) - 1, K=2, nb=16) == -4
    # ... and at most 2048 experts (the schedule's LDS arrays)
    for E, want in ((2049, -1), (2048, -4)):
        e_gu, e_dn = _weights(wl.small_config("v", 8, 128, 64, E, 2))
        assert st(E=E, gu=e_gu, dn=e_dn, nb=16) == want


def test_missing_library_fails_loudly(tmp_path):
    """Without libmoe_prefill.so every entry point raises ImportError: there is
    no fallback of any kind (in a child process, so this process keeps the
    library it has loaded)."""
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import quantized_moe_expert_scatter_amd._lib as L\n"
        "L.LIB_PATH = %r\n"
        "try:\n"
        "    L.moe_q8_1_bytes(4, 64)\n"
        "except ImportError as e:\n"
        "    print('ImportError', e)\n"
        "    sys.exit(0)\n"
        "sys.exit(3)\n" % (ROOT, str(tmp_path / "absent.so")))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "is missing" in r.stdout


def test_every_status_has_a_name_and_a_message():
    """Each status the header declares is named by the binding and described
    by moe_status_string (out-of-memory included: the allocating entry points
    return it instead of letting an exception cross the C boundary)."""
    with open(HEADER) as f:
        text = f.read()
    declared = {int(v): n for n, v in re.findall(r"\b(MOE_(?:OK|E[A-Z]+))\s*=\s*(-?\d+)", text)}
    assert declared[-7] == "MOE_ENOMEM"
    assert _lib.STATUS == declared
    L = _lib.lib()
    for code in declared:
        assert L.moe_status_string(code).decode() != "unknown status", code
    assert L.moe_status_string(-99).decode() == "unknown status"
