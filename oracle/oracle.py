"""Python face of the plain CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It takes plain numpy
arrays and imports nothing from the GPU package.

Each function restates one step of the prefill routed-expert product as the
"Strata" pages define it (PR #3752: quantize_scatter, the gate/up product over
all experts, the fused swiglu + q8_1 pass, the down product into one row per
(token, expert); PR #2145: Q2_0 blocks and the exact int32 block sums).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
# MOE_ORACLE_LIB names a prebuilt oracle library (the host sanitizer run in
# tests/sanitize loads an instrumented build); it is then used as it is
LIB_ENV = os.environ.get("MOE_ORACLE_LIB")
LIB = LIB_ENV or os.path.join(HERE, "libmoe_oracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]

Q2_0 = 1
NL4 = 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, fp32, no contraction)."""
    if LIB_ENV:
        return LIB
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.orc_plan.argtypes = [P, I, I, I, I, P, P, P, P, I]
        L.orc_plan.restype = I
        L.orc_q8_1_block.argtypes = [P, P, P, P]
        L.orc_q8_1_row.argtypes = [P, I, P]
        L.orc_quantize_scatter.argtypes = [P, I, I, I, P, I, P, I, P]
        L.orc_decode_row.argtypes = [I, P, I, I, I, P, P, P]
        L.orc_expert_product.argtypes = [I, P, P, I, I, I, P, P, P, I, P]
        L.orc_expert_product.restype = I
        L.orc_block_dots.argtypes = [I, P, P, I, I, I, P, P, P, I, P]
        L.orc_block_dots.restype = I
        L.orc_swiglu.argtypes = [ctypes.c_float, ctypes.c_float]
        L.orc_swiglu.restype = ctypes.c_float
        L.orc_swiglu_q8.argtypes = [P, I, I, I, P]
        L.orc_swiglu_rows.argtypes = [P, I, I, I, P]
        L.orc_combine.argtypes = [P, P, I, I, I, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ plan
@dataclass
class Plan:
    tokens: int
    topk: int
    n_expert: int
    chunk_rows: int
    counts: np.ndarray   # int32 [E]
    offsets: np.ndarray  # int32 [E+1]
    perm: np.ndarray     # int32 [R]: sorted row -> t*K + k
    chunks: np.ndarray   # int32 [n_chunks, 4]: expert, first row, rows, 0

    @property
    def rows(self) -> int:
        return self.tokens * self.topk

    def row_expert(self) -> np.ndarray:
        """Expert of every sorted row."""
        return np.repeat(np.arange(self.n_expert, dtype=np.int32), self.counts)


def plan(ids: np.ndarray, n_expert: int, chunk_rows: int = 64) -> Plan:
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, K = ids.shape
    R = T * K
    counts = np.zeros(n_expert, np.int32)
    offsets = np.zeros(n_expert + 1, np.int32)
    perm = np.zeros(max(R, 1), np.int32)
    max_chunks = R // chunk_rows + n_expert + 1
    chunks = np.zeros((max_chunks, 4), np.int32)
    n = lib().orc_plan(_p(ids), T, K, n_expert, chunk_rows, _p(counts), _p(offsets),
                       _p(perm), _p(chunks), max_chunks)
    if n < 0:
        raise ValueError("routing id out of range")
    return Plan(T, K, n_expert, chunk_rows, counts, offsets, perm[:R].copy(), chunks[:n].copy())


# ------------------------------------------------------------------ q8_1
def q8_1_row_bytes(cols: int) -> int:
    return cols + cols // 32 * 8


def q8_1_block(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape == (32,)
    d = np.zeros(1, np.float32)
    s = np.zeros(1, np.int32)
    q = np.zeros(32, np.int8)
    lib().orc_q8_1_block(_p(x), _p(d), _p(s), _p(q))
    return d[0], int(s[0]), q


def q8_1_rows(x: np.ndarray) -> np.ndarray:
    """q8_1 of every row of x [rows, cols] -> uint8 [rows, row_bytes]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    out = np.zeros((rows, q8_1_row_bytes(cols)), np.uint8)
    for r in range(rows):
        lib().orc_q8_1_row(_p(x[r]), cols, _p(out[r]))
    return out


def unpack_q8_1(buf: np.ndarray, cols: int):
    """Split q8_1 rows into (q int8 [rows, cols], d f32 [rows, nb], s i32 [rows, nb])."""
    buf = np.ascontiguousarray(buf).reshape(-1, q8_1_row_bytes(cols))
    nb = cols // 32
    q = buf[:, :cols].view(np.int8)
    d = buf[:, cols:cols + 4 * nb].copy().view(np.float32)
    s = buf[:, cols + 4 * nb:].copy().view(np.int32)
    return q, d, s


def quantize_scatter(x: np.ndarray, topk: int, perm: np.ndarray, rows=None) -> np.ndarray:
    """Sorted row r <- q8_1 of token perm[r] // topk (rows: optional subset)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, H = x.shape
    perm = np.ascontiguousarray(perm, dtype=np.int32)
    R = perm.shape[0]
    if rows is None:
        out = np.zeros((R, q8_1_row_bytes(H)), np.uint8)
        lib().orc_quantize_scatter(_p(x), T, H, topk, _p(perm), R, None, 0, _p(out))
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        out = np.zeros((rows.shape[0], q8_1_row_bytes(H)), np.uint8)
        lib().orc_quantize_scatter(_p(x), T, H, topk, _p(perm), R, _p(rows), rows.shape[0], _p(out))
    return out


# --------------------------------------------------------------- weights
def decode_row(wtype: int, expert_bytes: np.ndarray, wrows: int, cols: int, n: int, codebook=None):
    eb = np.ascontiguousarray(expert_bytes, dtype=np.uint8)
    vals = np.zeros(cols, np.int8)
    dw = np.zeros(cols // 32, np.float32)
    cb = np.ascontiguousarray(codebook if codebook is not None else np.zeros(16, np.int8), dtype=np.int8)
    lib().orc_decode_row(wtype, _p(eb), wrows, cols, n, _p(cb), _p(vals), _p(dw))
    return vals, dw


def expert_product(wtype: int, w_buf: np.ndarray, w_off: np.ndarray, n_expert: int,
                   wrows: int, cols: int, codebook, act: np.ndarray, act_expert: np.ndarray,
                   n_threads: int = 1) -> np.ndarray:
    """out[i, n] = per-32 epilogue over the int32 block dots of q8_1 row i and
    weight row n of expert act_expert[i].  n_threads > 1 splits the rows over
    threads (ctypes releases the GIL); rows are independent, so the result is
    the same at any thread count."""
    w_buf = np.ascontiguousarray(w_buf, dtype=np.uint8)
    w_off = np.ascontiguousarray(w_off, dtype=np.uint64)
    act = np.ascontiguousarray(act, dtype=np.uint8)
    act_expert = np.ascontiguousarray(act_expert, dtype=np.int32)
    n_act = act_expert.shape[0]
    cb = np.ascontiguousarray(codebook if codebook is not None else np.zeros(16, np.int8), dtype=np.int8)
    out = np.zeros((n_act, wrows), np.float32)

    def run(i0, i1):
        if i1 <= i0:
            return 0
        return lib().orc_expert_product(wtype, _p(w_buf), _p(w_off), n_expert, wrows, cols,
                                        _p(cb), _p(act[i0:i1]), _p(act_expert[i0:i1]), i1 - i0,
                                        _p(out[i0:i1]))

    if n_threads <= 1 or n_act < 2:
        st = run(0, n_act)
    else:
        from concurrent.futures import ThreadPoolExecutor
        bounds = np.linspace(0, n_act, n_threads + 1).astype(int)
        with ThreadPoolExecutor(n_threads) as ex:
            st = min(ex.map(lambda k: run(bounds[k], bounds[k + 1]), range(n_threads)))
    if st != 0:
        raise ValueError("activation row with an expert id out of range")
    return out


def block_dots(wtype: int, w_buf: np.ndarray, w_off: np.ndarray, n_expert: int,
               wrows: int, cols: int, codebook, act: np.ndarray, act_expert: np.ndarray) -> np.ndarray:
    w_buf = np.ascontiguousarray(w_buf, dtype=np.uint8)
    w_off = np.ascontiguousarray(w_off, dtype=np.uint64)
    act = np.ascontiguousarray(act, dtype=np.uint8)
    act_expert = np.ascontiguousarray(act_expert, dtype=np.int32)
    n_act = act_expert.shape[0]
    cb = np.ascontiguousarray(codebook if codebook is not None else np.zeros(16, np.int8), dtype=np.int8)
    dots = np.zeros((n_act, wrows, cols // 32), np.int32)
    st = lib().orc_block_dots(wtype, _p(w_buf), _p(w_off), n_expert, wrows, cols, _p(cb),
                              _p(act), _p(act_expert), n_act, _p(dots))
    if st != 0:
        raise ValueError("activation row with an expert id out of range")
    return dots


# ---------------------------------------------------------------- swiglu
def swiglu(g: float, u: float) -> float:
    return float(lib().orc_swiglu(float(g), float(u)))


def swiglu_rows(gu: np.ndarray, n_ff: int, interleaved: bool = False) -> np.ndarray:
    gu = np.ascontiguousarray(gu, dtype=np.float32)
    rows = gu.shape[0]
    h = np.zeros((rows, n_ff), np.float32)
    lib().orc_swiglu_rows(_p(gu), rows, n_ff, int(interleaved), _p(h))
    return h


def swiglu_q8(gu: np.ndarray, n_ff: int, interleaved: bool = False) -> np.ndarray:
    gu = np.ascontiguousarray(gu, dtype=np.float32)
    rows = gu.shape[0]
    hq = np.zeros((rows, q8_1_row_bytes(n_ff)), np.uint8)
    lib().orc_swiglu_q8(_p(gu), rows, n_ff, int(interleaved), _p(hq))
    return hq


# ----------------------------------------------------------------- layer
@dataclass
class LayerResult:
    plan: Plan
    xq: np.ndarray   # uint8 [R, q8_1 row of hidden], expert-sorted
    gu: np.ndarray   # float32 [R, 2*n_ff], expert-sorted
    hq: np.ndarray   # uint8 [R, q8_1 row of n_ff], expert-sorted
    dm: np.ndarray   # float32 [T*K, hidden], row t*K+k


def combine(dm: np.ndarray, w: np.ndarray) -> np.ndarray:
    """MoE combine (the step after the down product; "Strata" PR #3752 lists
    it among the fusions its port leaves out, without a formula): out[t] =
    sum over k of w[t, k] * dm[t*K + k], one fp32 fmaf per term, k ascending.
    dm: float32 [T*K, H] in (token, slot) order; w: float32 [T, K]."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, K = w.shape
    dm = np.ascontiguousarray(dm, dtype=np.float32).reshape(T * K, -1)
    H = dm.shape[1]
    out = np.zeros((T, H), np.float32)
    if T and H:
        lib().orc_combine(_p(dm), _p(w), T, K, H, _p(out))
    return out


def layer(x, ids, n_expert, n_ff, w_gu, w_down, chunk_rows: int = 64, n_threads: int = 1,
          gu_interleaved: bool = False) -> LayerResult:
    """The whole routed-expert product of one layer, step by step.

    w_gu / w_down: (wtype, buf, offsets, codebook) of the gate/up product
    [2*n_ff, hidden] and the down product [hidden, n_ff].  gu_interleaved:
    the gate/up rows alternate (row 2j gate j, row 2j+1 up j), so GU does too
    and swiglu reads it that way ("Strata" PR #3752, swiglu_quant commit: its
    test covers split and interleaved gate/up rows)."""
    T, H = x.shape
    K = ids.shape[1]
    pl = plan(ids, n_expert, chunk_rows)
    row_e = pl.row_expert()
    xq = quantize_scatter(x, K, pl.perm)
    gu = expert_product(w_gu[0], w_gu[1], w_gu[2], n_expert, 2 * n_ff, H, w_gu[3], xq, row_e,
                        n_threads=n_threads)
    hq = swiglu_q8(gu, n_ff, interleaved=gu_interleaved)
    d_sorted = expert_product(w_down[0], w_down[1], w_down[2], n_expert, H, n_ff, w_down[3], hq,
                              row_e, n_threads=n_threads)
    dm = np.zeros((T * K, H), np.float32)
    dm[pl.perm] = d_sorted
    return LayerResult(pl, xq, gu, hq, dm)
