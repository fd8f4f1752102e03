"""ctypes binding of the C ABI in include/moe_prefill.h (argument marshalling only).

Every function keeps the C name and forwards to libmoe_prefill.so; device
buffers are torch tensors on the current HIP device, host arrays are numpy
arrays.  A non-zero status raises MoeError.  If the library has not been
built, loading raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_PREFILL_LIB names another build of the same library (the host
# sanitizer run in tests/sanitize loads an instrumented one)
LIB_PATH = os.environ.get("MOE_PREFILL_LIB") or os.path.join(HERE, "libmoe_prefill.so")

MOE_W_Q2_0 = 1
MOE_W_NL4 = 2
MOE_W_TILED = 0x100
MOE_W_GU_INTERLEAVED = 0x200

STATUS = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_EALIGN", -3: "MOE_EFORMAT",
          -4: "MOE_ESIZE", -5: "MOE_EHIP", -6: "MOE_ESTATE", -7: "MOE_ENOMEM"}

# every symbol include/moe_prefill.h declares
EXPORTS = ["moe_q8_1_bytes", "moe_weight_bytes", "moe_weights_pack", "moe_plan_device_bytes",
           "moe_prefill_plan", "moe_prefill_plan_device", "moe_prefill_plan_device_noalloc",
           "moe_plan_query", "moe_plan_destroy", "quantize_scatter", "expert_gate_up",
           "swiglu_q8", "expert_gate_up_swiglu_q8", "expert_down", "moe_combine",
           "moe_debug_block_dots",
           "moe_status_string"]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


class moe_weights(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int), ("rows", ctypes.c_int), ("cols", ctypes.c_int),
                ("n_expert", ctypes.c_int), ("base", ctypes.c_void_p),
                ("base_bytes", ctypes.c_size_t), ("offset", ctypes.c_void_p),
                ("codebook", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_q8_1_bytes.argtypes = [I, I]
        L.moe_q8_1_bytes.restype = Z
        L.moe_weight_bytes.argtypes = [I, I, I]
        L.moe_weight_bytes.restype = Z
        L.moe_weights_pack.argtypes = [ctypes.POINTER(moe_weights), P, Z, P]
        L.moe_weights_pack.restype = I
        L.moe_plan_device_bytes.argtypes = [I, I, I, I]
        L.moe_plan_device_bytes.restype = Z
        L.moe_prefill_plan.argtypes = [P, I, I, I, I, ctypes.POINTER(moe_weights),
                                       ctypes.POINTER(moe_weights), P, Z, P, ctypes.POINTER(P)]
        L.moe_prefill_plan.restype = I
        L.moe_prefill_plan_device.argtypes = L.moe_prefill_plan.argtypes
        L.moe_prefill_plan_device.restype = I
        L.moe_prefill_plan_device_noalloc.argtypes = [P, I, I, I, I, ctypes.POINTER(moe_weights),
                                                      ctypes.POINTER(moe_weights), P, ctypes.POINTER(P)]
        L.moe_prefill_plan_device_noalloc.restype = I
        L.moe_plan_query.argtypes = [P, ctypes.POINTER(I), ctypes.POINTER(I), P, P, P, P]
        L.moe_plan_query.restype = I
        L.moe_plan_destroy.argtypes = [P]
        L.moe_plan_destroy.restype = None
        for name in ("quantize_scatter", "expert_gate_up", "swiglu_q8", "expert_gate_up_swiglu_q8",
                     "expert_down"):
            f = getattr(L, name)
            f.argtypes = [P, P, P, P]
            f.restype = I
        L.moe_combine.argtypes = [P, P, P, P, P]
        L.moe_combine.restype = I
        L.moe_debug_block_dots.argtypes = [P, I, P, I, I, P, P]
        L.moe_debug_block_dots.restype = I
        L.moe_status_string.argtypes = [I]
        L.moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(s: int) -> str:
    try:
        return lib().moe_status_string(int(s)).decode()
    except ImportError:
        return STATUS.get(s, "unknown")


def _check(st: int, what: str):
    if st != 0:
        raise MoeError(st, what)


def _ptr(t) -> int | None:
    """Device pointer of a torch tensor (None passes NULL)."""
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


# ------------------------------------------------------------------ sizes
def moe_q8_1_bytes(rows: int, cols: int) -> int:
    return int(lib().moe_q8_1_bytes(rows, cols))


def moe_weight_bytes(wtype: int, rows: int, cols: int) -> int:
    return int(lib().moe_weight_bytes(wtype, rows, cols))


def moe_plan_device_bytes(tokens: int, topk: int, n_expert: int, chunk_rows: int) -> int:
    return int(lib().moe_plan_device_bytes(tokens, topk, n_expert, chunk_rows))


# ------------------------------------------------------------------- plan
class Weights:
    """Keeps a moe_weights struct and the host arrays it points into alive."""

    def __init__(self, wtype: int, rows: int, cols: int, n_expert: int, base, base_bytes: int,
                 offsets: np.ndarray, codebook: np.ndarray | None = None):
        self.offsets = np.ascontiguousarray(offsets, dtype=np.uint64)
        self.codebook = None if codebook is None else np.ascontiguousarray(codebook, dtype=np.int8)
        self.base = base  # keep the device buffer alive
        base_ptr = base if isinstance(base, int) else _ptr(base)
        self.struct = moe_weights(
            wtype, rows, cols, n_expert, base_ptr, base_bytes,
            self.offsets.ctypes.data if self.offsets.size else None,
            None if self.codebook is None else self.codebook.ctypes.data)


def moe_weights_pack(w: Weights, dst, stream=None) -> Weights:
    """Writes the tiled layout of w (row-major planes) into the device tensor
    dst and returns the descriptor of the packed weights (same offsets)."""
    nbytes = dst.numel() * dst.element_size()
    _check(lib().moe_weights_pack(ctypes.byref(w.struct), _ptr(dst), nbytes, _stream(stream)),
           "moe_weights_pack")
    s = w.struct
    return Weights((s.type & ~MOE_W_GU_INTERLEAVED) | MOE_W_TILED, s.rows, s.cols, s.n_expert,
                   dst, nbytes, w.offsets, w.codebook)


class Plan:
    """Owns a moe_plan handle (host object); the device workspace is the
    caller's tensor and is kept alive here."""

    def __init__(self, handle: int, workspace, tokens: int, topk: int, n_expert: int, keep=()):
        self.handle = handle
        self.workspace = workspace
        self.tokens, self.topk, self.n_expert = tokens, topk, n_expert
        self._keep = keep

    def query(self):
        rows, nch = ctypes.c_int(), ctypes.c_int()
        _check(lib().moe_plan_query(self.handle, ctypes.byref(rows), ctypes.byref(nch),
                                    None, None, None, None), "moe_plan_query")
        counts = np.zeros(self.n_expert, np.int32)
        offsets = np.zeros(self.n_expert + 1, np.int32)
        perm = np.zeros(max(rows.value, 1), np.int32)
        chunks = np.zeros((max(nch.value, 1), 4), np.int32)
        _check(lib().moe_plan_query(self.handle, None, None, counts.ctypes.data,
                                    offsets.ctypes.data, perm.ctypes.data, chunks.ctypes.data),
               "moe_plan_query")
        return counts, offsets, perm[:rows.value], chunks[:nch.value]

    def close(self):
        if self.handle:
            lib().moe_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_prefill_plan(ids: np.ndarray, n_expert: int, chunk_rows: int, w_gu: Weights,
                     w_down: Weights, workspace=None, stream=None) -> Plan:
    """ids: host int32 [tokens, topk].  workspace: device uint8 tensor of
    moe_plan_device_bytes(...) bytes, or None for a host-only plan."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    tokens, topk = ids.shape
    h = ctypes.c_void_p()
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().moe_prefill_plan(ids.ctypes.data if ids.size else None, tokens, topk, n_expert,
                                chunk_rows, ctypes.byref(w_gu.struct), ctypes.byref(w_down.struct),
                                ws_ptr, ws_bytes, _stream(stream) if workspace is not None else None,
                                ctypes.byref(h))
    _check(st, "moe_prefill_plan")
    return Plan(h.value, workspace, tokens, topk, n_expert, keep=(w_gu, w_down))


def moe_prefill_plan_device(ids_dev, tokens: int, topk: int, n_expert: int, chunk_rows: int,
                            w_gu: Weights, w_down: Weights, workspace, stream=None) -> Plan:
    """ids_dev: device int32 tensor [tokens, topk] (kept alive with the plan)."""
    h = ctypes.c_void_p()
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().moe_prefill_plan_device(_ptr(ids_dev) if tokens else None, tokens, topk, n_expert,
                                       chunk_rows, ctypes.byref(w_gu.struct),
                                       ctypes.byref(w_down.struct), _ptr(workspace), ws_bytes,
                                       _stream(stream), ctypes.byref(h))
    _check(st, "moe_prefill_plan_device")
    return Plan(h.value, workspace, tokens, topk, n_expert, keep=(w_gu, w_down, ids_dev))


def moe_prefill_plan_device_noalloc(ids_dev, tokens: int, topk: int, n_expert: int, chunk_rows: int,
                                    w_gu: Weights, w_down: Weights, stream=None) -> Plan:
    """The device plan in the library's own per-device workspace: valid until
    the next such call on the device (ids_dev is kept alive with the plan)."""
    h = ctypes.c_void_p()
    st = lib().moe_prefill_plan_device_noalloc(_ptr(ids_dev) if tokens else None, tokens, topk, n_expert,
                                               chunk_rows, ctypes.byref(w_gu.struct),
                                               ctypes.byref(w_down.struct), _stream(stream),
                                               ctypes.byref(h))
    _check(st, "moe_prefill_plan_device_noalloc")
    return Plan(h.value, None, tokens, topk, n_expert, keep=(w_gu, w_down, ids_dev))


# ------------------------------------------------------------------ steps
def quantize_scatter(plan: Plan, x, xq, stream=None):
    _check(lib().quantize_scatter(plan.handle, _ptr(x), _ptr(xq), _stream(stream)), "quantize_scatter")


def expert_gate_up(plan: Plan, xq, gu, stream=None):
    _check(lib().expert_gate_up(plan.handle, _ptr(xq), _ptr(gu), _stream(stream)), "expert_gate_up")


def swiglu_q8(plan: Plan, gu, hq, stream=None):
    _check(lib().swiglu_q8(plan.handle, _ptr(gu), _ptr(hq), _stream(stream)), "swiglu_q8")


def expert_gate_up_swiglu_q8(plan: Plan, xq, hq, stream=None):
    _check(lib().expert_gate_up_swiglu_q8(plan.handle, _ptr(xq), _ptr(hq), _stream(stream)),
           "expert_gate_up_swiglu_q8")


def expert_down(plan: Plan, hq, dm, stream=None):
    _check(lib().expert_down(plan.handle, _ptr(hq), _ptr(dm), _stream(stream)), "expert_down")


def moe_combine(plan: Plan, dm, w, out, stream=None):
    _check(lib().moe_combine(plan.handle, _ptr(dm), _ptr(w), _ptr(out), _stream(stream)), "moe_combine")


def moe_debug_block_dots(plan: Plan, product: int, act, row_begin: int, n_rows: int, dots,
                         stream=None):
    _check(lib().moe_debug_block_dots(plan.handle, product, _ptr(act), row_begin, n_rows,
                                      _ptr(dots), _stream(stream)), "moe_debug_block_dots")
