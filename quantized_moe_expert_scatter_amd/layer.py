"""One MoE layer's routed-expert product on the device: buffers + the four steps.

Plumbing only: torch provides device memory and the stream, the C ABI does
every step of the computation.
"""
from __future__ import annotations

import numpy as np

from . import _lib
from .workloads import ExpertWeights


def _to_device(a: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceLayer:
    """Uploads one layer's weights and inputs, owns every buffer of the path.

    x: float32 [T, hidden]; ids: int32 [T, topk]; w_gu / w_down: ExpertWeights
    (row-major planes; packed here into the kernels' tiled layout).
    Buffers: xq (q8_1 rows of hidden), gu (fp32 [R, 2*n_ff]), hq (q8_1 rows of
    n_ff), dm (fp32 [T*topk, hidden]); R = T*topk.
    guard > 0 (tests): every output buffer sits between two guard regions of
    that many bytes filled with GUARD_BYTE; check_guards() names the buffers
    whose guards were written.
    """

    GUARD_BYTE = 0xA5

    def __init__(self, x: np.ndarray, ids: np.ndarray, w_gu: ExpertWeights, w_down: ExpertWeights,
                 chunk_rows: int = 128, device="cuda", stream=None, route_w: np.ndarray = None,
                 device_plan: bool = False, gu_interleaved: bool = False, guard: int = 0):
        import torch
        self.device = torch.device(device)
        self.guard = (guard + 255) // 256 * 256
        self._guarded = {}
        self.tokens, self.hidden = x.shape
        self.topk = ids.shape[1]
        self.n_expert = w_gu.n_expert
        self.n_ff = w_gu.rows // 2
        self.rows = self.tokens * self.topk
        self.chunk_rows = chunk_rows
        self.x = _to_device(x.astype(np.float32, copy=False), self.device)
        # weights arrive as row-major planes and are packed once into the
        # kernels' tiled layout; the row-major copies are dropped after that
        self.w_gu = self._packed(w_gu, stream, _lib.MOE_W_GU_INTERLEAVED if gu_interleaved else 0)
        self.w_dn = self._packed(w_down, stream)
        u8, f32 = torch.uint8, torch.float32
        ws = _lib.moe_plan_device_bytes(self.tokens, self.topk, self.n_expert, chunk_rows)
        self.workspace = self._buffer("workspace", (max(ws, 16),), u8)
        self.xq = self._buffer("xq", (max(_lib.moe_q8_1_bytes(self.rows, self.hidden), 16),), u8)
        self.gu = self._buffer("gu", (max(self.rows, 1), 2 * self.n_ff), f32)
        self.hq = self._buffer("hq", (max(_lib.moe_q8_1_bytes(self.rows, self.n_ff), 16),), u8)
        self.dm = self._buffer("dm", (max(self.rows, 1), self.hidden), f32)
        # the combine's routing weights [T, topk] and output [T, hidden]
        rw = np.zeros((self.tokens, self.topk), np.float32) if route_w is None else route_w
        self.route_w = _to_device(rw.astype(np.float32, copy=False).reshape(-1)
                                  if rw.size else np.zeros(4, np.float32), self.device)
        self.out = self._buffer("out", (max(self.tokens, 1), self.hidden), f32)
        if device_plan:
            # the routing ids go up first and the plan is built from them on the GPU
            self.ids_dev = _to_device(np.ascontiguousarray(ids, np.int32).reshape(-1)
                                      if ids.size else np.zeros(4, np.int32), self.device)
            self.plan = _lib.moe_prefill_plan_device(self.ids_dev, self.tokens, self.topk,
                                                     self.n_expert, chunk_rows, self.w_gu,
                                                     self.w_dn, self.workspace, stream)
        else:
            self.plan = _lib.moe_prefill_plan(ids, self.n_expert, chunk_rows, self.w_gu, self.w_dn,
                                              workspace=self.workspace, stream=stream)

    def _buffer(self, name: str, shape, dtype):
        """An output buffer; with guards, a view into the middle of a larger
        allocation whose two ends hold GUARD_BYTE."""
        import torch
        if not self.guard:
            return torch.empty(shape, dtype=dtype, device=self.device)
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        g = self.guard
        base = torch.full((g + n + g,), self.GUARD_BYTE, dtype=torch.uint8, device=self.device)
        self._guarded[name] = base
        return base[g:g + n].view(dtype).view(shape)

    def check_guards(self) -> list:
        """Names of the output buffers with a guard byte changed (waits for the device)."""
        import torch
        torch.cuda.synchronize(self.device)
        bad = []
        for name, base in self._guarded.items():
            g = self.guard
            ends = torch.cat([base[:g], base[base.numel() - g:]])
            if not bool(torch.all(ends == self.GUARD_BYTE)):
                bad.append(name)
        return bad

    def _packed(self, w: ExpertWeights, stream, flags: int = 0) -> "_lib.Weights":
        import torch
        raw = _to_device(w.buf, self.device)
        rw = _lib.Weights(w.wtype | flags, w.rows, w.cols, w.n_expert, raw, w.buf.nbytes, w.offsets,
                          w.codebook)
        dst = torch.empty_like(raw)
        packed = _lib.moe_weights_pack(rw, dst, stream)
        torch.cuda.synchronize(self.device)     # the pack has read raw before it is freed
        return packed

    # the four steps, each one kernel launch
    def quantize_scatter(self, stream=None):
        _lib.quantize_scatter(self.plan, self.x, self.xq, stream)

    def expert_gate_up(self, stream=None):
        _lib.expert_gate_up(self.plan, self.xq, self.gu, stream)

    def swiglu_q8(self, stream=None):
        _lib.swiglu_q8(self.plan, self.gu, self.hq, stream)

    def expert_gate_up_swiglu_q8(self, stream=None):
        _lib.expert_gate_up_swiglu_q8(self.plan, self.xq, self.hq, stream)

    def expert_down(self, stream=None):
        _lib.expert_down(self.plan, self.hq, self.dm, stream)

    def combine(self, stream=None):
        _lib.moe_combine(self.plan, self.dm, self.route_w, self.out, stream)

    def run(self, stream=None):
        """The four steps, one launch each (GU materialised)."""
        self.quantize_scatter(stream)
        self.expert_gate_up(stream)
        self.swiglu_q8(stream)
        self.expert_down(stream)

    def run_fused(self, stream=None):
        """The same layer with gate/up, swiglu and q8_1 in one launch (GU never
        stored): three launches, the same xq, hq and dm bytes."""
        self.quantize_scatter(stream)
        self.expert_gate_up_swiglu_q8(stream)
        self.expert_down(stream)

    # host copies
    def xq_host(self) -> np.ndarray:
        rb = self.hidden + self.hidden // 32 * 8
        return self.xq[: self.rows * rb].cpu().numpy().reshape(self.rows, rb)

    def hq_host(self) -> np.ndarray:
        rb = self.n_ff + self.n_ff // 32 * 8
        return self.hq[: self.rows * rb].cpu().numpy().reshape(self.rows, rb)

    def gu_host(self) -> np.ndarray:
        return self.gu[: self.rows].cpu().numpy()

    def dm_host(self) -> np.ndarray:
        return self.dm[: self.rows].cpu().numpy()

    def out_host(self) -> np.ndarray:
        return self.out[: self.tokens].cpu().numpy()

    def close(self):
        """Releases the plan; with guards, raises if a kernel wrote outside a buffer."""
        self.plan.close()
        if self.guard:
            bad = self.check_guards()
            if bad:
                raise AssertionError(f"writes outside the buffers {bad}")
