"""Shared helpers of the GPU parity tests: device runs through the C ABI and
oracle references on the same seeded inputs."""
from __future__ import annotations

import numpy as np

from oracle import oracle
from quantized_moe_expert_scatter_amd import workloads as wl
from quantized_moe_expert_scatter_amd.layer import DeviceLayer


# guard bytes on each side of every output buffer of a test layer; a layer's
# close() fails if a kernel wrote into them
GUARD = 4096


def device_layer(L: wl.Layer, chunk_rows: int = 64, **kw) -> DeviceLayer:
    return DeviceLayer(L.x, L.ids, L.w_gu, L.w_down, chunk_rows=chunk_rows, route_w=L.route_w,
                       guard=GUARD, **kw)


def w_tuple(w: wl.ExpertWeights):
    return (w.wtype, w.buf, w.offsets, w.codebook)


def oracle_rows(L: wl.Layer, pl: oracle.Plan, rows: np.ndarray, n_threads: int = 8):
    """The oracle's chain for a subset of sorted rows: (xq, gu, hq, dm rows)."""
    cfg = L.cfg
    row_e = pl.row_expert()[rows]
    xq = oracle.quantize_scatter(L.x, cfg.topk, pl.perm, rows=rows)
    gu = oracle.expert_product(*w_tuple(L.w_gu)[:3], cfg.n_expert, 2 * cfg.n_ff, cfg.hidden, L.w_gu.codebook,
                               xq, row_e, n_threads=n_threads)
    hq = oracle.swiglu_q8(gu, cfg.n_ff)
    dm = oracle.expert_product(L.w_down.wtype, L.w_down.buf, L.w_down.offsets, cfg.n_expert,
                               cfg.hidden, cfg.n_ff, L.w_down.codebook, hq, row_e,
                               n_threads=n_threads)
    return xq, gu, hq, dm


def flip_rows(hq_a: np.ndarray, hq_b: np.ndarray) -> np.ndarray:
    """Rows whose q8_1 bytes differ (an int8 rounding of H fell the other way)."""
    return np.nonzero(np.any(hq_a != hq_b, axis=1))[0]


def check_h_exact(hq_gpu: np.ndarray, hq_ref: np.ndarray, n_ff: int, what: str = ""):
    """H bytes equal the oracle's on every row: both sides take E = e^-g
    correctly rounded to binary32 and every quotient correctly rounded, so no
    int8 rounding of H can fall differently.  A mismatch is reported with its
    kind (an H value one int8 step away, as a misrounded E would give, or
    worse)."""
    rows = flip_rows(hq_gpu, hq_ref)
    if rows.size == 0:
        return
    q_g, d_g, s_g = oracle.unpack_q8_1(hq_gpu[rows], n_ff)
    q_o, d_o, s_o = oracle.unpack_q8_1(hq_ref[rows], n_ff)
    dq = np.abs(q_g.astype(np.int64) - q_o.astype(np.int64))
    d_ulps = np.abs(d_g.astype(np.float64) - d_o) / np.maximum(np.spacing(np.abs(d_o)), 1e-300)
    raise AssertionError(f"{what}: H bytes differ on {rows.size} of {hq_ref.shape[0]} rows "
                         f"(first {rows[:4].tolist()}; largest q step {int(dq.max())}, "
                         f"largest d move {float(d_ulps.max()):.1f} ulp)")


def check_exact(a_gpu: np.ndarray, a_ref: np.ndarray, what: str):
    """Bit-exact fp32 outputs (signed zeros included)."""
    assert a_gpu.shape == a_ref.shape, (what, a_gpu.shape, a_ref.shape)
    same = a_gpu.view(np.uint32) == a_ref.view(np.uint32)
    if not same.all():
        bad = np.argwhere(~same)
        raise AssertionError(f"{what}: {bad.shape[0]} values differ (first at {bad[0].tolist()}), "
                             f"rel RMS {rel_rms(a_gpu, a_ref):.3e}")


def row_rel(a: np.ndarray, ref: np.ndarray) -> np.ndarray:
    a = a.astype(np.float64)
    ref = ref.astype(np.float64)
    num = np.sqrt(np.sum((a - ref) ** 2, axis=1))
    den = np.sqrt(np.sum(ref ** 2, axis=1))
    return np.where(den > 0, num / np.maximum(den, 1e-300), num)


def rel_rms(a: np.ndarray, ref: np.ndarray) -> float:
    a = a.astype(np.float64)
    ref = ref.astype(np.float64)
    den = np.sqrt(np.sum(ref ** 2))
    return float(np.sqrt(np.sum((a - ref) ** 2)) / den) if den > 0 else float(np.sqrt(np.sum(a ** 2)))
