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


def check_flips(hq_gpu: np.ndarray, hq_ref: np.ndarray, n_ff: int, max_rows: int) -> np.ndarray:
    """The rows whose H bytes differ, each checked to be an int8 rounding of H
    that fell the other way: in every differing block each q moves by at most
    one, the block sum moves by the sum of those moves, and d is equal or one
    ulp away (the block's largest |h| itself rounded differently).  At most
    max_rows rows may differ.  Returns the differing rows."""
    rows = flip_rows(hq_gpu, hq_ref)
    assert rows.size <= max_rows, f"{rows.size} rows with H bytes differing (bound {max_rows})"
    if rows.size:
        q_g, d_g, s_g = oracle.unpack_q8_1(hq_gpu[rows], n_ff)
        q_o, d_o, s_o = oracle.unpack_q8_1(hq_ref[rows], n_ff)
        dq = q_g.astype(np.int64) - q_o.astype(np.int64)
        assert np.abs(dq).max() <= 1, "an H value moved by more than one int8 step"
        nb = n_ff // 32
        assert np.array_equal(s_g.astype(np.int64) - s_o.astype(np.int64),
                              dq.reshape(rows.size, nb, 32).sum(axis=2)), "block sums inconsistent"
        assert np.all(np.abs(d_g.astype(np.float64) - d_o) <= np.spacing(np.abs(d_o))), \
            "block scale moved by more than one ulp"
    return rows


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


def check_expert_outputs(dm_gpu: np.ndarray, dm_ref: np.ndarray, flips: np.ndarray, what: str):
    """The tolerance rule: rows whose H rounding flipped may reach rel 1e-2;
    all other rows together must reach rel RMS <= 1e-5."""
    mask = np.ones(dm_ref.shape[0], bool)
    mask[flips] = False
    if mask.any():
        e = rel_rms(dm_gpu[mask], dm_ref[mask])
        assert e <= 1e-5, f"{what}: rel RMS {e:.3e} on rows without an H flip"
    if flips.size:
        worst = float(row_rel(dm_gpu[flips], dm_ref[flips]).max())
        assert worst <= 1e-2, f"{what}: flip row rel {worst:.3e}"
