"""GPU parity on the edge cases of the two encodings, against the oracle and
against hand-worked values.

q8_1 ("Strata" PR #3752, quantize_scatter and swiglu_quant commits: d =
max|x|/127, int8 q rounded from x/d, block sums; the swiglu_quant test feeds
a zero row and a row with one huge value): the hand-worked blocks of
tests/golden/q8_1_blocks.json (d = 1 and d = 2 exactly with ties that round
away from zero, a zero block, a negative largest value, a subnormal d whose
quotient is clamped to 127) go through quantize_scatter, and the same values
arrive as H at swiglu_q8 and at the fused gate/up + swiglu epilogue (gate
values so large that silu(g) = g exactly, up values that make h land on the
ties).

Q2_0 and NL4 weight scales (PR #2145, description: a Q2_0 block's 64 values
share one binary16 scale) at the edges of binary16: subnormal, the smallest
normal, signed zero, negative, and 32752 (twice that is 65504, the largest
binary16, the limit the boundary accepts), through both product kernels (the
matrix-core kernel for experts of many rows and the int8 dot-product kernel
for experts of at most 8 rows).

Every output is compared bit for bit with the oracle; every output buffer
sits between guard bytes that must stay untouched.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle
from quantized_moe_expert_scatter_amd import _lib
from quantized_moe_expert_scatter_amd import workloads as wl
from tests.gpu_common import check_exact, check_h_exact, device_layer, rel_rms, w_tuple

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "q8_1_blocks.json")


def _say(*a):
    print(*a, flush=True)


def _golden_blocks():
    """(name, x float32 [32], d, q int8 [32], s) of every hand-worked block."""
    with open(GOLDEN) as f:
        blocks = json.load(f)["blocks"]
    out = []
    unit = np.float32(2.0 ** -149)               # the smallest binary32 subnormal
    for b in blocks:
        if "x" in b:
            x, d = np.array(b["x"], np.float32), np.float32(b["d"])
        else:                                    # small multiples of it are exact
            x = np.array(b["x_units_of_2^-149"], np.float32) * unit
            d = np.float32(b["d_units_of_2^-149"]) * unit
        out.append((b["name"], x, d, np.array(b["q"], np.int8), int(b["s"])))
    return out


def _oracle_full(L):
    cfg = L.cfg
    return oracle.layer(L.x, L.ids, cfg.n_expert, cfg.n_ff, w_tuple(L.w_gu), w_tuple(L.w_down),
                        n_threads=4)


def _check_block(q, d, s, name, want_q, want_d, want_s):
    assert np.float32(d).view(np.uint32) == np.float32(want_d).view(np.uint32), f"{name}: d {d} != {want_d}"
    assert np.array_equal(q, want_q), f"{name}: q {q} != {want_q}"
    assert s == want_s, f"{name}: s {s} != {want_s}"


# ------------------------------------------------------------- q8_1 of X
def test_quantize_scatter_golden_blocks():
    """Every hand-worked block, at every block position of a 256-value row,
    as given and negated (q and s negate, d stays)."""
    golden = _golden_blocks()
    H, nb = 256, 8
    cfg = wl.small_config("golden_x", 2 * len(golden), H, 128, 4, 2, seed=61)
    L = wl.make_layer(cfg)
    want = {}
    for t in range(cfg.tokens):
        sign = 1 if t < len(golden) else -1
        for b in range(nb):
            g = golden[(t + b) % len(golden)]
            L.x[t, 32 * b:32 * b + 32] = g[1] * np.float32(sign)
            want[t, b] = (g[0], (g[3].astype(np.int16) * sign).astype(np.int8), g[2], g[4] * sign)
    D = device_layer(L)
    D.quantize_scatter()
    xq = D.xq_host()
    perm = D.plan.query()[2]
    _say("case golden q8_1 blocks through quantize_scatter,", xq.shape[0], "rows")
    q, d, s = oracle.unpack_q8_1(xq, H)
    for r in range(xq.shape[0]):
        t = int(perm[r]) // cfg.topk
        for b in range(nb):
            name, wq, wd, ws = want[t, b]
            _check_block(q[r, 32 * b:32 * b + 32], d[r, b], int(s[r, b]), name, wq, wd, ws)
    pl = oracle.plan(L.ids, cfg.n_expert, 64)
    assert np.array_equal(xq, oracle.quantize_scatter(L.x, cfg.topk, pl.perm))
    # the whole chain on these rows still meets the output bar
    D.run()
    ref = _oracle_full(L)
    check_h_exact(D.hq_host(), ref.hq, cfg.n_ff, "golden_x")
    check_exact(D.dm_host(), ref.dm, "golden_x")
    D.close()


# ------------------------------------------------------------ q8_1 of H
G_BIG = np.float32(32.0)     # e^-32 < 2^-25, so 1 + E rounds to 1 and silu(32) = 32 exactly


def test_swiglu_q8_golden_ties():
    """GU rows with g = 32 and u = x / 32 give h = x exactly: the hand-worked
    blocks (except the subnormal one, which x / 32 would not keep) come back as
    their worked q8_1 bytes; a block with g = -100 (e^100 overflows binary32,
    silu(g) = -0) gives a zero block."""
    golden = [g for g in _golden_blocks() if g[2] >= np.float32(2.0 ** -126) or g[2] == 0]
    F = 192                                          # 6 blocks of H per row
    cfg = wl.small_config("golden_h", 40, 256, F, 4, 2, seed=62)
    L = wl.make_layer(cfg)
    D = device_layer(L)
    R = cfg.rows
    gu = np.zeros((R, 2 * F), np.float32)
    want = {}
    rng = np.random.default_rng(5)
    for r in range(R):
        for b in range(F // 32):
            k = (r + b) % (len(golden) + 1)
            if k == len(golden):                     # overflowing exponential
                gu[r, 32 * b:32 * b + 32] = -100.0
                gu[r, F + 32 * b:F + 32 * b + 32] = rng.standard_normal(32).astype(np.float32)
                want[r, b] = ("g = -100", np.zeros(32, np.int8), np.float32(0), 0)
                continue
            name, x, d, q, s = golden[k]
            gu[r, 32 * b:32 * b + 32] = G_BIG
            gu[r, F + 32 * b:F + 32 * b + 32] = x / G_BIG
            want[r, b] = (name, q, d, s)
    D.gu[:R].copy_(torch.from_numpy(gu))
    D.swiglu_q8()
    hq = D.hq_host()
    _say("case golden q8_1 blocks as H through swiglu_q8,", R, "rows")
    q, d, s = oracle.unpack_q8_1(hq, F)
    for r in range(R):
        for b in range(F // 32):
            name, wq, wd, ws = want[r, b]
            _check_block(q[r, 32 * b:32 * b + 32], d[r, b], int(s[r, b]), name, wq, wd, ws)
    assert np.array_equal(hq, oracle.swiglu_q8(gu, F))
    D.close()


def _q2_0_matrix(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Row-major Q2_0 planes of one matrix: codes int [rows, cols] in 0..3,
    scales float16 [rows, cols / 64]."""
    rows, cols = codes.shape
    c = codes.astype(np.uint8).reshape(rows, cols // 64, 4, 16)      # value 16 j + b
    blocks = c[:, :, 0] | (c[:, :, 1] << 2) | (c[:, :, 2] << 4) | (c[:, :, 3] << 6)
    return np.concatenate([blocks.reshape(-1), scales.astype(np.float16).reshape(-1).view(np.uint8)])


def _set_expert(w: wl.ExpertWeights, e: int, data: np.ndarray):
    o = int(w.offsets[e])
    assert data.size == w.per_expert
    w.buf[o:o + data.size] = data


@pytest.mark.parametrize("kernel,tokens,n_expert", [("matrix-core", 300, 2), ("small", 12, 8)])
def test_fused_swiglu_ties_from_weights(kernel, tokens, n_expert):
    """The fused gate/up + swiglu epilogue on exact ties.  Each token row is
    +-127 at value 0 and zero elsewhere (d = 1, q = +-127); gate row j has the
    single weight 0.25 at value 0, so g = +-31.75 (silu(31.75) = 31.75
    exactly); up row j has +-s_j at value 0 with s_j = (2k + 1) / 256, and
    s = 254 / 256 for the first j of each block, so that h / d_h = 128 s_j =
    k + 1/2 exactly: every value of a positive token's H block is a tie."""
    H, F = 256, 128
    cfg = wl.small_config(f"ties_{kernel}", tokens, H, F, n_expert, 1, seed=63)
    L = wl.make_layer(cfg)
    L.x[:] = 0.0
    rng = np.random.default_rng(9)
    L.x[:, 0] = np.where(rng.random(tokens) < 0.8, 127.0, -127.0).astype(np.float32)
    for e in range(n_expert):
        codes = np.full((2 * F, H), 2, np.int64)            # code 2: weight 0
        codes[:, 64:] = rng.integers(0, 4, (2 * F, H - 64))  # met only by zero activations
        codes[:F, 0] = 3                                      # gate: +1 * 0.25
        codes[F:, 0] = np.where(rng.random(F) < 0.5, 3, 1)    # up: +-1 * s_j
        scales = rng.uniform(0.01, 0.05, (2 * F, H // 64)).astype(np.float16)
        scales[:F, 0] = 0.25
        k = rng.integers(0, 127, F)
        s_up = ((2 * k + 1) / 256.0).astype(np.float16)
        s_up[0::32] = 254.0 / 256.0
        scales[F:, 0] = s_up
        _set_expert(L.w_gu, e, _q2_0_matrix(codes, scales))
    D = device_layer(L, chunk_rows=128)
    D.run_fused()
    ref = _oracle_full(L)
    counts = ref.plan.counts
    _say("case", cfg.name, "rows per expert", counts.tolist())
    assert (counts.max() > 8) == (kernel == "matrix-core")
    hq = D.hq_host()
    assert np.array_equal(hq, ref.hq), "fused H bytes"
    # the ties themselves: a positive token's h values are k + 1/2 in units of d_h
    q, _, _ = oracle.unpack_q8_1(hq, F)
    pos = np.nonzero(L.x[ref.plan.perm // cfg.topk, 0] > 0)[0]
    assert pos.size > 0
    for r in pos[:16]:
        e = int(np.searchsorted(ref.plan.offsets, r, side="right") - 1)
        o = int(L.w_gu.offsets[e])
        nblk = 2 * F * (H // 64)
        sc = L.w_gu.buf[o + 16 * nblk:o + 18 * nblk].view(np.float16).reshape(2 * F, H // 64)
        half_units = np.rint(sc[F:, 0].astype(np.float64) * 256.0).astype(np.int64)   # 2k + 1
        sign = np.where(codes_sign(L.w_gu, e, F, H) > 0, 1, -1)
        expect = sign * (half_units + 1) // 2                 # k + 1/2 rounded away from zero
        expect[0::32] = 127 * sign[0::32]
        assert np.array_equal(q[r].astype(np.int64), expect), f"row {r}"
    assert np.array_equal(D.dm_host().view(np.uint32), ref.dm.view(np.uint32)), "dm"
    D.close()


def codes_sign(w: wl.ExpertWeights, e: int, F: int, H: int) -> np.ndarray:
    """Sign (code - 2) of value 0 of every up row of expert e's gate/up matrix."""
    o = int(w.offsets[e])
    nbr = H // 64
    first = w.buf[o:o + 16 * 2 * F * nbr].reshape(2 * F, nbr, 16)[F:, 0, 0]
    return (first & 3).astype(np.int64) - 2


# ------------------------------------------------------ weight-scale edges
EDGE_SCALES = np.array([0x0001, 0x0002, 0x0155, 0x03FF, 0x8001, 0x83FF,  # subnormal
                        0x0400, 0x8400,                                  # smallest normal
                        0x0000, 0x8000,                                  # signed zero
                        0x77FF, 0xF7FF, 0x77FE,                          # +-32752, 32736
                        0x3C00, 0xBC00, 0x2266], np.uint16)              # 1, -1, 0.0125


def _edge_weights(w: wl.ExpertWeights, seed: int):
    """Replace every scale by an edge value (half of them) or keep the drawn one."""
    rng = np.random.default_rng(seed)
    nblk = w.rows * (w.cols // wl.block_of(w.wtype))
    for e in range(w.n_expert):
        o = int(w.offsets[e]) + 16 * nblk
        sc = w.buf[o:o + 2 * nblk].view(np.uint16).copy()
        pick = rng.random(nblk) < 0.5
        sc[pick] = rng.choice(EDGE_SCALES, int(pick.sum()))
        w.buf[o:o + 2 * nblk] = sc.view(np.uint8)


@pytest.mark.parametrize("kernel,tokens,n_expert", [("matrix-core", 300, 2), ("small", 12, 8)])
@pytest.mark.parametrize("down", ["q2_0", "nl4"])
def test_products_at_binary16_scale_edges(kernel, tokens, n_expert, down):
    """Scales that are subnormal, zero, negative or 32752 reach both products
    bit-exact: GU, the int32 block dots, and the down product fed the
    oracle's H; the chain meets the output bar."""
    H, F = 256, 128
    cfg = wl.small_config(f"edge_{kernel}_{down}", tokens, H, F, n_expert, 1, seed=64,
                          down_type=wl.NL4 if down == "nl4" else wl.Q2_0)
    L = wl.make_layer(cfg)
    _edge_weights(L.w_gu, 1)
    _edge_weights(L.w_down, 2)
    ref = _oracle_full(L)
    _say("case", cfg.name, "rows per expert", ref.plan.counts.tolist())
    assert (ref.plan.counts.max() > 8) == (kernel == "matrix-core")
    D = device_layer(L, chunk_rows=128)
    D.run()
    gu = D.gu_host()
    assert np.array_equal(gu.view(np.uint32), ref.gu.view(np.uint32)), \
        f"GU bits: rel RMS {rel_rms(gu, ref.gu):.3e}"
    check_h_exact(D.hq_host(), ref.hq, F, cfg.name)
    check_exact(D.dm_host(), ref.dm, cfg.name)
    # the down product alone on the oracle's H
    D.hq.copy_(torch.from_numpy(ref.hq.reshape(-1).copy()).cuda()[: D.hq.numel()])
    D.expert_down()
    assert np.array_equal(D.dm_host().view(np.uint32), ref.dm.view(np.uint32)), "down on the oracle's H"
    # the int32 block dots of both products (exact whatever the scale)
    row_e = ref.plan.row_expert()
    for product, act, w, rows_out, cols in ((0, ref.xq, L.w_gu, 2 * F, H), (1, ref.hq, L.w_down, H, F)):
        act_dev = torch.from_numpy(act.reshape(-1).copy()).cuda()
        dots = torch.zeros((cfg.rows, rows_out, cols // 32), dtype=torch.int32, device="cuda")
        _lib.moe_debug_block_dots(D.plan, product, act_dev, 0, cfg.rows, dots)
        exp = oracle.block_dots(w.wtype, w.buf, w.offsets, cfg.n_expert, rows_out, cols, w.codebook,
                                act, row_e)
        assert np.array_equal(dots.cpu().numpy(), exp), f"block dots of product {product}"
    D.close()
