"""GPU parity of the HIP path against the oracle, through the C ABI.

Bars (the contract of the prefill routed-expert product):
  * q8_1 bytes (d, s, q of every block) bit-exact: Xq from quantize_scatter,
    Hq from swiglu_q8 and from the fused gate/up epilogue (both sides take
    E = e^-g correctly rounded to binary32, and every quotient correctly
    rounded);
  * int32 block dots bit-exact (moe_debug_block_dots);
  * GU and the expert outputs bit-exact: the kernels follow the oracle's
    epilogue operation for operation (the down product is also checked
    alone on the oracle's H).
Small cases compare every element; the full layers (2k, 8k lognormal, 16k,
t128 with NL4 down) run in the launch configuration of the benchmark and
compare sampled rows the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from quantized_moe_expert_scatter_amd import _lib
from quantized_moe_expert_scatter_amd import workloads as wl
from quantized_moe_expert_scatter_amd.layer import DeviceLayer
from tests.gpu_common import (GUARD, check_exact, check_h_exact, device_layer, oracle_rows, rel_rms,
                              w_tuple)

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny": wl.CONFIGS["tiny"],
    # several N tiles, a ragged N tile (2*n_ff = 640), a ragged K step (n_ff = 320),
    # chunks of 64 and ragged chunk tails
    "ragged": wl.small_config("ragged", 300, 512, 320, 16, 4, seed=21),
    "ragged_nl4": wl.small_config("ragged_nl4", 97, 512, 224, 8, 3, down_type=wl.NL4, seed=22),
    "lognormal": wl.small_config("lognormal", 400, 256, 128, 32, 6, routing_kind="lognormal", seed=23),
    "one_token": wl.small_config("one_token", 1, 256, 128, 8, 2, seed=24),
    "top1": wl.small_config("top1", 130, 256, 128, 2, 1, seed=25),
    # NL4 gate/up (Q2_0 down), and both products NL4 with about 200 rows per
    # expert so 128-row chunks run 4-, 3-, 2- and 1-tile items
    "nl4_gu": wl.small_config("nl4_gu", 150, 448, 192, 6, 4, gu_type=wl.NL4, seed=26),
    "nl4_both": wl.small_config("nl4_both", 400, 512, 224, 6, 3, gu_type=wl.NL4,
                                down_type=wl.NL4, seed=27),
    # degenerate routings: one expert takes every row (full chunks and a ragged
    # tail of one expert), and every token names every expert (top-k = E)
    "one_expert": wl.small_config("one_expert", 300, 256, 128, 1, 1, seed=28),
    "all_experts": wl.small_config("all_experts", 70, 256, 192, 4, 4, seed=29),
}


def _say(*a):
    print(*a, flush=True)


def _small_layer(name, shuffle=False):
    return wl.make_layer(SMALL[name], shuffle_slots=shuffle)


def _oracle_full(L):
    cfg = L.cfg
    return oracle.layer(L.x, L.ids, cfg.n_expert, cfg.n_ff, w_tuple(L.w_gu), w_tuple(L.w_down),
                        n_threads=8)


@pytest.mark.parametrize("name", list(SMALL))
def test_small_chain_every_element(name):
    _chain_every_element(name, 64)


@pytest.mark.parametrize("name", ["nl4_both", "lognormal", "ragged", "nl4_gu"])
def test_small_chain_128_row_chunks(name):
    """The benchmark's chunk size: items of up to four 32-row tiles."""
    _chain_every_element(name, 128)


def _chain_every_element(name, chunk_rows):
    L = _small_layer(name)
    _say("case", name, "chunk_rows", chunk_rows, L.cfg)
    ref = _oracle_full(L)
    D = device_layer(L, chunk_rows=chunk_rows)
    D.run()
    torch.cuda.synchronize()
    assert np.array_equal(D.xq_host(), ref.xq), "q8_1 bytes of X"
    gu = D.gu_host()
    assert np.array_equal(gu.view(np.uint32), ref.gu.view(np.uint32)), \
        f"GU bits: rel RMS {rel_rms(gu, ref.gu):.3e}"
    check_h_exact(D.hq_host(), ref.hq, L.cfg.n_ff, name)
    check_exact(D.dm_host(), ref.dm, name)
    D.close()


@pytest.mark.parametrize("name", ["tiny", "ragged", "ragged_nl4", "nl4_gu"])
def test_block_dots_bit_exact(name):
    L = _small_layer(name)
    cfg = L.cfg
    _say("case", name)
    ref = _oracle_full(L)
    D = device_layer(L)
    row_e = ref.plan.row_expert()
    R = cfg.rows
    # gate/up on the oracle's xq, down on the oracle's hq
    for product, act, w, rows_out, cols in ((0, ref.xq, L.w_gu, 2 * cfg.n_ff, cfg.hidden),
                                            (1, ref.hq, L.w_down, cfg.hidden, cfg.n_ff)):
        act_dev = torch.from_numpy(act.reshape(-1).copy()).cuda()
        r0, n = (0, R) if R <= 400 else (R // 3, 300)
        dots = torch.zeros((n, rows_out, cols // 32), dtype=torch.int32, device="cuda")
        _lib.moe_debug_block_dots(D.plan, product, act_dev, r0, n, dots)
        torch.cuda.synchronize()
        exp = oracle.block_dots(w.wtype, w.buf, w.offsets, cfg.n_expert, rows_out, cols, w.codebook,
                                act[r0:r0 + n], row_e[r0:r0 + n])
        assert np.array_equal(dots.cpu().numpy(), exp), f"product {product}"
    D.close()


@pytest.mark.parametrize("name", ["ragged", "ragged_nl4", "tiny", "nl4_both"])
def test_swiglu_q8_and_down_alone_on_oracle_inputs(name):
    """swiglu_q8 fed the oracle's GU, and the down product fed the oracle's H
    (each step on its own)."""
    L = _small_layer(name)
    cfg = L.cfg
    _say("case", name)
    ref = _oracle_full(L)
    D = device_layer(L)
    D.gu[: cfg.rows].copy_(torch.from_numpy(ref.gu))
    D.swiglu_q8()
    torch.cuda.synchronize()
    hq = D.hq_host()
    check_h_exact(hq, ref.hq, cfg.n_ff, name)
    hq_dev = torch.from_numpy(ref.hq.reshape(-1).copy()).cuda()
    _lib.expert_down(D.plan, hq_dev, D.dm)
    torch.cuda.synchronize()
    dm = D.dm_host()
    assert np.array_equal(dm.view(np.uint32), ref.dm.view(np.uint32)), \
        f"down alone: rel RMS {rel_rms(dm, ref.dm):.3e}"
    D.close()


@pytest.mark.parametrize("chunk_rows", [1, 16, 37, 64, 100, 128])
def test_schedule_invariance(chunk_rows):
    """Outputs do not depend on the chunk size, the chunk order or where the
    experts lie in memory."""
    L = _small_layer("lognormal")
    Ls = _small_layer("lognormal", shuffle=True)
    _say("chunk_rows", chunk_rows)
    A = device_layer(L, chunk_rows=64)
    A.run()
    B = device_layer(Ls, chunk_rows=chunk_rows)
    B.run()
    torch.cuda.synchronize()
    for a, b in ((A.xq_host(), B.xq_host()), (A.gu_host(), B.gu_host()),
                 (A.hq_host(), B.hq_host()), (A.dm_host(), B.dm_host())):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    A.close()
    B.close()


def test_last_tile_row_steps():
    """Chunks whose last 32-row tile holds 1, 8, 9, 16, 17, 24, 25 or 32 rows,
    behind 0-3 full tiles: the product kernel runs such a tile in steps of 8
    rows (both edges of every step), in the four-launch form and in the fused
    gate/up.  Every element against the oracle."""
    counts = [32 * (na - 1) + m for na in range(1, 5) for m in (1, 8, 9, 16, 17, 24, 25, 32)]
    T = sum(counts)
    cfg = wl.small_config("row_steps", T, 512, 192, len(counts), 1, seed=31)
    L = wl.make_layer(cfg)
    # expert e takes counts[e] tokens, in a seeded token order
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    L.ids = np.random.default_rng(311).permutation(ids).reshape(T, 1)
    _say("case row_steps", counts)
    ref = _oracle_full(L)
    D = device_layer(L, chunk_rows=128)
    D.run()
    torch.cuda.synchronize()
    assert np.array_equal(D.xq_host(), ref.xq), "q8_1 bytes of X"
    gu = D.gu_host()
    assert np.array_equal(gu.view(np.uint32), ref.gu.view(np.uint32)), \
        f"GU bits: rel RMS {rel_rms(gu, ref.gu):.3e}"
    check_h_exact(D.hq_host(), ref.hq, cfg.n_ff, "row_steps")
    check_exact(D.dm_host(), ref.dm, "row_steps")
    D.hq.fill_(0x5A)
    D.dm.fill_(float("nan"))
    D.run_fused()
    torch.cuda.synchronize()
    check_h_exact(D.hq_host(), ref.hq, cfg.n_ff, "row_steps fused")
    check_exact(D.dm_host(), ref.dm, "row_steps fused")
    D.close()


def test_tile_streams():
    """Every chunk at most 64 rows and the layer's own widths (hidden 2560,
    n_ff 640): the down product's items (10 stages) then run several N tiles
    of their chunk as one stream of stages.  Row counts on both edges of every
    8-row step of one and two row tiles; every element against the oracle, in
    the four-launch form and in the fused one."""
    counts = [32 * (na - 1) + m for na in (1, 2) for m in (1, 8, 9, 16, 17, 24, 25, 32)]
    T = sum(counts)
    cfg = wl.small_config("tile_streams", T, 2560, 640, len(counts), 1, seed=32)
    L = wl.make_layer(cfg)
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    L.ids = np.random.default_rng(321).permutation(ids).reshape(T, 1)
    _say("case tile_streams", counts)
    ref = _oracle_full(L)
    D = device_layer(L, chunk_rows=128)
    D.run()
    torch.cuda.synchronize()
    assert np.array_equal(D.xq_host(), ref.xq), "q8_1 bytes of X"
    gu = D.gu_host()
    assert np.array_equal(gu.view(np.uint32), ref.gu.view(np.uint32)), \
        f"GU bits: rel RMS {rel_rms(gu, ref.gu):.3e}"
    check_h_exact(D.hq_host(), ref.hq, cfg.n_ff, "tile_streams")
    check_exact(D.dm_host(), ref.dm, "tile_streams")
    D.hq.fill_(0x5A)
    D.dm.fill_(float("nan"))
    D.run_fused()
    torch.cuda.synchronize()
    check_h_exact(D.hq_host(), ref.hq, cfg.n_ff, "tile_streams fused")
    check_exact(D.dm_host(), ref.dm, "tile_streams fused")
    D.close()


@pytest.mark.parametrize("device_plan", [False, True])
def test_tile_streams_short_groups_and_plans(device_plan):
    """The streams with 64-row chunks cut from experts of up to 150 rows, a
    hidden width of seven down-product tiles (items of five tiles and of two)
    and both the host-built and the device-built plan; every element against
    the oracle."""
    counts = [150, 129, 128, 100, 65, 64, 63, 40, 33, 32, 17, 9, 8, 1]
    T = sum(counts)
    cfg = wl.small_config("tile_streams_1792", T, 1792, 640, len(counts), 1, seed=33)
    L = wl.make_layer(cfg)
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    L.ids = np.random.default_rng(331).permutation(ids).reshape(T, 1)
    _say("case tile_streams_1792 device_plan", device_plan)
    ref = _oracle_full(L)
    D = device_layer(L, chunk_rows=64, device_plan=device_plan)
    D.run()
    torch.cuda.synchronize()
    assert np.array_equal(D.xq_host(), ref.xq), "q8_1 bytes of X"
    gu = D.gu_host()
    assert np.array_equal(gu.view(np.uint32), ref.gu.view(np.uint32)), \
        f"GU bits: rel RMS {rel_rms(gu, ref.gu):.3e}"
    check_h_exact(D.hq_host(), ref.hq, cfg.n_ff, "tile_streams_1792")
    check_exact(D.dm_host(), ref.dm, "tile_streams_1792")
    D.dm.fill_(float("nan"))
    D.run_fused()
    torch.cuda.synchronize()
    check_h_exact(D.hq_host(), ref.hq, cfg.n_ff, "tile_streams_1792 fused")
    check_exact(D.dm_host(), ref.dm, "tile_streams_1792 fused")
    D.close()


def test_deterministic_and_empty():
    L = _small_layer("ragged")
    D = device_layer(L)
    D.run()
    first = D.dm_host().copy()
    D.run()
    torch.cuda.synchronize()
    assert np.array_equal(first.view(np.uint32), D.dm_host().view(np.uint32))
    D.close()
    # zero tokens: every step is a valid no-op
    E = wl.make_layer(wl.small_config("empty", 1, 256, 128, 8, 2, seed=3))
    from quantized_moe_expert_scatter_amd.layer import DeviceLayer
    Z = DeviceLayer(np.zeros((0, 256), np.float32), np.zeros((0, 2), np.int32), E.w_gu, E.w_down,
                    guard=GUARD)
    Z.run()
    torch.cuda.synchronize()
    Z.close()


def test_zero_and_huge_token_rows():
    """A zero token row quantizes to zeros end to end; a token with one huge
    value keeps only that value in its block."""
    cfg = wl.small_config("edge", 20, 256, 128, 4, 2, seed=31)
    L = wl.make_layer(cfg)
    L.x[3] = 0.0
    L.x[7, 40] = 1e4
    ref = _oracle_full(L)
    D = device_layer(L)
    D.run()
    torch.cuda.synchronize()
    assert np.array_equal(D.xq_host(), ref.xq)
    rows3 = np.nonzero(ref.plan.perm // cfg.topk == 3)[0]
    assert np.all(D.xq_host()[rows3] == 0)
    assert np.all(D.dm_host()[ref.plan.perm[rows3]] == 0.0)
    check_h_exact(D.hq_host(), ref.hq, cfg.n_ff, "edge")
    check_exact(D.dm_host(), ref.dm, "edge")
    D.close()


def _fused_equals_two_steps(D):
    """Run the layer both ways on the same buffers; hq and dm must match byte
    for byte (compared on the device)."""
    D.run()
    torch.cuda.synchronize()
    hq_a, dm_a = D.hq.clone(), D.dm.clone()
    D.hq.fill_(0x5A)
    D.dm.fill_(float("nan"))
    D.run_fused()
    torch.cuda.synchronize()
    assert torch.equal(D.hq, hq_a), "fused hq differs from gate_up + swiglu_q8"
    assert torch.equal(D.dm.view(torch.int32), dm_a.view(torch.int32)), "dm after the fused path differs"


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_gate_up_swiglu_matches_two_steps(name):
    """expert_gate_up_swiglu_q8 writes the bytes of expert_gate_up followed by
    swiglu_q8, including n_ff not a multiple of its 128-value tile."""
    L = _small_layer(name)
    _say("case", name)
    D = device_layer(L)
    _fused_equals_two_steps(D)
    D.close()


@pytest.mark.parametrize("name", ["tiny", "ragged", "nl4_both", "top1", "one_token"])
def test_combine(name):
    """moe_combine is bit-exact against the oracle's combine of the same dm,
    and so is the whole chain with the combine."""
    L = _small_layer(name)
    _say("case", name)
    ref = _oracle_full(L)
    D = device_layer(L)
    D.run()
    D.out.fill_(float("nan"))
    D.combine()
    torch.cuda.synchronize()
    out = D.out_host()
    exp = oracle.combine(D.dm_host(), L.route_w)
    assert np.array_equal(out.view(np.uint32), exp.view(np.uint32))
    check_exact(out, oracle.combine(ref.dm, L.route_w), name)
    D.close()


@pytest.mark.parametrize("name", ["tiny", "ragged", "nl4_gu"])
def test_interleaved_gate_up_rows(name):
    """Gate/up weights stored with alternating rows give the bytes of the
    split-stored layer, and match the oracle run on the alternating rows with
    its interleaved swiglu."""
    L = _small_layer(name)
    _say("case", name)
    Li = wl.interleave_gate_up(L.w_gu)
    cfg = L.cfg
    ref = oracle.layer(L.x, L.ids, cfg.n_expert, cfg.n_ff, w_tuple(Li), w_tuple(L.w_down),
                       n_threads=8, gu_interleaved=True)
    A = device_layer(L)
    B = DeviceLayer(L.x, L.ids, Li, L.w_down, chunk_rows=64, route_w=L.route_w, gu_interleaved=True,
                    guard=GUARD)
    for D in (A, B):
        D.run_fused()
    torch.cuda.synchronize()
    assert torch.equal(A.hq, B.hq) and torch.equal(A.dm.view(torch.int32), B.dm.view(torch.int32))
    check_h_exact(B.hq_host(), ref.hq, cfg.n_ff, name)
    check_exact(B.dm_host(), ref.dm, name)
    A.close()
    B.close()


# ------------------------------------------------------------- full layers
FULL = ["2k", "8k", "16k", "t128", "2k_nl4"]


@pytest.mark.parametrize("name", FULL)
def test_full_layer_sampled_rows(name):
    _sampled_rows(wl.CONFIGS[name])


@pytest.mark.parametrize("name", list(wl.SWEEP))
def test_sweep_layer_sampled_rows(name):
    """The rows-per-expert sweep: 768..4096 tokens, lognormal and flat routing."""
    _sampled_rows(wl.SWEEP[name])


def _sampled_rows(cfg):
    name = cfg.name
    _say("case", name, "generating inputs")
    L = wl.make_layer(cfg)
    pl = oracle.plan(L.ids, cfg.n_expert, 64)
    D = device_layer(L, chunk_rows=128)          # the benchmark's launch configuration
    D.run()
    torch.cuda.synchronize()
    _say("device run done")
    rng = np.random.default_rng(7)
    # rows of the largest and the smallest expert plus a random spread
    big = int(np.argmax(pl.counts))
    small = int(np.argmin(np.where(pl.counts > 0, pl.counts, 1 << 30)))
    rows = np.unique(np.concatenate([
        rng.choice(cfg.rows, 96, replace=False),
        np.arange(pl.offsets[big], min(pl.offsets[big] + 16, pl.offsets[big + 1])),
        np.arange(pl.offsets[small], pl.offsets[small + 1])[:8],
        [0, cfg.rows - 1]])).astype(np.int32)
    xq, gu, hq, dm = oracle_rows(L, pl, rows)
    _say("oracle rows done", rows.size)
    # quantize_scatter: bit-exact on the sample, and every row is a copy of its token's row
    xq_dev = D.xq_host()
    assert np.array_equal(xq_dev[rows], xq)
    gu_dev = D.gu_host()[rows]
    assert np.array_equal(gu_dev.view(np.uint32), gu.view(np.uint32)), \
        f"GU bits: rel RMS {rel_rms(gu_dev, gu):.3e}"
    check_h_exact(D.hq_host()[rows], hq, cfg.n_ff, name)
    check_exact(D.dm_host()[pl.perm[rows]], dm, name)
    # property at full size: all topk copies of a token are identical rows
    tok_rows = np.argsort(pl.perm)[: cfg.topk * 4]          # sorted rows of tokens 0..3
    for t in range(4):
        rs = tok_rows[t * cfg.topk:(t + 1) * cfg.topk]
        assert all(np.array_equal(xq_dev[rs[0]], xq_dev[r]) for r in rs)
    # the combine on sampled tokens, against the oracle's combine of the device's dm
    D.combine()
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([rng.choice(cfg.tokens, min(cfg.tokens, 48), replace=False),
                                     [0, cfg.tokens - 1]]))
    slots = (toks[:, None] * cfg.topk + np.arange(cfg.topk)).reshape(-1)
    dm_tok = D.dm[torch.from_numpy(slots).cuda()].cpu().numpy()
    exp = oracle.combine(dm_tok, L.route_w[toks])
    got = D.out[torch.from_numpy(toks).cuda()].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), "combine"
    # the fused gate/up + swiglu launch the benchmark times: same bytes, whole layer
    _fused_equals_two_steps(D)
    _say("fused path equal")
    D.close()
