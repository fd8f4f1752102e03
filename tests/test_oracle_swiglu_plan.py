"""Pins of the oracle's fused swiglu + q8_1 step and of the plan (no GPU).

swiglu + q8_1: "Strata" PR #3752, swiglu_quant commit (swiglu of the
gate/up row, then q8_1 of every 32-value block, H never stored; tested with a
zero row and a row with one huge value).  Pinned against fp64 SiLU, special
values, and the q8_1 pins.

Plan: PR #3752 commit list (rows scattered so that each expert's rows are
contiguous; fixed-size row chunks of the experts, largest expert first; each
expert at its own row count).  Pinned by a hand-worked example
(tests/golden/plan_small.json) and invariants on random routings.
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle
from quantized_moe_expert_scatter_amd import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden", "plan_small.json")


# ---------------------------------------------------------------- swiglu
def test_swiglu_against_fp64():
    rng = np.random.default_rng(1)
    g = (rng.standard_normal(20000) * 6).astype(np.float32)
    u = (rng.standard_normal(20000) * 3).astype(np.float32)
    gu = np.concatenate([g, u])[None, :]
    h = oracle.swiglu_rows(gu, 20000)[0].astype(np.float64)
    g64, u64 = g.astype(np.float64), u.astype(np.float64)
    ref = g64 / (1.0 + np.exp(-g64)) * u64
    # expf, one add, one divide and one multiply in fp32: a few ulps
    tol = 8 * np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) + 1e-44
    assert np.all(np.abs(h - ref) <= tol)


def test_swiglu_exp_is_correctly_rounded():
    """e^-g inside silu is the binary32 value nearest to the exact
    exponential: pinned by a 60-digit decimal exponential rounded with exact
    rational arithmetic; the rest is one fp32 add, divide and multiply."""
    from decimal import Context, Decimal
    from fractions import Fraction
    from tests.oracle_pins import round_to_f32
    ctx = Context(prec=60)
    rng = np.random.default_rng(5)
    g = (rng.standard_normal(3000) * 5).astype(np.float32)
    u = rng.standard_normal(3000).astype(np.float32)
    for gi, ui in zip(g, u):
        e = round_to_f32(Fraction(ctx.exp(Decimal(-float(gi)))))
        silu = np.float32(gi) / (np.float32(1.0) + e)
        assert oracle.swiglu(gi, ui) == np.float32(silu * ui), (gi, ui)


def test_swiglu_special_values():
    assert oracle.swiglu(0.0, 5.0) == 0.0
    assert oracle.swiglu(3.0, 0.0) == 0.0
    assert oracle.swiglu(-200.0, 2.0) == 0.0          # exp overflows: silu -> -0
    assert oracle.swiglu(100.0, 2.0) == 200.0          # silu(g) = g once exp(-g) < ulp
    ref = 1.0 / (1.0 + np.exp(-1.0))
    assert abs(oracle.swiglu(1.0, 1.0) - ref) <= 2 * np.spacing(np.float32(ref))


def test_swiglu_q8_zero_and_huge_rows():
    F = 128
    gu = np.zeros((3, 2 * F), np.float32)
    gu[1, :F] = 1.0
    gu[1, F:] = 1.0
    gu[1, 5] = 1e20                                   # one huge gate value
    gu[2] = np.random.default_rng(2).standard_normal(2 * F).astype(np.float32)
    hq = oracle.swiglu_q8(gu, F)
    q, d, s = oracle.unpack_q8_1(hq, F)
    assert np.all(q[0] == 0) and np.all(d[0] == 0) and np.all(s[0] == 0)
    # block 0 of row 1 is dominated by the huge value: it alone is non-zero
    assert q[1, 5] == 127 and np.count_nonzero(q[1, :32]) == 1 and s[1, 0] == 127
    # the other blocks of row 1 quantize silu(1) alone: all 127
    assert np.all(q[1, 32:] == 127)


def test_swiglu_q8_is_quantized_swiglu_and_layouts_agree():
    rng = np.random.default_rng(3)
    F = 96
    gu = rng.standard_normal((7, 2 * F)).astype(np.float32) * 4
    hq = oracle.swiglu_q8(gu, F)
    assert np.array_equal(hq, oracle.q8_1_rows(oracle.swiglu_rows(gu, F)))
    inter = np.empty_like(gu)
    inter[:, 0::2] = gu[:, :F]
    inter[:, 1::2] = gu[:, F:]
    assert np.array_equal(oracle.swiglu_q8(inter, F, interleaved=True), hq)


# ------------------------------------------------------------------ plan
def test_plan_golden():
    g = json.load(open(GOLD))
    pl = oracle.plan(np.array(g["ids"], np.int32), g["n_expert"], g["chunk_rows"])
    assert pl.counts.tolist() == g["counts"]
    assert pl.offsets.tolist() == g["offsets"]
    assert pl.perm.tolist() == g["perm"]
    assert pl.chunks.tolist() == g["chunks"]


def check_plan_invariants(ids, E, C, counts, offsets, perm, chunks):
    T, K = ids.shape
    R = T * K
    flat = ids.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(perm), np.arange(R))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)              # stable
    covered = np.zeros(R, np.int64)
    last_count = None
    seen = []
    for e, r0, nr, pad in chunks:
        assert pad == 0 and 1 <= nr <= C
        assert offsets[e] <= r0 and r0 + nr <= offsets[e + 1]
        covered[r0:r0 + nr] += 1
        if not seen or seen[-1] != e:
            assert e not in seen                      # an expert's chunks are consecutive
            if last_count is not None:
                assert counts[e] < last_count or (counts[e] == last_count and e > seen[-1])
            seen.append(e)
            last_count = counts[e]
            assert r0 == offsets[e]
        else:
            assert r0 == prev_end
        prev_end = r0 + nr
    assert np.all(covered == 1)
    assert len(chunks) == sum((c + C - 1) // C for c in counts)


@pytest.mark.parametrize("kind,T,E,K,C", [("uniform", 300, 16, 4, 8), ("lognormal", 500, 32, 6, 16),
                                          ("uniform", 64, 8, 2, 64), ("lognormal", 2048, 512, 10, 64),
                                          ("flat", 768, 512, 10, 16), ("flat", 4096, 512, 10, 64)])
def test_plan_invariants(kind, T, E, K, C):
    if kind == "uniform":
        ids = wl.routing_uniform(T, E, K, seed=T)
    elif kind == "flat":
        ids = wl.routing_flat(T, E, K, 32, seed=T)   # many equal counts: the tie order decides
    else:
        ids = wl.routing_lognormal(T, E, K, 1.0, seed=T)
    pl = oracle.plan(ids, E, C)
    check_plan_invariants(ids, E, C, pl.counts, pl.offsets, pl.perm, pl.chunks)


def test_plan_rejects_bad_id():
    with pytest.raises(ValueError):
        oracle.plan(np.array([[0, 4]], np.int32), 4, 2)
    with pytest.raises(ValueError):
        oracle.plan(np.array([[0, -1]], np.int32), 4, 2)


def test_plan_empty_experts_and_duplicates():
    ids = np.array([[2, 2], [2, 0]], np.int32)      # duplicate id inside a token is two rows
    pl = oracle.plan(ids, 5, 1)
    assert pl.counts.tolist() == [1, 0, 3, 0, 0]
    assert pl.chunks[:, 0].tolist() == [2, 2, 2, 0]


@pytest.mark.parametrize("name", list(wl.SWEEP))
def test_sweep_routings(name):
    """The sweep's inputs: T tokens, top-10 distinct experts per token; the
    flat routing gives every routed expert the same row count, 32 where
    T*10/32 experts fit in 512, else T*10/512."""
    cfg = wl.SWEEP[name]
    ids = wl.routing(cfg)
    assert ids.shape == (cfg.tokens, cfg.topk)
    assert ids.min() >= 0 and ids.max() < cfg.n_expert
    assert all(len(set(r)) == cfg.topk for r in ids.tolist())
    counts = np.bincount(ids.ravel(), minlength=cfg.n_expert)
    if cfg.routing == "flat32":
        used = counts[counts > 0]
        assert used.size == min(cfg.n_expert, cfg.rows // 32)
        assert used.min() == used.max() == cfg.rows // used.size
    else:
        assert counts.max() > 2 * np.median(counts[counts > 0])      # skewed
