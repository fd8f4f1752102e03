"""Pins of the oracle's q8_1 quantizer (no GPU).

q8_1 as the "Strata" pages use it for the int8 activation rows (PR #3752,
quantize_scatter / swiglu_quant commits): 32 values, fp32 scale
d = max|x| / 127, int8 values, the block's integer sum.  Pinned by hand-worked
blocks (tests/golden/q8_1_blocks.json), the defining inequalities, and exact
power-of-two scaling.
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "q8_1_blocks.json")


def _golden():
    return json.load(open(GOLD))["blocks"]


@pytest.mark.parametrize("blk", _golden(), ids=lambda b: b["name"][:40])
def test_golden_blocks(blk):
    if "x" in blk:
        x = np.array(blk["x"], np.float32)
        d_exp = np.float32(blk["d"])
    else:
        unit = np.float32(2.0 ** -149)
        x = np.array(blk["x_units_of_2^-149"], np.float64).astype(np.float32) * unit
        d_exp = np.float32(blk["d_units_of_2^-149"]) * unit
    d, s, q = oracle.q8_1_block(x)
    assert d == d_exp
    assert q.tolist() == blk["q"]
    assert s == blk["s"]


def _random_blocks(n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 32)).astype(np.float32)
    x *= np.float32(2.0) ** rng.integers(-20, 20, size=(n, 1)).astype(np.float32)
    return x


def test_defining_inequalities():
    x = _random_blocks(2000, 1)
    rows = oracle.q8_1_rows(x.reshape(-1, 32 * 8))
    q, d, s = oracle.unpack_q8_1(rows, 32 * 8)
    q = q.reshape(-1, 32).astype(np.int64)
    d = d.reshape(-1).astype(np.float64)
    s = s.reshape(-1)
    xb = x.reshape(-1, 32).astype(np.float64)
    amax = np.abs(xb).max(axis=1)
    # d is the fp32 quotient amax / 127
    assert np.all(d == (amax.astype(np.float32) / np.float32(127.0)).astype(np.float64))
    assert np.all(np.abs(q) <= 127)
    # the largest magnitude quantizes to +-127
    arg = np.abs(xb).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(len(q)), arg]) == 127)
    # block sum
    assert np.all(s == q.sum(axis=1))
    # nearest integer of x/d: |x/d - q| <= 1/2 (+ rounding slack of the quotient)
    err = np.abs(xb / d[:, None] - q)
    assert np.all(err <= 0.5 + 1e-5)
    # signs agree
    assert np.all((q == 0) | (np.sign(q) == np.sign(xb)))


@pytest.mark.parametrize("k", [-30, -7, 1, 5, 40])
def test_power_of_two_scaling(k):
    x = _random_blocks(300, 2) * np.float32(2.0 ** -10)
    a = oracle.q8_1_rows(x)
    b = oracle.q8_1_rows(x * np.float32(2.0 ** k))
    qa, da, sa = oracle.unpack_q8_1(a, 32)
    qb, db, sb = oracle.unpack_q8_1(b, 32)
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb)
    assert np.array_equal(db, da * np.float32(2.0 ** k))


def test_row_layout():
    """A row of n blocks is q[cols] | d[cols/32] fp32 | s[cols/32] int32."""
    x = _random_blocks(4, 3).reshape(1, 128)
    row = oracle.q8_1_rows(x)[0]
    assert row.shape == (128 + 4 * 8,)
    for b in range(4):
        d, s, q = oracle.q8_1_block(x[0, 32 * b:32 * b + 32])
        assert np.array_equal(row[32 * b:32 * b + 32].view(np.int8), q)
        assert row[128 + 4 * b:128 + 4 * b + 4].view(np.float32)[0] == d
        assert row[144 + 4 * b:144 + 4 * b + 4].view(np.int32)[0] == s


def test_quantize_scatter_rows_follow_perm():
    rng = np.random.default_rng(4)
    T, H, K, E = 9, 64, 3, 5
    x = rng.standard_normal((T, H)).astype(np.float32)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    pl = oracle.plan(ids, E, 4)
    xq = oracle.quantize_scatter(x, K, pl.perm)
    per_token = oracle.q8_1_rows(x)
    for r in range(T * K):
        assert np.array_equal(xq[r], per_token[pl.perm[r] // K])
    sub = np.array([5, 0, 17], np.int32)
    assert np.array_equal(oracle.quantize_scatter(x, K, pl.perm, rows=sub), xq[sub])
