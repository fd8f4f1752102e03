"""Pins of the oracle's weight decoding (no GPU).

Q2_0 ("Strata" PR #2145 description: 64-value blocks, 2-bit codes, one
binary16 scale shared by the two 32-value halves) and the 4-bit non-linear
down format NL4 (PR #3752 commit list names IQ4_NL; this project's codebook
is drawn from the seed).  Pinned by hand-worked blocks
(tests/golden/weight_blocks.json), a second unpacker written with numpy
array operations, and numpy's own binary16 conversion.
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle
from quantized_moe_expert_scatter_amd import workloads as wl
from tests import oracle_pins as pins

GOLD = os.path.join(os.path.dirname(__file__), "golden", "weight_blocks.json")


def _gold():
    return json.load(open(GOLD))


@pytest.mark.parametrize("i", [0, 1])
def test_q2_0_golden(i):
    g = _gold()["q2_0"][i]
    blk = np.concatenate([np.array(g["codes_bytes"], np.uint8),
                          np.array([g["scale_f16_bits"]], np.uint16).view(np.uint8)])
    vals, dw = oracle.decode_row(oracle.Q2_0, blk, 1, 64, 0)
    assert vals.tolist() == g["values"]
    assert dw.tolist() == [g["scale"], g["scale"]]


def test_nl4_golden():
    g = _gold()["nl4"][0]
    blk = np.concatenate([np.array(g["codes_bytes"], np.uint8),
                          np.array([g["scale_f16_bits"]], np.uint16).view(np.uint8)])
    vals, dw = oracle.decode_row(oracle.NL4, blk, 1, 32, 0, np.array(g["codebook"], np.int8))
    assert vals.tolist() == g["values"]
    assert dw.tolist() == [g["scale"]]


def test_half_decode_all_patterns():
    """Every finite binary16 pattern decodes to numpy's value (one block per pattern)."""
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(bits.view(np.float16))
    bits = bits[finite]
    rows = bits.shape[0]
    expert = np.concatenate([np.zeros(rows * 16, np.uint8), bits.view(np.uint8)])
    got = np.empty(rows, np.float32)
    for n in range(rows):
        _, dw = oracle.decode_row(oracle.Q2_0, expert, rows, 64, n)
        got[n] = dw[0]
    ref = bits.view(np.float16).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("wtype,rows,cols", [(oracle.Q2_0, 6, 256), (oracle.NL4, 5, 96)])
def test_decode_matches_array_unpack(wtype, rows, cols):
    w = wl.expert_weights(wtype, rows, cols, 2, seed=9)
    for e in range(2):
        ex = w.expert(e)
        iw, sc = pins.int_weights(wtype, ex, rows, cols, w.codebook)
        for n in range(rows):
            vals, dw = oracle.decode_row(wtype, ex, rows, cols, n, w.codebook)
            assert np.array_equal(vals.astype(np.int64), iw[n])
            assert np.array_equal(dw, sc[n])


def test_codebook_draw():
    cb = wl.nl4_codebook(123)
    assert cb.dtype == np.int8 and cb.shape == (16,)
    assert np.all(np.diff(cb.astype(int)) > 0)
    assert cb.min() >= -127 and cb.max() <= 127
