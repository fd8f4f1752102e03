"""Independent helpers the oracle's pins compare against.

These do not reuse the oracle's code: weights are unpacked with numpy bit
operations on whole arrays (the oracle loops byte by byte in C), fp32
rounding of exact rationals is done with integer arithmetic on Fractions, and
the float references dequantize and multiply in fp64.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

Q2_0 = 1
NL4 = 2


def unpack_q2_0(expert: np.ndarray, rows: int, cols: int):
    """-> (codes uint8 [rows, cols] in 0..3, scales float32 [rows, cols//64])."""
    nb = cols // 64
    codes_plane = expert[: rows * nb * 16].reshape(rows, nb, 16)
    # field j of byte b is value 16*j + b: stack the four 2-bit fields as
    # quarters of the 64-value block
    quarters = [(codes_plane >> (2 * j)) & 3 for j in range(4)]
    codes = np.concatenate(quarters, axis=2).reshape(rows, cols)
    scales = expert[rows * nb * 16: rows * nb * 18].view(np.float16).reshape(rows, nb)
    return codes.astype(np.uint8), scales.astype(np.float32)


def unpack_nl4(expert: np.ndarray, rows: int, cols: int):
    """-> (codes uint8 [rows, cols] in 0..15, scales float32 [rows, cols//32])."""
    nb = cols // 32
    codes_plane = expert[: rows * nb * 16].reshape(rows, nb, 16)
    codes = np.concatenate([codes_plane & 15, codes_plane >> 4], axis=2).reshape(rows, cols)
    scales = expert[rows * nb * 16: rows * nb * 18].view(np.float16).reshape(rows, nb)
    return codes.astype(np.uint8), scales.astype(np.float32)


def int_weights(wtype, expert, rows, cols, codebook=None):
    """Signed integer weights [rows, cols] and per-32-block scales [rows, cols//32]."""
    if wtype == Q2_0:
        c, s = unpack_q2_0(expert, rows, cols)
        return c.astype(np.int64) - 2, np.repeat(s, 2, axis=1)
    c, s = unpack_nl4(expert, rows, cols)
    return np.asarray(codebook, np.int64)[c], s


def dequant(wtype, expert, rows, cols, codebook=None) -> np.ndarray:
    w, s = int_weights(wtype, expert, rows, cols, codebook)
    return w.astype(np.float64) * np.repeat(s.astype(np.float64), 32, axis=1)


def round_to_f32(x: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) binary32 value of a rational."""
    if x == 0:
        return np.float32(0.0)
    neg = x < 0
    a = -x if neg else x
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp_e = max(e - 23, -149)
    scaled = a / (Fraction(2) ** ulp_e)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = float(n) * 2.0 ** ulp_e
    if val >= 2.0 ** 128:
        val = float("inf")
    return np.float32(-val if neg else val)


def exact_epilogue(dx, dw, dots, round_product: bool) -> np.float32:
    """acc <- round32(acc + dx_b * P_b) over blocks in order, where
    P_b = dw_b * dot_b exactly (round_product False) or rounded to binary32
    first (round_product True)."""
    acc = Fraction(0)
    for b in range(len(dots)):
        p = Fraction(float(dw[b])) * int(dots[b])
        if round_product:
            p = Fraction(float(round_to_f32(p)))
        acc = Fraction(float(round_to_f32(acc + Fraction(float(dx[b])) * p)))
    return np.float32(float(acc))


def rel_rms(a: np.ndarray, ref: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.sqrt(np.sum(ref * ref))
    return float(np.sqrt(np.sum((a - ref) ** 2)) / den) if den > 0 else float(np.sqrt(np.sum(a * a)))
