"""moe_weights_pack on the GPU: the tiled layout is the documented byte
permutation of each plane, experts at a constant stride (one launch) or in a
shuffled slot order with gaps (one launch per expert), Q2_0 and NL4.

The expected bytes are the row-major planes rearranged here with numpy:
block b of row 32 i + r goes to slot (i * blocks_per_row + b) * 32 + r, and
within a Q2_0 block the code of value v = 32 h + 16 g + 8 kq + p (stored at
bits 2 (v // 16) of byte v % 16) moves to bits 2 g + 4 (p % 2) of byte
8 kq + 4 h + p // 2.
"""
import numpy as np
import pytest
import torch

from quantized_moe_expert_scatter_amd import _lib
from quantized_moe_expert_scatter_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _q2_codes_rearranged(codes: np.ndarray) -> np.ndarray:
    """codes: uint8 [n, 16] Q2_0 code blocks -> the kernels' order within each block."""
    out = np.zeros_like(codes)
    for v in range(64):
        c = (codes[:, v % 16] >> (2 * (v // 16))) & 3
        h, g, kq, p = v // 32, (v // 16) % 2, (v // 8) % 2, v % 8
        out[:, 8 * kq + 4 * h + p // 2] |= (c << (2 * g + 4 * (p % 2))).astype(np.uint8)
    return out


def _tiled(plane: np.ndarray, rows: int, nb: int, item: int) -> np.ndarray:
    """plane: bytes of rows x nb items of `item` bytes in (row, block) order."""
    a = plane.reshape(rows // 32, 32, nb, item)
    return a.transpose(0, 2, 1, 3).reshape(-1)


@pytest.mark.parametrize("wtype,rows,cols,E,shuffle", [
    (wl.Q2_0, 64, 64, 1, False),
    (wl.Q2_0, 128, 192, 5, False),
    (wl.Q2_0, 192, 128, 6, True),
    (wl.NL4, 256, 96, 4, False),
    (wl.NL4, 64, 224, 7, True),
    (wl.Q2_0, 1280, 2560, 3, True),
])
def test_pack_is_the_tiled_permutation(wtype, rows, cols, E, shuffle):
    print(f"case wtype={wtype} rows={rows} cols={cols} E={E} shuffle={shuffle}", flush=True)
    w = wl.expert_weights(wtype, rows, cols, E, seed=rows + cols + E, shuffle_slots=shuffle)
    src = torch.from_numpy(w.buf).cuda()
    rw = _lib.Weights(w.wtype, rows, cols, E, src, w.buf.nbytes, w.offsets, w.codebook)
    dst = torch.full_like(src, 0xA5)
    packed = _lib.moe_weights_pack(rw, dst)
    torch.cuda.synchronize()
    assert packed.struct.type == w.wtype | _lib.MOE_W_TILED
    out = dst.cpu().numpy()
    nb = cols // wl.block_of(wtype)
    n = rows * nb
    expect = np.full_like(w.buf, 0xA5)               # gaps between slots stay untouched
    for e in range(E):
        o = int(w.offsets[e])
        m = w.expert(e)
        codes = m[:16 * n]
        if wtype == wl.Q2_0:
            codes = _q2_codes_rearranged(codes.reshape(n, 16)).reshape(-1)
        expect[o:o + 16 * n] = _tiled(codes, rows, nb, 16)
        expect[o + 16 * n:o + 18 * n] = _tiled(m[16 * n:], rows, nb, 2)
    assert np.array_equal(out, expect)


@pytest.mark.parametrize("wtype,rows,cols,E", [(wl.Q2_0, 128, 192, 3), (wl.NL4, 192, 96, 2)])
def test_pack_deinterleaves_gate_up(wtype, rows, cols, E):
    """Alternating gate/up rows are packed into split order: the result equals
    packing the split-stored matrices."""
    print(f"case interleaved wtype={wtype} rows={rows} cols={cols} E={E}", flush=True)
    w = wl.expert_weights(wtype, rows, cols, E, seed=rows + 7)
    wi = wl.interleave_gate_up(w)
    outs = []
    for ww, flag in ((w, 0), (wi, _lib.MOE_W_GU_INTERLEAVED)):
        src = torch.from_numpy(ww.buf).cuda()
        rw = _lib.Weights(ww.wtype | flag, rows, cols, E, src, ww.buf.nbytes, ww.offsets, ww.codebook)
        dst = torch.zeros_like(src)
        packed = _lib.moe_weights_pack(rw, dst)
        torch.cuda.synchronize()
        assert packed.struct.type == wtype | _lib.MOE_W_TILED
        outs.append(dst.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
