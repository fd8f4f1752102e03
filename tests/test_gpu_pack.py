"""moe_weights_pack on the GPU: the tiled layout is the documented byte
permutation of each plane, experts at a constant stride (one launch) or in a
shuffled slot order with gaps (one launch per expert), Q2_0 and NL4.

The expected bytes are the row-major planes rearranged here with numpy:
block b of row 32 i + r goes to slot (i * blocks_per_row + b) * 32 + r.
"""
import numpy as np
import pytest
import torch

from quantized_moe_expert_scatter_amd import _lib
from quantized_moe_expert_scatter_amd import workloads as wl

pytestmark = pytest.mark.gpu


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
        expect[o:o + 16 * n] = _tiled(m[:16 * n], rows, nb, 16)
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
