"""Seeded random layer shapes through the whole chain, every element against
the oracle.

Each case draws hidden and n_ff widths (some with stage counts the product
kernel streams over, some with ragged N tiles), the expert count, top-k,
token count, chunk size, routing (uniform or lognormal), the down product's
format (Q2_0 or NL4) and the plan (host- or device-built), so that the
kernels' launch-time choices (small-chunk kernel or product kernel, 8-row
steps of the last row tile, tile streams, prefetch depths) meet in
combinations the hand-written cases do not list. The draw is fixed by its
seed; the oracle's work per case is capped so the set runs in seconds.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from quantized_moe_expert_scatter_amd import workloads as wl
from tests.gpu_common import check_exact, check_h_exact, device_layer, rel_rms, w_tuple

pytestmark = pytest.mark.gpu

HIDDEN = (256, 448, 640, 1280, 1792)
N_FF = (128, 192, 320, 640)
CHUNKS = (16, 32, 37, 64, 100, 128)
MAX_MACS = 3.0e9          # oracle work per case: rows * 3 * hidden * n_ff


def _draw_cases(n, seed, stream=False):
    """stream: shapes where the down product runs items of several N tiles
    (whole 256-row tiles, n_ff 640 = 10 stages, Q2_0, chunks of <= 64 rows)."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        hidden = int(rng.choice((1280, 1792, 2560) if stream else HIDDEN))
        n_ff = 640 if stream else int(rng.choice(N_FF))
        n_expert = int(rng.integers(1, 65))
        topk = int(rng.integers(1, min(n_expert, 8) + 1))
        tokens = int(rng.integers(1, 401))
        if tokens * topk * 3.0 * hidden * n_ff > MAX_MACS:
            continue
        cases.append(dict(
            name=f"{'stream' if stream else 'rand'}{len(cases)}", tokens=tokens, hidden=hidden, n_ff=n_ff,
            n_expert=n_expert, topk=topk,
            chunk_rows=int(rng.choice(CHUNKS[:4] if stream else CHUNKS)),
            routing="lognormal" if rng.random() < 0.5 else "uniform",
            down=wl.Q2_0 if stream or rng.random() >= 0.3 else wl.NL4,
            device_plan=bool(rng.random() < 0.3),
            seed=int(rng.integers(100, 10_000))))
    return cases


CASES = _draw_cases(12, seed=20261203) + _draw_cases(4, seed=20261204, stream=True)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_random_layer_every_element(case):
    print("case", case, flush=True)
    cfg = wl.small_config(case["name"], case["tokens"], case["hidden"], case["n_ff"], case["n_expert"],
                          case["topk"], routing_kind=case["routing"], down_type=case["down"], seed=case["seed"])
    L = wl.make_layer(cfg)
    ref = oracle.layer(L.x, L.ids, cfg.n_expert, cfg.n_ff, w_tuple(L.w_gu), w_tuple(L.w_down), n_threads=8)
    D = device_layer(L, chunk_rows=case["chunk_rows"], device_plan=case["device_plan"])
    D.run()
    torch.cuda.synchronize()
    assert np.array_equal(D.xq_host(), ref.xq), "q8_1 bytes of X"
    gu = D.gu_host()
    assert np.array_equal(gu.view(np.uint32), ref.gu.view(np.uint32)), \
        f"GU bits: rel RMS {rel_rms(gu, ref.gu):.3e}"
    check_h_exact(D.hq_host(), ref.hq, cfg.n_ff, case["name"])
    check_exact(D.dm_host(), ref.dm, case["name"])
    D.hq.fill_(0x5A)
    D.dm.fill_(float("nan"))
    D.run_fused()
    torch.cuda.synchronize()
    check_h_exact(D.hq_host(), ref.hq, cfg.n_ff, case["name"] + " fused")
    check_exact(D.dm_host(), ref.dm, case["name"] + " fused")
    D.close()                 # also checks the guard bytes around every output buffer
