"""moe_prefill_plan_device on the GPU against the host-built plan.

Integer work, so the bar is byte equality: every workspace section the
kernels read (perm, inverse perm, the XCD-grouped chunk table, the XCD table,
the weight offset tables) equals the host plan's, for several routings and
chunk sizes; the plan query reads back the same counts, offsets, perm and
chunk list; the whole chain run from a device plan writes the same bytes.
Routing ids out of range are reported by the query, and every step still runs
inside its buffers (their rows join no product).
"""
import numpy as np
import pytest
import torch

from quantized_moe_expert_scatter_amd import _lib
from quantized_moe_expert_scatter_amd import workloads as wl
from quantized_moe_expert_scatter_amd.layer import DeviceLayer
from tests.gpu_common import GUARD

pytestmark = pytest.mark.gpu

FAKE_BASE = 1 << 20          # weights are never read by the plan kernels


def _a16(n):
    return (n + 15) & ~15


def _n_tiles(R):
    """Id tiles of the device plan: multiples of 2048 ids, at most 256 tiles."""
    per = -(-R // 256)
    tile = max(2048, -(-per // 2048) * 2048)
    return -(-R // tile) if R > 0 else 1


def _device_only_bytes(E, R):
    """Bytes of the sections only a device-built plan fills (counts, offsets,
    scratch, per-tile bucket counts), which sit at the end of the workspace."""
    return (_a16(4 * (E + 1)) + _a16(4 * (E + 2)) + _a16(4 * (3 * E + 4))
            + _a16(4 * (E + 1) * _n_tiles(R)))


def _weights(E, H=128, F=64):
    gu_per = _lib.moe_weight_bytes(1, 2 * F, H)
    dn_per = _lib.moe_weight_bytes(1, H, F)
    t = _lib.MOE_W_Q2_0 | _lib.MOE_W_TILED
    w_gu = _lib.Weights(t, 2 * F, H, E, FAKE_BASE, gu_per * E, np.arange(E, dtype=np.uint64) * gu_per)
    w_dn = _lib.Weights(t, H, F, E, FAKE_BASE, dn_per * E, np.arange(E, dtype=np.uint64) * dn_per)
    return w_gu, w_dn


def _both_plans(ids, E, C):
    T, K = ids.shape
    w_gu, w_dn = _weights(E)
    n = _lib.moe_plan_device_bytes(T, K, E, C)
    ws_h = torch.full((n,), 0x77, dtype=torch.uint8, device="cuda")
    ws_d = torch.full((n,), 0x33, dtype=torch.uint8, device="cuda")
    ph = _lib.moe_prefill_plan(ids, E, C, w_gu, w_dn, workspace=ws_h)
    ids_dev = torch.from_numpy(np.ascontiguousarray(ids, np.int32).reshape(-1).copy()
                               if ids.size else np.zeros(4, np.int32)).cuda()
    pd = _lib.moe_prefill_plan_device(ids_dev, T, K, E, C, w_gu, w_dn, ws_d)
    torch.cuda.synchronize()
    return ph, pd, ws_h, ws_d, n - _device_only_bytes(E, T * K)


CASES = [
    ("uniform", 300, 16, 4, 8), ("lognormal", 500, 32, 6, 16), ("uniform", 64, 8, 2, 64),
    ("lognormal", 2048, 512, 10, 64), ("flat", 768, 512, 10, 128), ("lognormal", 4096, 512, 10, 128),
    ("uniform", 1, 8, 2, 1), ("uniform", 130, 2, 1, 37), ("empty", 0, 8, 2, 64),
    ("uniform", 16384, 512, 10, 128), ("lognormal", 3001, 2048, 7, 32),
    ("uniform", 60000, 64, 10, 128),
]


@pytest.mark.parametrize("kind,T,E,K,C", CASES)
def test_device_plan_bytes_equal_host_plan(kind, T, E, K, C):
    print(f"case {kind} T={T} E={E} K={K} C={C}", flush=True)
    if kind == "uniform":
        ids = wl.routing_uniform(T, E, K, seed=T + E)
    elif kind == "lognormal":
        ids = wl.routing_lognormal(T, E, K, 1.0, seed=T + E)
    elif kind == "flat":
        ids = wl.routing_flat(T, E, K, 32, seed=T)
    else:
        ids = np.zeros((0, K), np.int32)
    ph, pd, ws_h, ws_d, shared = _both_plans(ids, E, C)
    assert torch.equal(ws_h[:shared], ws_d[:shared])
    for a, b in zip(ph.query(), pd.query()):
        assert np.array_equal(a, b)
    ph.close()
    pd.close()


def test_device_plan_runs_the_same_chain():
    """Host plan vs device plan, every output byte: the lognormal small layer,
    the 2K layer, the 128-token layer (its down product's small-chunk items
    outnumber the workgroups a device plan launches per XCD, so they take
    several each) and the 16K layer (the same for the product kernel)."""
    for cfg in (wl.small_config("lognormal", 400, 256, 128, 32, 6, routing_kind="lognormal", seed=23),
                wl.CONFIGS["2k"], wl.CONFIGS["t128"], wl.CONFIGS["16k"]):
        print("case", cfg.name, flush=True)
        L = wl.make_layer(cfg)
        outs = []
        for dev in (False, True):
            D = DeviceLayer(L.x, L.ids, L.w_gu, L.w_down, chunk_rows=128, route_w=L.route_w,
                            device_plan=dev, guard=GUARD)
            D.run_fused()
            D.combine()
            torch.cuda.synchronize()
            outs.append((D.xq.clone(), D.hq.clone(), D.dm.clone(), D.out.clone()))
            D.close()
        for a, b in zip(*outs):
            assert torch.equal(a, b)


def test_device_plan_reports_ids_out_of_range():
    """Ids outside [0, E) go to a bucket no product reads: the query refuses
    the plan and every step still runs inside its buffers."""
    cfg = wl.small_config("bad", 50, 256, 128, 8, 2, seed=41)
    L = wl.make_layer(cfg)
    ids = L.ids.copy()
    ids[3, 1] = 8
    ids[17, 0] = -5
    D = DeviceLayer(L.x, ids, L.w_gu, L.w_down, chunk_rows=64, route_w=L.route_w, device_plan=True,
                    guard=GUARD)
    with pytest.raises(_lib.MoeError) as e:
        D.plan.query()
    assert e.value.status == -1
    D.run_fused()
    D.combine()
    torch.cuda.synchronize()
    # the tokens without a bad id get the outputs of the same tokens under a
    # host plan of the valid ids (their rows sit elsewhere, the values do not move)
    ok = np.setdiff1d(np.arange(cfg.tokens), [3, 17])
    good = L.ids.copy()
    H = DeviceLayer(L.x, good, L.w_gu, L.w_down, chunk_rows=64, route_w=L.route_w, guard=GUARD)
    H.run_fused()
    H.combine()
    torch.cuda.synchronize()
    assert np.array_equal(D.out_host()[ok].view(np.uint32), H.out_host()[ok].view(np.uint32))
    D.close()
    H.close()
