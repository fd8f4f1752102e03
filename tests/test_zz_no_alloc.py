"""moe_prefill_plan_device_noalloc (the plan for callers that cannot allocate)
against moe_prefill_plan_device, through the C ABI: two calls in a row on one
device, the second with a smaller layer, each checked before the next call
overwrites the library's workspace.  Integer plan, so the bar is byte
equality: the plan query (counts, offsets, perm, chunk list) and every output
of the chain run from each plan (xq, hq, dm, the combine)."""
import numpy as np
import pytest
import torch

from quantized_moe_expert_scatter_amd import _lib
from quantized_moe_expert_scatter_amd import workloads as wl
from quantized_moe_expert_scatter_amd.layer import DeviceLayer
from tests.gpu_common import GUARD

pytestmark = pytest.mark.gpu


def _run(D):
    D.run_fused()
    D.combine()
    torch.cuda.synchronize()
    return [D.xq.clone(), D.hq.clone(), D.dm.clone(), D.out.clone()]


def test_noalloc_plan_matches_device_plan_twice():
    cfgs = [wl.CONFIGS["2k"], wl.small_config("lognormal", 400, 256, 128, 32, 6,
                                              routing_kind="lognormal", seed=23)]
    for cfg in cfgs:                                   # the second call is the smaller layer
        print("case", cfg.name, cfg.tokens, "tokens", flush=True)
        L = wl.make_layer(cfg)
        A = DeviceLayer(L.x, L.ids, L.w_gu, L.w_down, chunk_rows=128, route_w=L.route_w,
                        device_plan=True, guard=GUARD)
        B = DeviceLayer(L.x, L.ids, L.w_gu, L.w_down, chunk_rows=128, route_w=L.route_w,
                        device_plan=True, guard=GUARD)
        B.plan.close()
        B.plan = _lib.moe_prefill_plan_device_noalloc(B.ids_dev, cfg.tokens, cfg.topk, cfg.n_expert,
                                                      128, B.w_gu, B.w_dn)
        for a, b in zip(A.plan.query(), B.plan.query()):
            assert np.array_equal(a, b)
        for a, b in zip(_run(A), _run(B)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
        A.close()
        B.close()


def test_noalloc_plan_refusals():
    """Beyond the workspace: MOE_ESIZE; experts not at a constant stride: MOE_EINVAL."""
    cfg = wl.small_config("refuse", 8, 256, 128, 4, 2, seed=5)
    L = wl.make_layer(cfg)
    D = DeviceLayer(L.x, L.ids, L.w_gu, L.w_down, chunk_rows=64, route_w=L.route_w, device_plan=True)
    # a million rows need more than the 4 MiB workspace: refused on the host,
    # before anything would read the (smaller) id buffer
    big = 1 << 20
    assert _lib.moe_plan_device_bytes(big, 1, cfg.n_expert, 64) > 4 << 20
    with pytest.raises(_lib.MoeError) as e:
        _lib.moe_prefill_plan_device_noalloc(D.ids_dev, big, 1, cfg.n_expert, 64, D.w_gu, D.w_dn)
    assert e.value.status == -4
    Ls = wl.make_layer(cfg, shuffle_slots=True)      # experts in a shuffled slot order with gaps
    off = Ls.w_gu.offsets.astype(np.int64)
    assert np.any(off - off[0] != np.arange(cfg.n_expert) * (off[1] - off[0]))
    S = DeviceLayer(Ls.x, Ls.ids, Ls.w_gu, Ls.w_down, chunk_rows=64, route_w=Ls.route_w,
                    device_plan=True)
    with pytest.raises(_lib.MoeError) as e:
        _lib.moe_prefill_plan_device_noalloc(S.ids_dev, cfg.tokens, cfg.topk, cfg.n_expert, 64,
                                             S.w_gu, S.w_dn)
    assert e.value.status == -1
    D.close()
    S.close()
