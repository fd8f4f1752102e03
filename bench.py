"""Benchmark of the prefill routed-expert product on one MI355X.

One step = one layer's whole routed-expert product in three launches
(quantize_scatter; the gate/up product with swiglu and q8_1 of H fused into
its epilogue; the down product) over inputs already resident in HBM.  The
plan (host counting sort + one upload, or the device-built plan) is built once
outside the timed region and timed separately.

Every layer's inputs are generated and uploaded before any timing; all layers
are warmed up together; the headline layer is then timed over exactly
--steps steps between two synchronizations (value, ms_per_step), and every
layer in every form (three launches, four launches with GU in memory, and
with the combine) over --rounds interleaved rounds, reported as medians.

Prints ONE JSON line: value = effective int8 TOPS of the 16,384-token layer
(2 x useful MACs / time), ms_per_step = ms per layer; the 2k, 8k, t128 and
2k_nl4 layers alongside, the roofline of the dominant kernel and of the
layer, and the oracle timed on a bounded sample of rows on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms/layer + effective int8 TOPS (512 experts, top-10) at 2K/8K/16K tokens"
# "Strata" PR #2145, Kernels table: the fused int8 expert layer on an RTX 2080
# Ti at 2,048 and 16,384 tokens (ms per layer)
PAGES_MS = {"2k": 6.61, "16k": 37.15}
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
# the method's products are int8 contractions: dense int8 MFMA peak of MI355X
MFMA_I8_PEAK_TOPS = 5000.0
# they run on fp16 matrix cores here (int8 values and 2/4-bit weights are
# exact in fp16): dense fp16 MFMA peak, reported alongside
MFMA_F16_PEAK_TFLOPS = 2500.0
# fp32 FMA on the vector ALU, MI355X's published rate: 256 CU x 4 SIMD x 32
# lanes per clock x 2 flop x 2.4 GHz = 157.3 TFLOP/s.  That rate counts the
# packed two-wide fp32 forms, which these kernels do not use: a plain wave64
# v_fmac_f32 holds its SIMD for 4 cycles (measured), half of it.
VALU_F32_PEAK_TFLOPS = 256 * 4 * 32 * 2 * 2.4e9 / 1e12
# the timed step: the whole path in three launches (gate/up, swiglu and q8_1
# fused); the four-launch form with GU in memory is reported alongside
KERNELS = ["quantize_scatter", "expert_gate_up_swiglu_q8", "expert_down"]
KERNELS_4 = ["quantize_scatter", "expert_gate_up", "swiglu_q8", "expert_down"]
KERNEL_SOURCES = {
    "expert_gate_up_swiglu_q8": "quantized_moe_expert_scatter_amd/csrc/expert_kernels.hip",
    "expert_gate_up": "quantized_moe_expert_scatter_amd/csrc/expert_kernels.hip",
    "expert_down": "quantized_moe_expert_scatter_amd/csrc/expert_kernels.hip",
    "quantize_scatter": "quantized_moe_expert_scatter_amd/csrc/quant_kernels.hip",
    "swiglu_q8": "quantized_moe_expert_scatter_amd/csrc/quant_kernels.hip",
    "moe_combine": "quantized_moe_expert_scatter_amd/csrc/combine_kernels.hip",
}


def algorithmic(cfg, counts):
    """Bytes and int8 ops each step moves / performs, counted once (weights of
    touched experts only)."""
    T, H, F, K = cfg.tokens, cfg.hidden, cfg.n_ff, cfg.topk
    R = T * K
    touched = int(np.count_nonzero(counts))
    dn_blk = 64 if cfg.down_type == 1 else 32
    gu_blk = 64 if cfg.gu_type == 1 else 32
    w_gu = touched * 2 * F * (H // gu_blk) * 18
    w_dn = touched * H * (F // dn_blk) * 18
    q8 = lambda n: n + n // 32 * 8
    by = {
        "quantize_scatter": T * H * 4 + R * q8(H),
        "expert_gate_up": R * q8(H) + w_gu + R * 2 * F * 4,
        "swiglu_q8": R * 2 * F * 4 + R * q8(F),
        "expert_gate_up_swiglu_q8": R * q8(H) + w_gu + R * q8(F),
        "expert_down": R * q8(F) + w_dn + R * H * 4,
        "moe_combine": R * H * 4 + R * 4 + T * H * 4,
    }
    ops = {"expert_gate_up": 2 * R * 2 * F * H, "expert_gate_up_swiglu_q8": 2 * R * 2 * F * H,
           "expert_down": 2 * R * H * F}
    # epilogue: one fp32 FMA (2 flop) per (row, output, 32-value block) for
    # Q2_0 (d*dot comes out of the MFMA), two for NL4 (d*dot, then the FMA)
    dn_epi = 2 if cfg.down_type == 1 else 4
    gu_epi = 2 if cfg.gu_type == 1 else 4
    alu = {"expert_gate_up": gu_epi * R * 2 * F * (H // 32),
           "expert_gate_up_swiglu_q8": gu_epi * R * 2 * F * (H // 32),
           "expert_down": dn_epi * R * H * (F // 32)}
    return by, ops, alu


def _forms(D, form):
    """(kernel names, launch callables) of one step in the given form."""
    if form == "fused":
        return list(KERNELS), [D.quantize_scatter, D.expert_gate_up_swiglu_q8, D.expert_down]
    if form == "four":
        return list(KERNELS_4), [D.quantize_scatter, D.expert_gate_up, D.swiglu_q8, D.expert_down]
    return (list(KERNELS) + ["moe_combine"],
            [D.quantize_scatter, D.expert_gate_up_swiglu_q8, D.expert_down, D.combine])


def time_layer(D, steps, warmup, form="fused"):
    """The contract's timing: warm-up steps, then exactly `steps` steps between
    two synchronizations; HIP events on the launch stream around every kernel.
    Returns (ms per step over the bracket, mean ms per kernel)."""
    import torch
    stream = torch.cuda.current_stream()
    names, fns = _forms(D, form)
    for _ in range(warmup):
        for f in fns:
            f()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(steps):
        ev[s][0].record(stream)
        for i, f in enumerate(fns):
            f()
            ev[s][i + 1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    per_kernel = {k: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)]))
                  for i, k in enumerate(names)}
    return total_ms / steps, per_kernel


def interleaved_medians(devs, rounds, forms=("fused", "four", "combine")):
    """The pages' protocol for comparing configurations: one step of every
    (layer, form) per round, rounds repeated, the median over rounds of each
    (layer, form) and of each of its kernels.  devs: {name: DeviceLayer}."""
    import torch
    stream = torch.cuda.current_stream()
    order = [(n, f) for n in devs for f in forms]
    rec = {k: [] for k in order}
    for _ in range(rounds):
        for key in order:
            names, fns = _forms(devs[key[0]], key[1])
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
            ev[0].record(stream)
            for i, f in enumerate(fns):
                f()
                ev[i + 1].record(stream)
            rec[key].append((names, ev))
    torch.cuda.synchronize()
    out = {}
    for key, samples in rec.items():
        names = samples[0][0]
        step = [ev[0].elapsed_time(ev[-1]) for _, ev in samples]
        kern = {k: float(np.median([ev[i].elapsed_time(ev[i + 1]) for _, ev in samples]))
                for i, k in enumerate(names)}
        out[key] = (float(np.median(step)), kern)
    return out


def time_plans(D, L, chunk_rows, reps=5):
    """The plan built on the host (sort + upload, wall clock to completion) and
    on the device from device ids (GPU time of its launches), median of reps."""
    import torch
    from quantized_moe_expert_scatter_amd import _lib
    cfg = L.cfg
    ws = torch.empty_like(D.workspace)
    ids_dev = torch.from_numpy(np.ascontiguousarray(L.ids, np.int32).reshape(-1).copy()).cuda()
    host, dev = [], []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        p = _lib.moe_prefill_plan(L.ids, cfg.n_expert, chunk_rows, D.w_gu, D.w_dn, workspace=ws)
        torch.cuda.synchronize()
        host.append((time.perf_counter() - t0) * 1e3)
        p.close()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        p = _lib.moe_prefill_plan_device(ids_dev, cfg.tokens, cfg.topk, cfg.n_expert, chunk_rows,
                                         D.w_gu, D.w_dn, ws)
        e1.record()
        torch.cuda.synchronize()
        dev.append(e0.elapsed_time(e1))
        p.close()
    return {"host_ms": round(float(np.median(host)), 3), "device_ms": round(float(np.median(dev)), 3)}


def _load(path):
    with open(path) as f:
        return json.load(f)


def _record_sha(path):
    return _load(path).get("source_sha1")


def _source_sha(kernel):
    with open(os.path.join(ROOT, KERNEL_SOURCES[kernel]), "rb") as f:
        return hashlib.sha1(f.read()).hexdigest()


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    if _record_sha(path) != _source_sha(kernel):
        return None
    return _load(path).get("bytes_per_launch")


def issue_for(kernel, workload):
    """VALU and MFMA busy fractions of a kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"issue_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    if _record_sha(path) != _source_sha(kernel):
        return None
    rec = _load(path)
    return {k: rec[k] for k in ("valu_busy", "mfma_busy", "cycles_per_valu_instruction", "clock_ghz")}


def host_cpu():
    """The host's CPU model and logical CPU count (for the oracle's timing)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count()}


def run_cpu_baseline(L, threads, target_rows):
    from oracle import oracle
    cfg = L.cfg
    pl = oracle.plan(L.ids, cfg.n_expert, 64)
    row_e = pl.row_expert()
    # all rows of the first experts, so every sampled expert's weights are
    # decoded once for many rows, as in a whole layer
    n_e = int(np.searchsorted(pl.offsets, target_rows))
    n_e = max(1, min(n_e, cfg.n_expert))
    rows = np.arange(0, int(pl.offsets[n_e]), dtype=np.int32)
    t0 = time.perf_counter()
    xq = oracle.quantize_scatter(L.x, cfg.topk, pl.perm, rows=rows)
    gu = oracle.expert_product(L.w_gu.wtype, L.w_gu.buf, L.w_gu.offsets, cfg.n_expert,
                               2 * cfg.n_ff, cfg.hidden, L.w_gu.codebook, xq, row_e[rows],
                               n_threads=threads)
    hq = oracle.swiglu_q8(gu, cfg.n_ff)
    oracle.expert_product(L.w_down.wtype, L.w_down.buf, L.w_down.offsets, cfg.n_expert,
                          cfg.hidden, cfg.n_ff, L.w_down.codebook, hq, row_e[rows],
                          n_threads=threads)
    dt = time.perf_counter() - t0
    ms_layer = dt * 1e3 * cfg.rows / rows.size
    useful_ops = 2 * cfg.rows * (2 * cfg.n_ff * cfg.hidden + cfg.hidden * cfg.n_ff)
    return {"value": round(useful_ops / (ms_layer * 1e-3) / 1e12, 4), "unit": "effective int8 TOPS",
            "ms_per_layer": round(ms_layer, 1), "cores": threads, "kind": "oracle",
            "sample": f"{rows.size} of {cfg.rows} expert-sorted rows (all rows of experts "
                      f"0..{n_e - 1}) of the {cfg.name} layer, full chain, {dt:.1f} s wall, "
                      f"scaled by rows"}


def build_layers(names, layers, args, wl, DeviceLayer, torch, keep=()):
    """Every layer's seeded inputs generated and resident in HBM before any
    timing starts.  Returns {name: (cfg, host Layer or None, DeviceLayer,
    expert row counts, setup seconds)}; host inputs are kept only for `keep`."""
    out = {}
    for name in names:
        cfg = layers[name]
        print(f"[bench] {name}: generating inputs", file=sys.stderr, flush=True)
        L = wl.make_layer(cfg)
        t0 = time.perf_counter()
        D = DeviceLayer(L.x, L.ids, L.w_gu, L.w_down, chunk_rows=args.chunk_rows, route_w=L.route_w)
        torch.cuda.synchronize()
        setup_s = time.perf_counter() - t0
        counts = D.plan.query()[0]
        out[name] = (cfg, L if name in keep else None, D, counts, setup_s)
    return out


def warm(devs, steps):
    """Untimed steps of every layer, interleaved, until the clock has settled."""
    import torch
    for _ in range(steps):
        for D in devs.values():
            for f in _forms(D, "fused")[1]:
                f()
    torch.cuda.synchronize()


def layer_bytes(cfg, counts):
    """The layer's algorithmic HBM bytes as the method moves them (each
    counted once: X read, Xq write and read, GU write and read, Hq write and
    read, Dm write, the touched experts' weights), and the bytes of the path
    this library runs (GU never stored)."""
    by, _, _ = algorithmic(cfg, counts)
    method = sum(by[k] for k in KERNELS_4)
    return method, sum(by[k] for k in KERNELS)


def run_sweep(args, wl, DeviceLayer, torch):
    """ms/layer and effective TOPS over the sweep's layers, three- and
    four-launch forms, medians of interleaved rounds."""
    built = build_layers(list(wl.SWEEP), wl.SWEEP, args, wl, DeviceLayer, torch)
    devs = {n: v[2] for n, v in built.items()}
    warm(devs, args.warmup)
    med = interleaved_medians(devs, args.rounds, forms=("fused", "four"))
    out = {}
    for name, (cfg, _, D, counts, _) in built.items():
        n_chunks = D.plan.query()[3].shape[0]
        ms, pk = med[name, "fused"]
        ms4, pk4 = med[name, "four"]
        _, ops, _ = algorithmic(cfg, counts)
        useful = ops["expert_gate_up"] + ops["expert_down"]
        used = counts[counts > 0]
        out[name] = {"tokens": cfg.tokens, "routing": cfg.routing if cfg.routing != "lognormal"
                     else f"lognormal sigma {cfg.sigma}",
                     "experts_used": int(used.size), "rows_per_expert_median": float(np.median(used)),
                     "rows_per_expert_max": int(used.max()), "chunks": int(n_chunks),
                     "ms_per_layer": round(ms, 4), "tops": round(useful / (ms * 1e-3) / 1e12, 1),
                     "per_kernel_ms": {k: round(v, 4) for k, v in pk.items()},
                     "four_launch_ms": round(ms4, 4),
                     "four_launch_per_kernel_ms": {k: round(v, 4) for k, v in pk4.items()}}
        print(f"[sweep] {name}: {ms:.3f} ms (four-launch {ms4:.3f}) {out[name]['tops']} TOPS",
              file=sys.stderr, flush=True)
    for v in built.values():
        v[2].close()
    print(json.dumps({"metric": "ms/layer over the rows-per-expert sweep", "unit": "ms",
                      "n_gpus": 1, "chunk_rows": args.chunk_rows,
                      "timing": f"median of {args.rounds} interleaved rounds after {args.warmup} "
                                f"warm-up steps of every layer",
                      "layers": out}), flush=True)


def roofline(dom, by, ops, alu, pk, workload, cfg, counts, ms_layer):
    """The dominant kernel against the int8 matrix-core peak (the method's
    int8 operations: 2 x useful MACs) and the HBM peak (its algorithmic
    bytes), with the fp16 matrix-core peak it actually runs on and the vector
    ALU alongside; and the whole layer against HBM."""
    t = pk[dom] * 1e-3
    fr = {"hbm": (by[dom] / t / 1e9, HBM_PEAK_GBS, "GB/s")}
    if dom in ops:
        fr["mfma"] = (ops[dom] / t / 1e12, MFMA_I8_PEAK_TOPS, "TOP/s (int8)")
    bound = max(fr, key=lambda k: fr[k][0] / fr[k][1])
    if dom in ops:
        fr["mfma_fp16"] = (ops[dom] / t / 1e12, MFMA_F16_PEAK_TFLOPS, "TFLOP/s (fp16)")
        fr["alu"] = (alu[dom] / t / 1e12, VALU_F32_PEAK_TFLOPS, "TFLOP/s (fp32 vector)")
    ach, peak, unit = fr[bound]
    method_bytes, path_bytes = layer_bytes(cfg, counts)
    s = ms_layer * 1e-3
    return {"kernel": dom, "bound": bound, "achieved": round(ach, 1), "peak": round(peak, 1),
            "unit": unit, "frac": round(ach / peak, 3),
            "traffic": traffic_for(dom, workload),
            # what the counters say binds it: the share of SIMD cycles its VALU
            # and its matrix cores are busy (rocprofv3, committed summary)
            "issue": issue_for(dom, workload),
            "algorithmic_bytes_per_launch": int(by[dom]),
            "other_bounds": {k: {"achieved": round(v[0], 1), "peak": round(v[1], 1), "unit": v[2],
                                 "frac": round(v[0] / v[1], 3)} for k, v in fr.items() if k != bound},
            "layer_hbm": {"algorithmic_bytes": int(method_bytes),
                          "achieved_gbs": round(method_bytes / s / 1e9, 1),
                          "frac": round(method_bytes / s / 1e9 / HBM_PEAK_GBS, 3),
                          "path_bytes": int(path_bytes),
                          "path_frac": round(path_bytes / s / 1e9 / HBM_PEAK_GBS, 3)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the clock needs tens of ms of steady load to settle: 5 warm-up steps read
    # 0.63 ms at 2,048 tokens against 0.56 in steady state
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--rounds", type=int, default=15,
                    help="interleaved rounds whose medians give every layer's ms (the pages' protocol)")
    ap.add_argument("--workload", default="16k",
                    help="tiny | 2k | 8k | 16k | t128 | 2k_nl4, or a sweep layer sw<T>_<ln0.5|ln1.0|flat32>")
    ap.add_argument("--also", default="2k,8k,t128,2k_nl4", help="other layers reported alongside")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=6000)
    ap.add_argument("--cpu-rows-one-core", type=int, default=1000,
                    help="rows of the 2k layer for the one-core oracle time (when 2k is run)")
    ap.add_argument("--chunk-rows", type=int, default=128)
    ap.add_argument("--sweep", action="store_true",
                    help="instead: the rows-per-expert sweep (768..4096 tokens x lognormal "
                         "sigma 0.5 / 1.0 and flat 32-row routing), one JSON line of ms/layer")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1"}))
        sys.exit(2)

    import torch
    from quantized_moe_expert_scatter_amd import workloads as wl
    from quantized_moe_expert_scatter_amd.layer import DeviceLayer

    assert torch.cuda.is_available(), "bench needs the GPU"
    torch.cuda.set_device(0)
    if args.sweep:
        run_sweep(args, wl, DeviceLayer, torch)
        return
    layers = {**wl.CONFIGS, **wl.SWEEP}
    names = [args.workload] + [n for n in args.also.split(",") if n and n != args.workload]
    built = build_layers(names, layers, args, wl, DeviceLayer, torch, keep=(args.workload, "2k"))
    devs = {n: v[2] for n, v in built.items()}
    main_cfg, main_layer, main_dev, main_counts, _ = built[args.workload]

    # warm-up of every layer, then the contract's timed region on the headline layer
    print(f"[bench] warm-up: {args.warmup} steps of each layer", file=sys.stderr, flush=True)
    warm(devs, args.warmup)
    ms_main, pk_main = time_layer(main_dev, args.steps, 0)
    print(f"[bench] {args.workload}: {ms_main:.4f} ms/layer over {args.steps} steps {pk_main}",
          file=sys.stderr, flush=True)
    # every layer and form, medians over interleaved rounds
    med = interleaved_medians(devs, args.rounds)
    results = {}
    for name, (cfg, _, D, counts, setup_s) in built.items():
        by, ops, alu = algorithmic(cfg, counts)
        useful_ops = ops["expert_gate_up"] + ops["expert_down"]
        ms, pk = med[name, "fused"]
        ms4, pk4 = med[name, "four"]
        msc, pkc = med[name, "combine"]
        step_bytes = sum(by[k] for k in KERNELS)
        method_bytes, _ = layer_bytes(cfg, counts)
        results[name] = {"ms_per_layer": round(ms, 4), "tops": round(useful_ops / (ms * 1e-3) / 1e12, 1),
                         "per_kernel_ms": {k: round(v, 4) for k, v in pk.items()},
                         "algorithmic_bytes": int(step_bytes),
                         "hbm_floor_ms": round(step_bytes / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
                         "layer_hbm_frac": round(method_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
                         "four_launch": {"ms_per_layer": round(ms4, 4),
                                         "per_kernel_ms": {k: round(v, 4) for k, v in pk4.items()}},
                         "with_combine": {"ms_per_layer": round(msc, 4),
                                          "combine_ms": round(pkc["moe_combine"], 4),
                                          "combine_gbs": round(by["moe_combine"] /
                                                               (pkc["moe_combine"] * 1e-3) / 1e9, 1)},
                         "setup_s": round(setup_s, 2)}
        print(f"[bench] {name}: median {ms:.4f} ms/layer {results[name]['tops']} TOPS {pk}",
              file=sys.stderr, flush=True)
    for name, (cfg, L, D, counts, _) in built.items():
        results[name]["plan"] = time_plans(D, L if L is not None else wl.make_layer(cfg), args.chunk_rows)

    m = results[args.workload]
    by, ops, alu = algorithmic(main_cfg, main_counts)
    # the dominant kernel: the one with the largest share of the timed step
    dom = max(pk_main, key=pk_main.get)
    roof = roofline(dom, by, ops, alu, pk_main, args.workload, main_cfg, main_counts, ms_main)

    cpu = None
    if not args.no_cpu_baseline:
        threads = min(16, os.cpu_count() or 1)
        print(f"[bench] cpu baseline on {threads} threads", file=sys.stderr, flush=True)
        cpu = run_cpu_baseline(main_layer, threads, args.cpu_rows)
        if "2k" in built and built["2k"][1] is not None:
            # the same chain on one core, at 2,048 tokens
            print("[bench] cpu baseline on one core, 2k layer", file=sys.stderr, flush=True)
            cpu["one_core_2k"] = run_cpu_baseline(built["2k"][1], 1, args.cpu_rows_one_core)
        cpu["host"] = host_cpu()
    for v in built.values():
        v[2].close()

    useful_main = ops["expert_gate_up"] + ops["expert_down"]
    line = {
        "metric": METRIC,
        "value": round(useful_main / (ms_main * 1e-3) / 1e12, 1),
        "unit": "effective int8 TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_main, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded: X ~ N(0,1), uniform Q2_0 codes, fp16 scales U[0.01,0.05])",
        "config": {"workload": f"{main_cfg.name}: T={main_cfg.tokens}, hidden {main_cfg.hidden}, "
                               f"n_ff {main_cfg.n_ff}, {main_cfg.n_expert} experts, top-{main_cfg.topk} "
                               f"{main_cfg.routing}, gate/up {'Q2_0' if main_cfg.gu_type == 1 else 'NL4'}, down "
                               f"{'Q2_0' if main_cfg.down_type == 1 else 'NL4'}",
                   "tokens": main_cfg.tokens, "rows": main_cfg.rows, "chunk_rows": args.chunk_rows},
        "per_kernel_ms": {k: round(v, 4) for k, v in pk_main.items()},
        "hbm_floor_ms": m["hbm_floor_ms"],
        "timing": {"value": f"{args.steps} steps between two synchronizations after {args.warmup} "
                            f"warm-up steps of every layer",
                   "layers": f"median of {args.rounds} interleaved rounds (fused, four-launch and "
                             f"with-combine forms of every layer)"},
        "layers": {k: {kk: v[kk] for kk in ("ms_per_layer", "tops", "per_kernel_ms", "hbm_floor_ms",
                                            "layer_hbm_frac", "four_launch", "with_combine", "plan")}
                   for k, v in results.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
        # the pages' own figures for one layer (512 experts, top 10), measured on
        # an RTX 2080 Ti with real model weights: context, not a target
        "context": {"pages_ms_per_layer_rtx2080ti": PAGES_MS,
                    "ratio_to_pages": {k: round(PAGES_MS[k] / results[k]["ms_per_layer"], 2)
                                       for k in PAGES_MS if k in results}},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
