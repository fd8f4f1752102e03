"""bench.py's contract parts that need no GPU: one GPU only (N > 1 exits with
a message and a non-zero status before touching the device), and the
options the driver passes."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "3",
                        "--warmup", "1"], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, r.stdout + r.stderr
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_options():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--workload", "--sweep"):
        assert opt in r.stdout


def test_cpu_baseline_leg_on_the_tiny_layer():
    """The oracle leg times whole experts' rows and scales by rows; on one
    core as on several it reports the fields the bench line carries."""
    sys.path.insert(0, ROOT)
    import bench
    from quantized_moe_expert_scatter_amd import workloads as wl
    L = wl.make_layer(wl.CONFIGS["tiny"])
    for threads in (1, 2):
        cpu = bench.run_cpu_baseline(L, threads, 40)
        assert cpu["kind"] == "oracle" and cpu["cores"] == threads
        assert cpu["unit"] == "effective int8 TOPS" and cpu["value"] > 0 and cpu["ms_per_layer"] > 0
        assert "of 128 expert-sorted rows" in cpu["sample"]
    host = bench.host_cpu()
    assert host["logical_cpus"] >= 1 and isinstance(host["model"], str)


def test_counter_records_apply_only_to_their_source(tmp_path, monkeypatch):
    """traffic and issue figures come from committed counter records, and only
    while the kernel file they were taken on is unchanged."""
    import hashlib
    sys.path.insert(0, ROOT)
    import bench
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "k.hip"
    src.write_text("// kernel\n")
    sha = hashlib.sha1(src.read_bytes()).hexdigest()
    (tmp_path / "profiles" / "traffic_k_w.json").write_text(
        json.dumps({"source_sha1": sha, "bytes_per_launch": 1234}))
    (tmp_path / "profiles" / "issue_k_w.json").write_text(json.dumps(
        {"source_sha1": sha, "valu_busy": 0.8, "mfma_busy": 0.3, "cycles_per_valu_instruction": 4.0,
         "clock_ghz": 2.0}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "k", "k.hip")
    assert bench.traffic_for("k", "w") == 1234
    assert bench.issue_for("k", "w")["valu_busy"] == 0.8
    assert bench.traffic_for("k", "other") is None and bench.issue_for("k", "other") is None
    src.write_text("// kernel, changed\n")
    assert bench.traffic_for("k", "w") is None and bench.issue_for("k", "w") is None


def test_layer_bytes_and_roofline_fields():
    """The layer's algorithmic bytes at the 16,384-token shape (every expert
    touched) are 5,541.7 MB: per (token, expert) row 28,480 B,
    per token 10,240 B, per expert 1,382,400 B of Q2_0 weights; the dominant
    kernel is placed against the int8 matrix-core peak and HBM."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    from quantized_moe_expert_scatter_amd import workloads as wl
    cfg = wl.CONFIGS["16k"]
    counts = np.full(cfg.n_expert, cfg.rows // cfg.n_expert, np.int64)
    method, path = bench.layer_bytes(cfg, counts)
    assert method == cfg.rows * 28480 + cfg.tokens * 10240 + cfg.n_expert * 1382400
    assert abs(method / 1e6 - 5541.7) < 0.1
    assert path == method - cfg.rows * 2 * 8 * cfg.n_ff          # GU is never stored
    by, ops, alu = bench.algorithmic(cfg, counts)
    pk = {"quantize_scatter": 0.13, "expert_gate_up_swiglu_q8": 1.5, "expert_down": 0.95}
    r = bench.roofline("expert_gate_up_swiglu_q8", by, ops, alu, pk, "none", cfg, counts, 2.58)
    assert r["bound"] == "mfma" and r["peak"] == 5000.0
    assert abs(r["achieved"] - ops["expert_gate_up_swiglu_q8"] / 1.5e-3 / 1e12) < 0.1
    assert set(r["other_bounds"]) == {"hbm", "mfma_fp16", "alu"}
    assert abs(r["layer_hbm"]["frac"] - method / 2.58e-3 / 8e12) < 1e-3
