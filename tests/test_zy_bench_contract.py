"""The benchmark's output contract: one JSON line with the fields a round's
measurement is read from, the one-GPU guard, and the CPU baseline leg (the
oracle timed on a bounded sample).  Named to run after the parity tests."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_leg_on_the_smallest_workload():
    w = wl.workload(0)
    parents = wl.trees(w, w.seed)
    lens = wl.lengths(w, w.seed)
    logits, tokens, _ = wl.logits_and_drafts(w, parents, w.seed)
    cb = bench.cpu_baseline(w, parents, lens, logits, tokens, w.seed, 0.5)
    import oracle
    assert cb["kind"] == "oracle" and cb["cores"] == oracle.default_threads()
    assert cb["single_thread"]["cores"] == 1
    assert cb["unit"] == "verified tree nodes/s" and cb["cpu_model"]
    for leg in (cb, cb["single_thread"]):
        assert np.isfinite(leg["value"]) and leg["value"] > 0
        parts = leg["est_parts_s"]
        step = parts["mask"] + w.layers * parts["attention_per_layer"] + parts["accept"] + parts["commit"]
        assert leg["value"] == pytest.approx(w.B * w.M / step)
    assert str(int(lens.sum())) in cb["sample"]


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_the_contract_fields():
    print("bench.py --workload 0 --steps 2 --warmup 1 --no-cpu-baseline", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "0", "--steps", "2",
                        "--warmup", "1", "--no-cpu-baseline"], capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    w = wl.workload(0)
    assert d["metric"] == bench.METRIC
    assert d["unit"] == "verified tree nodes/s" and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["vs_baseline"] is None and d["dtype"] == w.dtype
    assert d["config"]["workload"] == w.name
    assert d["ms_per_step"] > 0
    assert d["value"] == pytest.approx(w.B * w.M / (d["ms_per_step"] * 1e-3))
    for key in ("roofline", "roofline_attention"):
        roof = d[key]
        for f in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
            assert f in roof
    ra = d["roofline_attention"]
    assert ra["frac"] == pytest.approx(ra["achieved"] / ra["peak"])
    t = d["timing"]
    for k in ("mask_us", "attention_us_per_layer", "accept_us", "commit_us", "step_us"):
        assert t[k]["p10"] <= t[k]["p50"] <= t[k]["p90"] and t[k]["p50"] > 0, k
    assert t["attention_us_per_layer"]["mean"] == pytest.approx(d["attn_us_per_layer"])
    assert d["copy_GBps"] > 0
    cold = d["attention_cold"]
    assert cold["copies"] >= 2 and cold["us_per_call"] > 0
