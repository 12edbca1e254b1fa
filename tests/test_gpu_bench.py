"""bench.py's one-line JSON report, end to end on the GPU (a few steps).

The report's fields are a contract with the tools that read it: the metric,
the whole-job value and its unit, the run's shape, the roofline object of the
dominant kernel and the CPU-oracle baseline.
"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [l for l in out.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, out.stdout
    return json.loads(lines[0])


def test_default_report_carries_every_field():
    r = run_bench("--steps", "5", "--warmup", "2", "--cpu-seconds", "0.2")
    assert r["metric"].startswith("QK-norm+RoPE")
    assert r["unit"] == "GB/s" and r["value"] > 0
    assert (r["n_gpus"], r["steps"], r["warmup"]) == (1, 5, 2)
    assert r["higher_is_better"] is True and r["scaling"] == "weak"
    assert r["vs_baseline"] is None and r["data"] == "synthetic" and r["dtype"] == "f32"
    assert r["ms_per_step"] > 0
    cfg = r["config"]
    assert cfg["workload"].startswith("headline") and (cfg["tokens"], cfg["heads"],
                                                        cfg["head_dim"]) == (32760, 40, 128)
    roof = r["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None or roof["traffic"] > 0
    cpu = r["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s" and cpu["value"] > 0
    assert cpu["cores"] >= 1 and cpu["sample"]
    assert r["kernel"]["scratch_bytes"] == 0


@pytest.mark.parametrize("op", ["fuse_scale_shift", "group_norm_silu"])
def test_step_reports(op):
    r = run_bench("--op", op, "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    assert r["unit"] == "GB/s" and r["value"] > 0 and r["roofline"]["bound"] == "hbm"
    assert r["config"]["parallelism"] == "single GPU"


@pytest.mark.parametrize("mode", ["clean", "dirty"])
def test_graph_and_flush_modes(mode):
    """--graph adds the per-call time replayed from a captured HIP graph;
    --flush evicts the caches before each call (by reading 1 GiB, or with
    --flush-mode dirty by writing it) and reports the per-call rate."""
    g = run_bench("--workload", "tiny", "--graph", "--steps", "20", "--warmup", "2",
                  "--no-cpu-baseline")
    assert g["graph_us_per_call"] > 0
    f = run_bench("--workload", "mid", "--flush", "--flush-mode", mode, "--steps", "5",
                  "--warmup", "1", "--no-cpu-baseline")
    assert "cache flushed (%s)" % mode in f["config"]["workload"]
    assert abs(f["value"] - f["roofline"]["achieved"]) <= 0.1
    assert f["pct_of_peak_median"] > 0


@pytest.mark.parametrize("extra", [(), ("--workload", "flux", "--flush")])
def test_floor_report(extra):
    """--op floor times the pass beside its no-arithmetic access-pattern
    probes (a library of their own) in two rounds, for a fused buffer and
    for separate q and k with flushed caches; the pass cannot beat the probe
    that moves the same bytes the same way."""
    r = run_bench("--op", "floor", "--steps", "10", "--warmup", "2", *extra)
    legs = set(r["legs"])
    want = {"pass", "floor_table", "floor_phase", "floor_wave", "floor_wave_uncapped",
            "floor_qk", "read_only", "write_only", "copy"}
    assert legs == (want if extra else want | {"floor_flat"})
    assert len(r["rounds"]) == 2 and all(set(x) == legs for x in r["rounds"])
    b = r["best_us"]
    assert all(v > 0 for v in b.values())
    assert r["value"] == round(b["pass"] / b["floor_table"], 4)
    assert r["value"] > 0.9


@pytest.mark.parametrize("workload", ["adaln_wan", "gn_vae_out"])
def test_floor_report_for_the_row_steps(workload):
    """--op floor on an AdaLN or group-norm workload times the step beside
    out-of-place probes of its bytes (capped and uncapped), the bytes read
    alone and written alone, and a device copy."""
    r = run_bench("--op", "floor", "--workload", workload, "--steps", "10", "--warmup", "2")
    legs = set(r["legs"])
    assert legs == {"pass", "floor_oop", "floor_oop_uncapped", "read_only", "write_only", "copy"}
    assert len(r["rounds"]) == 2 and all(set(x) == legs for x in r["rounds"])
    b = r["best_us"]
    assert all(v > 0 for v in b.values())
    assert r["value"] == round(b["pass"] / min(b["floor_oop"], b["floor_oop_uncapped"]), 4)
    assert r["value"] > 0.8

