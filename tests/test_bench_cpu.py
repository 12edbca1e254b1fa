"""bench.py pieces that need no GPU: the one-GPU refusal and the traffic record."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "4"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 2
    assert "one GPU" in out.stderr


def test_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256_16": bench.kernel_source_hash(),
           "runs": {"headline/shared/interleaved/bf16": {"bytes_per_launch": 123}}}
    path = os.path.join(tmp_path, "t.json")
    with open(path, "w") as f:
        json.dump(rec, f)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", path)
    assert bench.measured_traffic("headline", "shared", "interleaved", "bf16") == 123
    assert bench.measured_traffic("headline", "per_head", "interleaved", "bf16") is None
    assert bench.measured_traffic("headline", "shared", "interleaved", "fp16") is None
    rec["kernel_source_sha256_16"] = "0" * 16
    with open(path, "w") as f:
        json.dump(rec, f)
    assert bench.measured_traffic("headline", "shared", "interleaved", "bf16") is None


@pytest.mark.parametrize("op,key", [("fuse_scale_shift", "adaln_wan/bf16/fp32/out"),
                                    ("group_norm_silu", "gn_vae_out/bf16/fp32/out")])
def test_step_traffic_records_follow_their_own_sources(tmp_path, op, key):
    rec = {"kernel_source_sha256_16": bench.kernel_source_hash(op),
           "runs": {key: {"bytes_per_launch": 77}}}
    path = os.path.join(tmp_path, "t.json")
    with open(path, "w") as f:
        json.dump(rec, f)
    assert bench.recorded_traffic(path, op, key) == 77
    assert bench.recorded_traffic(path, op, key + "x") is None
    other = "qknorm_rope" if op != "qknorm_rope" else "fuse_scale_shift"
    assert bench.kernel_source_hash(other) != bench.kernel_source_hash(op)
    assert bench.recorded_traffic(path, other, key) is None
