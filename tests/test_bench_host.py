"""bench.py's host logic (no GPU): the one-GPU contract, the traffic lookup keyed by the kernel
sources' hash, and the CPU baseline record."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "8"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                       text=True, timeout=120, env={**os.environ, **env}, cwd=ROOT)
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "exactly one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_profiled_sources(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        entry = json.load(f)["c2:wgrad_gateup"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: entry["source_hash"])
    assert bench.load_traffic("wgrad_gateup", "c2") == entry["bytes_per_launch"]
    assert bench.load_traffic("wgrad_gateup", "c9") is None      # no such workload
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.load_traffic("wgrad_gateup", "c2") is None      # kernels changed since


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0 and h == bench.kernel_source_hash()


def test_cpu_baseline_record():
    import synth as Sy
    cfg = Sy.get_config("c1", T=32)
    x, w1, w2 = Sy.draw_x(cfg), Sy.draw_w1_all(cfg), Sy.draw_w2_all(cfg)
    rec = bench.cpu_baseline_fwd(cfg, x, w1, w2, Sy.draw_wg(cfg), None, Sy.draw_sel_bias(cfg), 16)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1 and "16 tokens" in rec["sample"]


def test_training_cpu_baseline_sample_has_no_padding():
    """One token in 32 of the uniformly routed 8192-token batch goes to 12 experts with exactly
    128 rows each (one whole block), so the timed oracle sample computes no padding rows."""
    import synth as Sy
    cfg = Sy.get_config("c2", H=128, I=64)
    x, w1, w2 = Sy.draw_x(cfg), Sy.draw_w1_all(cfg), Sy.draw_w2_all(cfg)
    rec = bench.cpu_baseline_fwd_bwd(cfg, x, w1, w2, Sy.uniform_logits(cfg), Sy.draw_dy(cfg), 32)
    assert rec["rows_useful"] == 256 * 6 and rec["rows_padded"] == rec["rows_useful"]
    assert rec["padded_over_useful"] == 1.0 and rec["cpu_model"]
    assert "one token in 32" in rec["sample"]


def test_clock_sampler_without_a_gpu_reports_nothing():
    c = bench.ClockSampler()
    with c:
        pass
    assert c.summary() is None or c.summary()["samples"] >= 1
