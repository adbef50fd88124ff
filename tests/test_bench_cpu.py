"""Host-side checks of bench.py's contract: the one-GPU rule and the counter lookup."""

import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True,
                          text=True, env=env, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_exits_with_a_message(args, env):
    r = run_bench(args, env)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line


def test_record_bytes():
    assert bench.rec_bytes(32) == (32 * 32 + 32) * 4 == 4224
    assert bench.rec_bytes(64) == (64 * 64 + 64) * 4


def committed_record():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic_minute_bf16.md")) as f:
        return json.loads(re.search(r"```json\n(.*?)\n```", f.read(), re.S).group(1))


def test_measured_traffic_follows_the_source_digest(monkeypatch):
    rec = committed_record()
    # counters taken on these sources: the recorded bytes, within a few percent of algorithmic
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: rec["kernel_sources_sha256"])
    alg = 374400 * 70 * 128 + 70 * 30 * bench.rec_bytes(32)
    for kernel in ("k_block_state", "k_readout"):
        t = bench.measured_traffic("minute_bf16", kernel)
        assert t == rec["kernels"][kernel]["traffic_bytes"]
        assert 0.99 * alg < t < 1.05 * alg
    # other sources: no figure
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 64)
    assert bench.measured_traffic("minute_bf16", "k_readout") is None
    assert bench.measured_traffic("no_such_workload", "k_readout") is None


def test_digest_covers_the_kernel_sources():
    d = bench.kernel_source_digest()
    assert re.fullmatch(r"[0-9a-f]{64}", d)
    assert set(bench.KERNEL_SOURCES) == {"la_kernels.hip", "la_internal.h", "la_api.cpp"}


def test_cpu_baseline_reports_the_oracle_and_the_host():
    """The cpu_baseline object of the bench line: the oracle timed on a bounded
    sample, with the worker count, the host's core count and CPU model beside it."""
    from linear_attention_video_relu_amd import workloads as W
    cfg = W.workload("tiny_f32")
    arrs = {x: W.draw(cfg, x) for x in W.TENSORS}
    r = bench.cpu_baseline(cfg, arrs, 2)
    assert r["kind"] == "oracle"
    assert r["unit"] == "tokens·heads/s" and r["value"] > 0
    assert r["workers"] == r["cores"] == min(2, r["host_cores"], bench.MAX_CPU_WORKERS)
    assert r["host_cores"] == len(os.sched_getaffinity(0))
    assert r["cpu_model"] is None or isinstance(r["cpu_model"], str)
    assert "2 of 2 (batch, head) streams of tiny_f32" in r["sample"]
    assert r["cpu_seconds"] >= 0 and r["wall_seconds"] > 0
