"""Host-side checks of bench.py's measurement contract (no GPU): the refusal
of a multi-GPU run, the work and byte counts the roofline uses, the gating of
the recorded HBM traffic on the kernel source, and the CPU baseline's record
(the oracle as it stands, timed on a tiny budget)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line


def test_work_counts_of_the_workload():
    # 3 chunks of 4680 tokens in the window plus the 4680-token sink from chunk 3 on
    assert [bench.keys_at(c) for c in (0, 1, 2, 3, 10)] == [4680, 9360, 14040, 18720, 18720]
    assert bench.attn_flops(18720) == 4 * 4680 * 18720 * 128 * 12
    # backward: S, dP and dQ over every key, dV and dK over the current chunk
    assert bench.backward_flops() == 2 * 128 * 12 * 4680 * (3 * 18720 + 2 * 4680)


def test_recorded_traffic_is_gated_on_the_kernel_digest(tmp_path, monkeypatch):
    rec = tmp_path / "rec.txt"
    rec.write_text("# counters\nkernel_source_sha256: abc123\ntraffic_bytes_per_launch: 214846898\n")
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(rec))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "abc123")
    assert bench.recorded_traffic() == 214846898
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "changed")
    assert bench.recorded_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(tmp_path / "missing.txt"))
    assert bench.recorded_traffic() is None


def test_kernel_digest_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) { return x + 1; }  // one\n")
    b.write_text("/* two */\nint f(int x)\n{\n  return x + 1;\n}\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    digests = []
    for p in (a, b, c):
        monkeypatch.setattr(bench, "KERNEL_SOURCE", str(p))
        digests.append(bench.kernel_source_digest())
    assert digests[0] == digests[1] != digests[2]


def test_cpu_baseline_record():
    res = bench.cpu_baseline(k_steps=2, warmup=4, budget_s=0.01)
    json.dumps(res)                         # one JSON line can carry it
    assert res["kind"] == "oracle" and res["unit"] == "latent frames/s"
    assert res["value"] > 0 and res["cores"] >= 1 and res["host_cpus"] >= 1
    assert "heads" in res["sample"] and "chunk 4" in res["sample"]
    for key in ("cpu_model", "blas", "s_per_call", "gflops_per_call", "tiny_fp32_8_chunks_s"):
        assert key in res
