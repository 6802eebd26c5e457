"""Host-side pieces of bench.py: the roofline arithmetic, the stored traffic
reader and the single-GPU guard. No device is touched."""

import hashlib
import os
import subprocess
import sys

import bench
from partitioned_kv_cache_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_attention_work_of_the_long_history_launch():
    """One launch of the long-history step: 18 layers, 8 query heads on one KV
    head of width 256, 51 suffix tokens, 256 pinned + 8 x 768 window tokens.
    Cached K and V are read once (2 x 18 x 6400 x 256 x 2 B), plus Q and the
    suffix K/V; QK^T and PV are 2 M T D flops each with M = 51 x 8 rows and
    T = 6400 + 51 keys."""
    s = configs.LONG_18L
    cached = s.pin_tokens + s.num_slots * s.tokens_per_frame
    assert cached == 6400
    algo, flops, kv = bench.attention_work(s, cached)
    assert kv == 117_964_800
    assert algo == 117_964_800 + 3_760_128 + 940_032 == 122_664_960
    assert flops == 4 * 408 * 6451 * 256 * 18 == 48_513_171_456


def _traffic_file(tmp_path, sha, value):
    p = tmp_path / "traffic.md"
    p.write_text(f"# counters\n\nsource_sha256: {sha}\ntraffic_bytes: {value}\n")
    return str(p)


def test_stored_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_bytes(b"__global__ void k() {}\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))

    monkeypatch.setattr(bench, "TRAFFIC_FILE", _traffic_file(tmp_path, sha, 172920193))
    assert bench.stored_traffic() == 172920193

    src.write_bytes(b"__global__ void k() { }\n")            # the kernel changed since the counters
    assert bench.stored_traffic() is None

    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.stored_traffic() is None


def test_committed_traffic_summary_is_readable():
    text = open(bench.TRAFFIC_FILE).read()
    fields = dict(l.split(":", 1) for l in text.splitlines() if l.startswith(("source_sha256:", "traffic_bytes:")))
    assert len(fields["source_sha256"].strip()) == 64
    assert int(fields["traffic_bytes"]) > 122_664_960        # at least the algorithmic bytes


def test_bench_measures_one_gpu_only():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert "one GPU only" in r.stdout + r.stderr
    assert not any(l.startswith("{") for l in r.stdout.splitlines())
