"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, the gate that
reports counter traffic only for the kernel sources it was measured on, the
percentile summary, and the bounded oracle baseline."""
import hashlib
import importlib.util
import os
import subprocess
import sys

import numpy as np

from long_context_kv_hs2_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    bench = load_bench()
    src = tmp_path / "kernel.hip"
    src.write_bytes(b"__global__ void k() {}\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", (str(src),))
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "traffic.md"
    prof.write_text(f"# summary\n\ntraffic_bytes_per_launch: 12345\nsource_sha256: {sha}\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", {2: str(prof)})
    assert bench.measured_traffic(2) == 12345
    assert bench.measured_traffic(3) is None  # no summary for this workload
    src.write_bytes(b"__global__ void k() { /* changed */ }\n")
    assert bench.measured_traffic(2) is None  # the kernel changed since the counters were taken


def test_committed_traffic_summaries_carry_their_fields():
    bench = load_bench()
    for workload, path in bench.TRAFFIC_PROFILE.items():
        text = open(os.path.join(ROOT, path), encoding="utf-8").read()
        fields = dict(line.split(": ", 1) for line in text.splitlines()
                      if line.startswith(("traffic_bytes_per_launch: ", "source_sha256: ")))
        assert int(fields["traffic_bytes_per_launch"]) > 0, path
        assert len(fields["source_sha256"].strip()) == 64, path
        assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text, path


def test_percentiles():
    bench = load_bench()
    assert bench.pct([]) is None
    p = bench.pct(np.arange(1, 101, dtype=np.float64))
    assert p["n"] == 100 and p["mean"] == 50.5 and p["median"] == 50.5
    assert p["p10"] < p["median"] < p["p90"]


def test_cpu_baseline_is_the_oracle_on_a_bounded_sample():
    bench = load_bench()
    d = inputs.make_decode(1)  # one 4096-token sequence
    cb = bench.cpu_baseline(d, budget_s=0.0)  # stops after the first sequence
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert cb["sample"].startswith("1 of 1 sequences (4096 context tokens)")
