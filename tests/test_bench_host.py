"""Host-side behaviour of bench.py (no GPU): the single-GPU guard and the
counter-summary lookup behind roofline.traffic."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_only_for_the_profiled_sources_and_workload():
    """The summary's traffic is used only for its workload and while the GEMM
    sources hash to the value it records; otherwise None."""
    t = bench.measured_traffic("llama3-8b-bf16")
    with open(bench.COUNTERS) as fh:
        text = fh.read()
    if bench.kernel_source_hash() in text:
        assert isinstance(t, int) and t > 0
    else:
        assert t is None
    assert bench.measured_traffic("some-other-workload") is None


def test_wide_prefill_eligibility():
    import synth
    assert bench.wide_ok(synth.WORKLOADS["llama3-8b-bf16"]())
    assert bench.wide_ok(synth.WORKLOADS["llama3-8b-int8"]())
    assert bench.wide_ok(synth.WORKLOADS["llama3-8b-q8_0"]())
    assert bench.wide_ok(synth.WORKLOADS["llama3-8b-q4_0"]())
    assert not bench.wide_ok(synth.WORKLOADS["llama3-8b-q4_0-kvq4-32k"]())
    assert bench.wide_ok(synth.WORKLOADS["mixtral-8x7b-16slots"]())
