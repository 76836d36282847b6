"""The benchmark's JSON line on the GPU: the fields its contract names.

A short run (two timed steps, no CPU baseline, no clock sample) of the
headline forward and of the backward, each printing exactly one JSON line
whose metric, units, step counts, roofline block and workload config are
those the benchmark documents.  The throughput itself is not checked here.
"""
import json

import pytest

import bench
from exact_attention_04_amd.workloads import WORKLOADS


def _line(capsys, argv):
    assert bench.main(argv) == 0
    out = [l for l in capsys.readouterr().out.splitlines() if l.strip()]
    assert len(out) == 1, out
    return json.loads(out[0])


@pytest.mark.gpu
def test_forward_line(capsys):
    d = _line(capsys, ["--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--no-clock"])
    assert d["metric"] == bench.METRIC
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True
    assert (d["n_gpus"], d["steps"], d["warmup"]) == (1, 2, 1)
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert d["config"]["workload"] == "sdpa_b4h32n4096d128_bf16_causal"
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == bench.PEAK_TFLOPS["bf16"]
    assert r["achieved"] > 0 and r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    # the traffic record under profiles/ matches the kernel source, so the line carries it
    assert r["traffic"] is not None and r["traffic"] > r["algorithmic_bytes_per_launch"] * 0.9
    assert d["cpu_baseline"] is None


@pytest.mark.gpu
def test_backward_line(capsys):
    d = _line(capsys, ["--pass", "bwd", "--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--no-clock"])
    assert d["unit"] == "TFLOP/s" and (d["n_gpus"], d["steps"], d["warmup"]) == (1, 2, 1)
    assert d["config"]["pass"] == "bwd" and d["config"]["workload"] == "sdpa_b4h32n4096d128_bf16_causal"
    r = d["roofline"]
    assert r["flop_per_launch"] == pytest.approx(2.5 * bench.workload_flops(WORKLOADS["sdpa_b4h32n4096d128_bf16_causal"]), rel=1e-12)
    assert r["achieved"] > 0 and r["traffic"] is not None
    assert "clock" not in d and d["cpu_baseline"] is None
