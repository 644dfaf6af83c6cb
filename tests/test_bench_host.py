"""Host logic of bench.py (no GPU): the reduction of per-process step times
to the line's figures, the roofline arithmetic, the multi-GPU refusal, and
the counter-summary lookup that gives a roofline its traffic."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(step_ms, gate_up_ms, launches, graph=None):
    return {"step_ms": step_ms, "total_ms": float(np.sum(step_ms)), "steps": len(step_ms),
            "warmup": 2, "T": 8, "step_bytes": 8e8, "step_flops": 2e9,
            "graph_ms": graph, "eager_ms": graph and float(np.median(step_ms)),
            "kernels": {"ffn_i8_gate_up": {"launches": launches, "total_ms": gate_up_ms},
                        "combine": {"launches": launches, "total_ms": 0.004 * launches}},
            "roofline": {"bound": "hbm", "kernel": "ffn_i8_gate_up", "bytes_per_launch": 5e8,
                         "launches_per_step": 1.0, "traffic": None},
            "config": {"workload": "w"}, "dtype": "int8", "data": "synthetic"}


def test_summarize_reduces_processes_and_prices_the_roofline():
    runs = [_run([0.20, 0.10, 0.30], gate_up_ms=0.27, launches=3),    # median 0.20, 90 us
            _run([0.16, 0.16, 0.17], gate_up_ms=0.24, launches=3),    # median 0.16, 80 us
            _run([0.50, 0.18, 0.19], gate_up_ms=0.30, launches=3)]    # median 0.19, 100 us
    out = bench.summarize(runs)
    # the median of the three process medians, not of the pooled steps
    assert out["ms_per_step"] == pytest.approx(0.19)
    pooled = [0.20, 0.10, 0.30, 0.16, 0.16, 0.17, 0.50, 0.18, 0.19]
    assert out["ms_p10"] == pytest.approx(np.percentile(pooled, 10))
    assert out["ms_p90"] == pytest.approx(np.percentile(pooled, 90))
    assert out["processes"] == 3
    assert out["tokens_per_s"] == pytest.approx(8 / 0.19e-3, rel=1e-4)
    assert out["hbm_gbps_algorithmic"] == pytest.approx(8e8 / 0.19e-3 / 1e9, rel=1e-4)
    assert out["tflops_algorithmic"] == pytest.approx(2e9 / 0.19e-3 / 1e12, rel=1e-3)
    # per-kernel duration: the median over processes of each one's mean launch
    assert out["kernels"]["ffn_i8_gate_up"]["avg_us"] == pytest.approx(90.0)
    roof = out["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] == pytest.approx(5e8 / 90e-6 / 1e9, rel=1e-4)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 8000.0, abs=1e-4)
    assert roof["avg_launch_us"] == pytest.approx(90.0)


def test_summarize_mfma_roofline_and_graph_timing():
    r = _run([0.5, 0.5], gate_up_ms=2.0, launches=2, graph=0.45)
    r["roofline"] = {"bound": "mfma", "kernel": "ffn_i8_gate_up", "flops_per_launch": 7e11,
                     "launches_per_step": 1.0, "traffic": 123}
    out = bench.summarize([r])
    roof = out["roofline"]
    assert roof["unit"] == "TFLOP/s" and roof["peak"] == bench.INT8_PEAK_TOPS
    assert roof["achieved"] == pytest.approx(7e11 / 1e-3 / 1e12, rel=1e-4)
    assert roof["frac_of_bf16_peak"] == pytest.approx(roof["achieved"] / 2500.0, abs=1e-4)
    assert roof["traffic"] == 123
    assert out["hip_graph_ms_per_step"] == pytest.approx(0.45)


def test_summarize_without_the_dominant_kernel_has_no_roofline():
    r = _run([0.3], gate_up_ms=0.1, launches=1)
    r["roofline"]["kernel"] = "ffn_i8_gate_up_gemm"  # not timed in this run
    assert bench.summarize([r])["roofline"] is None


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_counter_traffic_needs_the_current_kernel_source(tmp_path, monkeypatch):
    import hashlib
    src = os.path.join(ROOT, "sparse_moe_expert_sigmoid_amd", "csrc", "ffn.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    body = ("# summary\n\n| a | b |\n|---|---|\n\ndominant_kernel: gate_up_kernel<1, 1>\n"
            "traffic_bytes_per_launch: 4242\nkernel_source_sha256: {}\n")
    (prof / "wl__gate_up.md").write_text(body.format(sha))
    (prof / "old__gate_up.md").write_text(body.format("0" * 64))
    # the lookup reads <ROOT>/profiles and <ROOT>/sparse_moe_expert_sigmoid_amd/csrc
    csrc = tmp_path / "sparse_moe_expert_sigmoid_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "ffn.hip").write_bytes(open(src, "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic("wl", "gate_up_kernel<") == 4242
    assert bench.counter_traffic("wl", "down_kernel<") is None     # another kernel
    assert bench.counter_traffic("old", "gate_up_kernel<") is None  # stale source
    assert bench.counter_traffic("none", "gate_up_kernel<") is None
