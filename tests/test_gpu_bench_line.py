"""bench.py's JSON line on the GPU (needs an MI355X): a short run of the
32-layer OPT-6.7B launch shape (one layer, a few decode steps) and of the tiny
fp32 workload with its CPU-oracle leg, in this process, checked for the fields
the line promises and for the arithmetic that ties them together (rates from
byte and flop counts over measured times, fractions of the stated peaks and of
the measured ceilings)."""
import json
import math
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _run(monkeypatch, capsys, *args):
    monkeypatch.setattr(sys, "argv", ["bench.py", *args])
    bench.main()
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, lines
    return json.loads(lines[0])


def _close(a, b, rel=1e-9):
    return math.isclose(a, b, rel_tol=rel)


def test_default_shape_line(monkeypatch, capsys):
    print("bench line: opt6.7b-32L-b64, 1 layer, 8 decode steps", flush=True)
    r = _run(monkeypatch, capsys, "--layers", "1", "--decode-steps", "8", "--steps", "1", "--warmup", "1",
             "--no-cpu-baseline")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in r, key
    assert r["n_gpus"] == 1 and r["steps"] == 1 and r["warmup"] == 1
    assert r["unit"] == "tokens/s" and r["higher_is_better"] is True and r["vs_baseline"] is None
    assert r["dtype"] == "bf16" and r["data"] == "synthetic" and r["cpu_baseline"] is None
    c = r["config"]
    assert c["workload"] == "opt6.7b-32L-b64" and c["layers"] == 1 and c["decode_steps"] == 8
    assert (c["batch"], c["heads"], c["head_dim"], c["prompt_len"]) == (64, 32, 128, 2048)
    # value: generated tokens (batch x steps) over the whole step's time
    assert _close(r["value"], 64 * 8 / (r["ms_per_step"] / 1e3), 1e-6)

    rf = r["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["bytes_per_launch"] == 2048 * bench.decode_bytes_per_unit(410, 128, 2)
    assert rf["launches"] == 8
    assert _close(rf["achieved"], rf["bytes_per_launch"] / (rf["avg_launch_us"] * 1e-6) / 1e9, 1e-6)
    assert _close(rf["frac"], rf["achieved"] / rf["peak"])
    assert 0.0 < rf["frac"] < 1.0
    # a one-layer run is a profiling shape: no counter figure is attached
    assert rf["traffic"] is None
    mc = rf["measured_ceilings"]
    assert mc["launch_size_bytes"] == rf["bytes_per_launch"] // 256 * 256
    for key in ("read_GBps", "read_launch_size_GBps", "copy_GBps"):
        assert 0.0 < mc[key] < rf["peak"], (key, mc[key])
    assert _close(rf["frac_of_measured_read"], rf["achieved"] / mc["read_GBps"])
    assert _close(rf["frac_of_measured_read_launch_size"], rf["achieved"] / mc["read_launch_size_GBps"])

    p = r["prefill"]
    assert _close(p["mfma_frac"], p["mfma_tflops"] / 2500.0, 1e-6)
    assert _close(p["mfma_tflops"], 2048 * bench.prefill_flops_per_unit(2048, 128) / (p["ms"] * 1e-3) / 1e12, 1e-6)
    cc = p["measured_ceilings"]
    for key in ("mfma_only_TFs", "mix_TFs", "vector_only_TFs"):
        assert 0.0 < cc[key] < 2500.0 * 1.2, (key, cc[key])  # the dense peak is quoted at 2.4 GHz
    assert cc["mix_TFs"] <= cc["mfma_only_TFs"] * 1.05
    assert _close(p["frac_of_measured_mix"], p["mfma_tflops"] / cc["mix_TFs"])


def test_tiny_line_with_cpu_baseline(monkeypatch, capsys):
    print("bench line: tiny-fp32 with the CPU-oracle leg", flush=True)
    r = _run(monkeypatch, capsys, "--workload", "tiny-fp32", "--steps", "1", "--warmup", "1", "--cpu-units", "2")
    assert r["dtype"] == "f32" and r["config"]["workload"] == "tiny-fp32"
    cb = r["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s" and cb["value"] > 0.0
    assert 1 <= cb["cores"] <= 2  # one process per sampled unit at most
    assert cb["sample"].startswith("2 of 1 ") and "host" in cb
    par = r["parity"]
    assert par is not None and par["ok"], par
    assert par["units"] == 2 and par["max_out_err"] <= 2e-3 and par["max_score_rel"] <= 1e-4
