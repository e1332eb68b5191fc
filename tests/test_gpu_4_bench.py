"""bench.py on the GPU: one run of the small fp32 workload prints one JSON line with every field of the
benchmark contract, a roofline for the dominant kernel and the CPU oracle baseline."""
import contextlib
import io
import json
import os
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    sys.path.insert(0, ROOT)
    import bench
    argv = sys.argv
    sys.argv = ["bench.py", "--workload", "tiny-fp32-T128-d512-E32-k4", "--steps", "3", "--warmup", "1",
                "--cpu-tokens", "8"]
    buf = io.StringIO()
    try:
        with contextlib.redirect_stdout(buf):
            bench.main()
    finally:
        sys.argv = argv
    lines = [l for l in buf.getvalue().splitlines() if l.strip()]
    assert len(lines) == 1, lines
    r = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in r, key
    assert r["n_gpus"] == 1 and r["steps"] == 3 and r["warmup"] == 1
    assert r["value"] > 0 and r["ms_per_step"] > 0
    assert r["config"]["workload"] == "tiny-fp32-T128-d512-E32-k4"
    roof = r["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] in ("hbm", "mfma", "alu") and roof["peak"] > 0 and roof["achieved"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) <= 1e-6 * max(1.0, roof["frac"])
    pk = r["peaks_measured"]
    for key in ("hbm_read_GBs", "mfma_bf16_TFLOPs", "mfma_fp8_TFLOPs", "gemm_bf16_TFLOPs"):
        assert pk[key] > 0, key
    # the sustained ceilings lie below the published peaks (8 TB/s; 2.5 / 5.0 PFLOP/s at the nominal clock)
    assert pk["hbm_read_GBs"] <= 8000 * 1.02 and pk["mfma_bf16_TFLOPs"] <= 2500 * 1.02
    assert pk["mfma_fp8_TFLOPs"] <= 5000 * 1.02
    if "peak_measured" in roof:
        assert abs(roof["frac_measured"] - roof["achieved"] / roof["peak_measured"]) <= 1e-6 * max(1.0, roof["frac_measured"])
    rt = r["layer"]["router"]
    assert rt["unit"] == "valu fp32" and rt["TFLOP_per_s"] > 0 and abs(rt["frac"] - rt["TFLOP_per_s"] / rt["peak_TFLOPs"]) < 1e-9
    cb = r["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cb, key
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1


@pytest.mark.parametrize("variant", ["route-limited", "route-grouped", "utilization"])
def test_bench_variant_json_line(variant):
    # the rows beyond the core layer, each one JSON line with a roofline and the oracle timed beside it
    sys.path.insert(0, ROOT)
    import bench
    argv = sys.argv
    sys.argv = ["bench.py", "--workload", "tiny-fp32-T128-d512-E32-k4", "--variant", variant, "--steps", "3",
                "--warmup", "1", "--no-peaks"]
    buf = io.StringIO()
    try:
        with contextlib.redirect_stdout(buf):
            bench.main()
    finally:
        sys.argv = argv
    lines = [l for l in buf.getvalue().splitlines() if l.strip()]
    assert len(lines) == 1, lines
    r = json.loads(lines[0])
    assert r["value"] > 0 and r["ms_per_step"] > 0 and r["n_gpus"] == 1
    roof = r["roofline"]
    assert roof["achieved"] > 0 and roof["peak"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) <= 1e-6 * max(1.0, roof["frac"])
    assert r["cpu_baseline"]["kind"] == "oracle" and r["cpu_baseline"]["value"] > 0
    if variant == "route-grouped":
        assert "group-limited" in r["metric"]
