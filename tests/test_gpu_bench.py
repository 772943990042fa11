"""The bench line's contract: bench.py prints one JSON line per run with the keys a driver
reads, a roofline entry for the dominant kernel and, unless disabled, the oracle's
host-side baseline. Runs bench.main in this process with small step counts."""
import json
import os
import sys

import pytest

pytestmark = pytest.mark.gpu
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

REQUIRED = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
            "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"}
ROOF = {"bound", "achieved", "peak", "unit", "frac", "traffic"}
CPU = {"value", "unit", "cores", "host_cpus", "cpu_model", "kind", "sample"}


def _line(capsys, argv):
    bench.main(argv)
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, lines
    return json.loads(lines[0])


def _check(line, steps, warmup, workload):
    assert REQUIRED <= set(line), REQUIRED - set(line)
    assert line["n_gpus"] == 1 and line["steps"] == steps and line["warmup"] == warmup
    assert line["value"] > 0 and line["ms_per_step"] > 0
    assert line["higher_is_better"] is True and line["scaling"] == "weak"
    assert line["config"]["workload"] == workload
    assert "model" not in line["config"]
    roof = line["roofline"]
    assert ROOF <= set(roof), ROOF - set(roof)
    assert roof["bound"] in ("hbm", "mfma")
    assert roof["unit"] == ("GB/s" if roof["bound"] == "hbm" else "TFLOP/s")
    assert roof["achieved"] > 0 and roof["peak"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3


@pytest.mark.parametrize("workload", ["tiny_fp32", "fp8_small", "swiglu_small"])
def test_bench_line_with_oracle_baseline(capsys, workload):
    line = _line(capsys, ["--workload", workload, "--steps", "2", "--warmup", "1",
                          "--kernel-reps", "2", "--cpu-budget", "1"])
    _check(line, 2, 1, workload)
    cpu = line["cpu_baseline"]
    assert CPU <= set(cpu), CPU - set(cpu)
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert cpu["unit"] == line["unit"]
    if workload == "tiny_fp32":  # a small batch also reports the whole batch on one thread
        assert cpu["single_thread"]["value"] > 0


@pytest.mark.parametrize("workload", ["qwen3_bf16", "qwen3_pre_permute_bs64"])
def test_bench_line_full_size(capsys, workload):
    line = _line(capsys, ["--workload", workload, "--steps", "2", "--warmup", "1",
                          "--kernel-reps", "2", "--no-cpu-baseline"])
    _check(line, 2, 1, workload)
    assert "cpu_baseline" not in line
    if workload == "qwen3_bf16":  # a layer line: targets and the measured ceilings
        assert line["mfma_target"] == 0.60 and 0 < line["layer_mfma_frac"] < 1
        c = line["ceilings"]
        assert 1000 < c["hbm_read_GBs"] < 8000 and 500 < c["mfma_bf16_TFLOPs"] < 2600
        # L2-resident reads run well above the HBM read ceiling, in either load form
        assert c["l2_read_to_lds_GBs"] > c["hbm_read_GBs"]
        assert c["l2_read_to_registers_GBs"] > c["hbm_read_GBs"]
        assert line["roofline"]["measured_ceiling"] > 0
        assert line["step_ms"]["min"] <= line["step_ms"]["median"]


def test_bench_refuses_several_gpus(capsys):
    with pytest.raises(SystemExit):
        bench.main(["--gpus", "2"])
