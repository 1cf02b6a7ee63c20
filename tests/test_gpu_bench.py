"""bench.py's one-line JSON contract, run in this process on the smallest layer
(fp32 tiny) and on a bf16 layer with preset overrides: every field the contract
names is there with the right type, and the timing fields agree with each other."""

import json

import pytest
import torch

import bench
from gpu_util import print_case

pytestmark = pytest.mark.gpu

CONTRACT = {"metric": str, "value": float, "unit": str, "n_gpus": int, "steps": int, "warmup": int,
            "ms_per_step": float, "higher_is_better": bool, "scaling": str, "dtype": str, "data": str,
            "config": dict, "roofline": dict}


def _run(capsys, argv):
    assert bench.main(argv) == 0
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, lines
    return json.loads(lines[0])


def _check_contract(rec, workload, steps, warmup):
    for key, typ in CONTRACT.items():
        assert isinstance(rec[key], typ), (key, rec.get(key))
    assert rec["n_gpus"] == 1 and rec["steps"] == steps and rec["warmup"] == warmup
    assert rec["higher_is_better"] is False and rec["unit"] == "ms/layer"
    assert rec["vs_baseline"] is None
    assert rec["config"]["workload"] == workload
    r = rec["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == bench.PEAK_BF16_TFLOPS
    assert r["achieved"] > 0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    # the pass contains its three steps
    assert rec["value"] > 0 and rec["t_attend_ms"] > 0 and rec["t_score_ms"] > 0 and rec["t_select_ms"] > 0
    assert rec["t_score_ms"] + rec["t_select_ms"] + rec["t_attend_ms"] <= rec["value"] * 1.05


def test_bench_line_tiny_with_cpu_baseline(capsys):
    assert torch.cuda.is_available()
    print_case("bench.py --config tiny --steps 3 --warmup 1 --no-ceiling (with the CPU oracle baseline)")
    rec = _run(capsys, ["--config", "tiny", "--steps", "3", "--warmup", "1", "--no-ceiling"])
    _check_contract(rec, "tiny", 3, 1)
    assert rec["dtype"] == "fp32"
    cpu = rec["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "ms/layer" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert isinstance(cpu["sample"], str) and cpu["sample"]


def test_bench_line_overrides(capsys):
    print_case("bench.py --config wan13b --heads 2 --temperature 2.0 --seed 5 --select-seed 7, no dense, no oracle")
    rec = _run(capsys, ["--config", "wan13b", "--heads", "2", "--temperature", "2.0", "--seed", "5",
                        "--select-seed", "7", "--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--no-dense",
                        "--no-ceiling"])
    _check_contract(rec, "wan13b", 2, 1)
    c = rec["config"]
    assert (c["H"], c["temperature"], c["seed"], c["select_seed"]) == (2, 2.0, 5, 7)
    assert rec["dtype"] == "bf16" and rec["cpu_baseline"] is None and rec["t_dense_ms"] is None
    assert rec["roofline"]["traffic"] is None  # counters were taken on the presets only
