"""Host-side pieces of bench.py (no GPU): the JSON line's contract, the
roofline's choice of bound and its arithmetic, and the algorithmic byte and
FLOP counts of the five headline workloads against their closed forms
(2·L·M·N·K FLOP; each fp16 operand read once, each output written once)."""
import json
import os
import subprocess
import sys

import pytest

import bench
from dense_gemm_elementwise_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, FLOP, compulsory HBM bytes, epilogue bytes, bound at 2516.6 TFLOP/s and 8 TB/s)
HEADLINE = [
    ("aux_scale_128", 4_194_304, 163_840, 98_304, "hbm"),
    ("aux_scale_1024", 2_147_483_648, 10_485_760, 6_291_456, "hbm"),
    ("lincomb_2400x3232x4096", 63_543_705_600, 77_164_544, 31_027_200, "mfma"),
    ("x_acc_8192", 1_099_511_627_776, 805_306_368, 536_870_912, "mfma"),
    ("relu_square_16x2048x2048x1024", 137_438_953_472, 536_870_912, 402_653_184, "hbm"),
]


@pytest.mark.parametrize("name,flops,hbm,epi,bound", HEADLINE)
def test_workload_counts_and_bound(name, flops, hbm, epi, bound):
    w = workloads.WORKLOADS[name]
    assert w.flops == flops == 2 * w.L * w.M * w.N * w.K
    assert w.hbm_bytes == hbm
    assert w.epilogue_bytes == epi
    r = bench.roofline(w, 1.0)  # a 1 ms launch
    assert r["bound"] == bound
    if bound == "mfma":
        assert r["unit"] == "TFLOP/s" and r["peak"] == 2516.6
        assert r["achieved"] == pytest.approx(flops / 1e-3 / 1e12, abs=0.01)
    else:
        assert r["unit"] == "GB/s" and r["peak"] == 8000.0
        assert r["achieved"] == pytest.approx(hbm / 1e-3 / 1e9, abs=0.01)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    t_bound = max(flops / 2516.6e12, hbm / 8000e9)
    assert r["attainable_frac"] == pytest.approx(t_bound / 1e-3, abs=1e-4)


def test_result_line_contract():
    w = workloads.WORKLOADS[workloads.HEADLINE]
    g = {"ms_per_step": 0.9, "kernel_ms": 0.88, "launch_ms": {"median": 0.88, "min": 0.86, "mean": 0.88},
         "plan": {"bm": 256, "bn": 256, "bk": 64, "workgroups": 1024}}
    cpu = {"value": 0.08, "unit": "TFLOP/s", "cores": 16, "kind": "oracle", "sample": "rows"}
    line = bench.result_line(w, g, 50, 10, cpu)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 50 and line["warmup"] == 10
    assert line["value"] == pytest.approx(w.flops / 0.9e-3 / 1e12, abs=0.01)
    assert line["unit"] == "TFLOP/s" and line["higher_is_better"] is True
    assert line["vs_baseline"] is None and line["data"] == "synthetic" and line["dtype"] == "f16"
    assert line["config"]["workload"] == "x_acc_8192"
    assert set(line["roofline"]) >= {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert line["cpu_baseline"]["kind"] == "oracle"
    json.dumps(line)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_report_configurations_and_cpu_model():
    """The default line reports the five configurations (the headline plus
    four in "configs"), and the CPU baseline names the host's CPU model."""
    from dense_gemm_elementwise_amd import workloads
    assert len(workloads.CONFIGS) == 5 and workloads.HEADLINE in workloads.CONFIGS
    assert all(c in workloads.WORKLOADS for c in workloads.CONFIGS)
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)


def test_ragged_shapes_take_the_staged_path():
    """bench.py --ragged measures shapes off the 16-byte rule: each one's plan
    (host-only) stages operands for the fast kernel through a workspace."""
    import dense_gemm_elementwise_amd as ge
    base = 0x7F0000001000
    for (M, N, K, off) in bench.RAGGED_SHAPES:
        assert M % 8 or N % 8 or K % 8 or off % 8
        P = base + 2 * off
        rc, plan = ge.gemm_epi_plan_ws(1, M, N, K, P, P, P, None, None, None, "LINCOMB", P, None, None)
        assert rc == 0 and plan["vec"] == 1 and plan["workspace_bytes"] > 16384, (M, N, K, off, plan)
        rc, gen = ge.gemm_epi_plan(1, M, N, K, P, P, P, None, "LINCOMB", P, None)
        assert rc == 0 and gen["vec"] == 0  # without a workspace: the general kernel
