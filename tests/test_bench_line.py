"""The benchmark's stdout line: one compact JSON object that carries the
roofline and the CPU baseline (built here from a made-up measurement; no GPU)."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from lossless_bit_weight_amd import inputs  # noqa: E402


def _fake():
    case = inputs.CASES["qkv"]
    head = {"workload": case.name, "M": 1, "w12_kernel": "w12_gemv_m1_r1_kw2_d4_xdirect",
            "bf16_kernel": "bf16_gemv_m1_r1_kw2_d4_xdirect", "w12_us": 10.4, "bf16_us": 12.6,
            "w12_weight_gbps": 5300.0, "w12_alg_gbps": 5325.0, "w12_alg_bytes": 55375872,
            "speedup_vs_bf16": 1.21, "launches": 400}
    sweep = []
    for name in ("qkv", "o", "gate_up", "down"):
        for M in (1, 2, 4, 8, 16, 32, 64, 128):
            sweep.append({"workload": inputs.CASES[name].name, "M": M,
                          "speedup_vs_bf16": 1.1 + 0.001 * M, "w12_us": 10.0 + M})
    cpu = {"value": 5.1, "unit": "GB/s", "cores": 16, "kind": "oracle",
           "sample": "99 full passes over QKV 7168x5120, M=1 (decode + fp64 GEMM), 12.1 s",
           "cpu_model": "AMD EPYC 9575F 64-Core Processor", "nproc": 256,
           "single_thread": {"value": 0.36, "unit": "GB/s", "sample": "x"},
           "pack": {"seconds": 0.2}, "stack_m1": {"layer_s": 1.0}}
    stack = {"by_m": [{"M": 1, "w12_ms": 5.42, "speedup_vs_bf16": 1.23}]}
    ceiling = ({"gbps": 5766.0}, {"gbps": 5800.0})
    return head, case, cpu, sweep, stack, ceiling


def test_headline_line_is_compact_and_complete():
    head, case, cpu, sweep, stack, ceiling = _fake()
    out = bench.headline_record(head, "qkv", case, 1, 40, 20, ceiling, 55630000, cpu, sweep, stack)
    line = json.dumps(out, separators=(",", ":"))
    assert "\n" not in line and len(line) < 2048, len(line)
    back = json.loads(line)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert key in back, key
    assert back["n_gpus"] == 1 and back["vs_baseline"] is None
    assert "workload" in back["config"] and "7168" in back["config"]["workload"]
    rf = back["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-4
    assert rf["traffic"] == 55630000
    cb = back["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == 16 and cb["value"] > 0 and cb["sample"]
    assert back["sweep_min_speedup_m1_32"]["M"] == 1   # smallest speedup at M <= 32
    assert abs(back["ms_per_step"] - 0.0104) < 1e-9


def test_headline_line_without_optional_parts():
    head, case, _, _, _, ceiling = _fake()
    out = bench.headline_record(head, "qkv", case, 1, 5, 20, ceiling, None, None, [], None)
    line = json.dumps(out, separators=(",", ":"))
    assert len(line) < 2048
    assert out["cpu_baseline"] is None and out["roofline"]["traffic"] is None
