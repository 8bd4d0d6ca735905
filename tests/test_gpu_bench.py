"""bench.py end to end on a small weight: the headline line it prints names
the kernel the timed launches ran -- the default tiling's, or the one given
with --tiling (W12 and the BF16 control alike) -- and carries a positive
rate and time."""
import json
import os
import subprocess
import sys

import pytest

from lossless_bit_weight_amd import w12

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*extra):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--no-sweep", "--no-stack",
           "--no-cpu-baseline", "--workload", "qkv_tp8", "--steps", "5", "--warmup", "2", *extra]
    print("bench:", " ".join(extra), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    assert len(line) < 2048
    return json.loads(line)


@pytest.mark.parametrize("M,tiling", [(4, None), (4, "0,1,2,4,1"), (16, "1,1,4,2,0,1,8")])
def test_bench_line_names_the_timed_kernel(M, tiling):
    out = _run("--m", str(M), *(["--tiling", tiling] if tiling else []))
    N, K = 896, 5120
    if tiling is None:
        want = w12.w12_gemm_variant(M, N, K)
    else:
        want = w12.w12_tiling_variant(M, N, K, tuple(int(v) for v in tiling.split(",")))
    assert want is not None
    assert out["roofline"]["kernel"] == want
    assert out["config"]["M"] == M and out["config"]["N"] == N and out["config"]["K"] == K
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["n_gpus"] == 1
