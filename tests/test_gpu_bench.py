"""The benchmark's output contract on the GPU: one JSON line with the metric,
tokens/s, the dominant kernel against its roofline and the per-kernel
launch times, for small workloads of each kind (run as child processes)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    print(f"[bench] {' '.join(args)}", file=sys.stderr, flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.parametrize("workload,kernels", [("tiny-f32", {"forward", "bwd_query", "bwd_key"}),
                                              ("small-bf16-proj", {"forward", "proj_forward"})])
def test_bench_line(workload, kernels):
    j = _bench("--workload", workload, "--steps", "2", "--warmup", "1", "--cpu-baseline", "off")
    assert j["n_gpus"] == 1 and j["steps"] == 2 and j["warmup"] == 1
    assert j["value"] > 0 and j["ms_per_step"] > 0 and j["higher_is_better"] is True
    assert j["config"]["workload"] == workload
    assert j["dtype"] == ("f32" if workload == "tiny-f32" else "bf16")
    assert kernels <= set(j["kernels"])
    for key in ("roofline", "roofline_hbm"):
        r = j[key]
        assert r["bound"] in ("alu", "hbm", "mfma") and r["peak"] > 0 and r["achieved"] > 0
        assert abs(r["frac"] - r["achieved"] / r["peak"]) <= 1e-4
    # tokens/s is the whole grid over the step time (ms_per_step is printed to 3 decimals)
    n = _tokens(j)
    assert abs(j["value"] * j["ms_per_step"] / 1e3 - n) <= n * (0.0006 / j["ms_per_step"] + 1e-4)


def _tokens(j):
    B, T, H, W = j["config"]["grid"]
    return B * T * H * W
