"""bench.py's host logic: algorithmic bytes and flops, the kernel-code hash
that keys the recorded HBM traffic, and the one-GPU contract. No GPU needed."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from deformable_local_attention_amd import synth  # noqa: E402


def test_headline_algorithmic_bytes_and_flops_per_token():
    # 24 heads x 128, P = 75, bf16: each tensor read or written once; the
    # backward's 8d + 6P elements + 4 B and the forward's 4d + 3P elements + 4 B
    # per (token, head) make 106,320 B per token; flops 32dP + 80dP per
    # (token, head) make 25.8 MFLOP per token.
    wl = synth.WORKLOADS["1080p-bf16-p75-det"]
    alg = bench.algorithmic(wl)
    assert (alg["fwd_bytes"] + alg["bwd_bytes"]) * wl.heads == 106_320
    assert (alg["fwd_flops"] + alg["bwd_flops"]) * wl.heads == 25_804_800
    # the per-kernel flops add up to the whole step
    assert alg["forward_flops"] == alg["fwd_flops"]
    assert alg["bwd_query_flops"] + alg["bwd_key_flops"] == alg["bwd_flops"]
    # bytes per unit of the three kernels: forward reads q, k, v and the
    # offsets and writes o and lse; the query kernel reads q, k, v, o, dO, the
    # offsets and lse and writes dq and doffsets; the key kernel reads q, dO and
    # writes dk, dv
    d, P = wl.head_dim, wl.P
    assert alg["forward"] == 4 * d * 2 + 3 * P * 2 + 4
    assert alg["bwd_query"] == 6 * d * 2 + 6 * P * 2 + 4
    assert alg["bwd_key"] == 4 * d * 2


def test_fixed_window_accounting():
    wl = synth.WORKLOADS["1080p-bf16-fixed377"]
    alg = bench.algorithmic(wl)
    d, P = wl.head_dim, wl.P
    assert alg["fwd_flops"] == 4 * d * P
    assert alg["bwd_query_flops"] + alg["bwd_key_flops"] == alg["bwd_flops"] == 10 * d * P


def test_fixed_window_matrix_core_eligibility():
    """The shapes bench.py reports against the MFMA peak are those the library
    runs on the matrix cores (bf16, 32-256 channels forward, 32-128 backward,
    undilated w, k_w <= 17; two rows per wave where h is undilated)."""
    wl = synth.WORKLOADS["1080p-bf16-fixed377"]
    assert bench.fixed_on_mfma(wl) == {"forward": 2, "bwd_query": 2, "bwd_key": 1}
    mk = lambda **kw: synth.Workload("f", 1, 2, 3, 4, kw.get("heads", 2), kw.get("d", 64), kw.get("win", (3, 7, 7)),
                                     kw.get("dil", (1, 1, 1)), kw.get("dtype", "bf16"), "none", backward=True)
    assert bench.fixed_on_mfma(mk(d=64)) == {"forward": 2, "bwd_query": 2, "bwd_key": 2}
    assert bench.fixed_on_mfma(mk(d=256)) == {"forward": 1}
    assert bench.fixed_on_mfma(mk(dil=(1, 2, 1))) == {"forward": 1, "bwd_query": 1, "bwd_key": 1}
    assert bench.fixed_on_mfma(mk(dtype="f32")) is None
    assert bench.fixed_on_mfma(mk(d=16)) is None
    assert bench.fixed_on_mfma(mk(dil=(1, 1, 2))) is None
    assert bench.fixed_on_mfma(mk(win=(1, 1, 19))) is None
    # a grid row of all heads at 2 GiB or more leaves the buffer loads' 31-bit record range
    wide = synth.Workload("f", 1, 1, 1, 2**16, 128, 128, (3, 7, 7), (1, 1, 1), "bf16", "none", backward=True)
    assert bench.fixed_on_mfma(wide) is None
    assert bench.fixed_on_mfma(wide.with_grid(W=2**16 - 1)) is not None
    assert bench.fixed_on_mfma(synth.WORKLOADS[synth.HEADLINE]) is None


def test_code_hash_ignores_comments_and_layout():
    a = "int f(int x) {  // first\n    return x + 1; /* block\n comment */ }\n"
    b = "int f(int x)\n{\n    return x + 1;\n}\n"
    c = "int f(int x) { return x + 2; }"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
    files = {f: open(os.path.join(ROOT, "deformable_local_attention_amd", "csrc", f)).read()
             for f in bench.ATTN_SOURCES}
    h = bench.kernel_source_hash(lambda f: files[f])
    assert h == bench.kernel_source_hash()
    edited = dict(files)
    edited["dsa3d_bwd.hip"] = "// a new comment line\n" + files["dsa3d_bwd.hip"]
    assert bench.kernel_source_hash(lambda f: edited[f]) == h
    edited["dsa3d_bwd.hip"] = files["dsa3d_bwd.hip"].replace("kScanItems = 16", "kScanItems = 8", 1)
    assert bench.kernel_source_hash(lambda f: edited[f]) != h


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout == ""
