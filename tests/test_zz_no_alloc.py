"""dsa3d_backward_noalloc -- the backward with its scratch memory in a fixed
array of the library, for callers that cannot allocate -- against
dsa3d_backward with a workspace from the caller, through the C ABI.

Two calls in a row on one GPU, the second with a smaller problem (the array
keeps what the first call left), in both accumulation modes, for the
deformable path (several passes over the heads through the 64 MiB array) and
the fixed window. Deterministic runs must agree bit for bit; in the fast mode
dq and doffsets are still bitwise equal and dk/dv agree within the bf16
tolerance (their summation order may vary).
"""
import sys

import numpy as np
import pytest
import torch

import deformable_local_attention_amd as dsa
from deformable_local_attention_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16_TOL = 1e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _rel_l2(a, b):
    a, b = a.double(), b.double()
    return float((a - b).norm() / b.norm())


def _compare(wl, seed, det):
    say(f"[noalloc] {synth.describe(wl)} det={det} seed={seed}")
    x = synth.make_inputs(wl, DEV, seed=seed)
    offsets = x.get("offsets")
    out, lse = dsa.forward(x["q"], x["k"], x["v"], offsets, wl.window, wl.dilation)
    ref = dsa.backward(x["q"], x["k"], x["v"], offsets, out, lse, x["dout"], wl.window, wl.dilation,
                       deterministic=det)
    desc = dsa.desc_like(x["q"], wl.window, wl.dilation, 0.0, det)
    kind = dsa.WS_BACKWARD if offsets is not None else dsa.WS_BACKWARD_FIXED
    need = dsa.dsa3d_workspace_min(desc, kind)
    assert 0 < need <= dsa.NOALLOC_SCRATCH_BYTES
    say(f"    one-head pass {need / 2**20:.1f} MiB; recommended workspace "
        f"{dsa.dsa3d_workspace_size(desc, kind) / 2**20:.1f} MiB")
    dq, dk, dv = (torch.full_like(x["q"], float("nan")) for _ in range(3))
    doff = None if offsets is None else torch.full_like(offsets, float("nan"))
    dsa.dsa3d_backward_noalloc(desc, x["q"], x["k"], x["v"], offsets, out, lse, x["dout"], dq, dk, dv, doff)
    torch.cuda.synchronize()
    got = (dq, dk, dv, doff)
    for name, a, b in zip(("dq", "dk", "dv", "doff"), got, ref):
        if b is None:
            assert a is None
            continue
        same = torch.equal(_bits(a), _bits(b))
        if det or name in ("dq", "doff") or offsets is None:
            assert same, f"{name} differs from dsa3d_backward"
        else:
            err = _rel_l2(a, b)
            say(f"    {name}: rel-L2 {err:.2e} against dsa3d_backward (bitwise equal: {same})")
            assert err <= BF16_TOL
    return got


@pytest.mark.parametrize("det", [True, False])
def test_noalloc_matches_backward_two_calls_second_smaller(det):
    # 4 heads of 12,288 tokens x 75 points: ~30 MiB per head, so the 64 MiB
    # array takes two heads per pass; then a problem a tenth the size
    big = synth.Workload("noalloc-big", 1, 8, 32, 48, 4, 64, (3, 5, 5), (1, 1, 1), "bf16", "direct",
                         offset_sigma=2.0, backward=True, deterministic=det)
    small = synth.Workload("noalloc-small", 1, 4, 12, 20, 2, 64, (3, 3, 3), (1, 2, 2), "bf16", "direct",
                           offset_sigma=1.0, backward=True, deterministic=det)
    _compare(big, 61, det)
    _compare(small, 62, det)


def test_noalloc_fixed_window_two_calls_second_smaller():
    big = synth.Workload("noalloc-fixed-big", 1, 6, 20, 40, 3, 128, (3, 7, 7), (1, 1, 1), "bf16", "none",
                         backward=True)
    small = synth.Workload("noalloc-fixed-small", 1, 3, 5, 9, 2, 32, (3, 3, 3), (1, 1, 2), "f32", "none",
                           backward=True)
    _compare(big, 63, False)
    _compare(small, 64, False)
