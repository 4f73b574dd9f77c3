"""GPU parity of hybrid attention -- the local 3D-DSA samples plus G global
tokens per (batch, head) in one softmax -- through the C ABI against the
oracle's hybrid functions, on whole small grids and at full size.

Acceptance as for the operator: float32 max |err| <= 1e-4, bf16 rel-L2
<= 1e-2 per tensor (lse within 1e-3), the oracle fed the same inputs.
"""
import sys

import numpy as np
import pytest
import torch

import deformable_local_attention_amd as dsa
import oracle
from deformable_local_attention_amd import synth
from deformable_local_attention_amd.chain import Chain
from gpu_helpers import rel_l2, to_np, to_np32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _check(name, gpu, ref, dtype):
    if dtype == "f32":
        err = float(np.abs(gpu - ref).max()) if gpu.size else 0.0
        say(f"    {name}: max abs err {err:.3e} (tolerance 1e-4)")
        assert err <= 1e-4, f"{name}: {err:.3e}"
    else:
        err = rel_l2(gpu, ref)
        say(f"    {name}: rel-L2 err {err:.3e} (tolerance 1e-2)")
        assert err <= 1e-2, f"{name}: {err:.3e}"


def _wl(B=1, T=3, H=4, W=5, heads=2, d=32, window=(3, 3, 3), dil=(1, 1, 1), dtype="f32", sigma=1.0, G=4,
        offsets="direct", det=False):
    return synth.Workload("hybrid", B, T, H, W, heads, d, window, dil, dtype, offsets, offset_sigma=sigma,
                          backward=True, deterministic=det, global_tokens=G)


def _run_whole(wl, seed, det=None, ws_bytes=None):
    say(f"[hybrid] {synth.describe(wl)} det={det} ws={ws_bytes}")
    x = synth.make_inputs(wl, "cpu", seed=seed)
    xd = {k: v.to(DEV) for k, v in x.items()}
    ch = Chain(wl, xd, bwd_workspace_bytes=ws_bytes, deterministic=det)
    ch.run()
    torch.cuda.synchronize()
    off = (to_np32(x["offsets"]) if "offsets" in x
           else np.zeros(tuple(x["q"].shape[:5]) + (wl.P, 3), dtype=np.float32))
    args = (to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), off, to_np(x["gk"]), to_np(x["gv"]))
    o, lse = oracle.forward_hybrid(*args, wl.window, wl.dilation)
    _check("o", to_np(ch.out), o, wl.dtype)
    lerr = float(np.abs(to_np(ch.lse) - lse).max())
    assert lerr <= (1e-4 if wl.dtype == "f32" else 1e-3), lerr
    dq, dk, dv, doff, dgk, dgv = oracle.backward_hybrid(*args, to_np(x["dout"]), wl.window, wl.dilation)
    for name, g, r in (("dq", ch.dq, dq), ("dk", ch.dk, dk), ("dv", ch.dv, dv), ("dgk", ch.dgk, dgk),
                       ("dgv", ch.dgv, dgv)):
        _check(name, to_np(g), r, wl.dtype)
    if ch.doff is not None:
        _check("doff", to_np(ch.doff), doff, wl.dtype)
    return ch


# global rows: fewer than one staged chunk, several chunks (d = 64 bf16 stages
# 256 rows, d = 256 f32 32 rows), one row, the fixed window, ragged batches
CASES = {
    "f32-G1": dict(G=1),
    "f32-b2-h3-d16-G5": dict(B=2, T=3, H=5, W=7, heads=3, d=16, sigma=1.5, G=5),
    "bf16-p75-d128-G64": dict(T=5, H=6, W=9, heads=2, d=128, window=(3, 5, 5), sigma=2.0, dtype="bf16", G=64),
    "bf16-d64-dil-G300": dict(T=4, H=7, W=6, heads=2, d=64, window=(3, 3, 3), dil=(1, 2, 2), sigma=0.6,
                              dtype="bf16", G=300),
    "f32-d256-G40": dict(T=2, H=3, W=4, heads=1, d=256, G=40),
    "f32-d8-p1-G3": dict(T=3, H=4, W=5, heads=2, d=8, window=(1, 1, 1), sigma=0.5, G=3),
    "bf16-fixed377-G8": dict(T=3, H=9, W=20, heads=2, d=128, window=(3, 7, 7), dtype="bf16", G=8, offsets="none"),
    # bf16 rows of 32/64/128 channels take the matrix-core kernels: ragged key
    # slices and staging rounds, several query blocks per head, several slabs
    "bf16-d32-b2-h3-G17": dict(B=2, T=3, H=5, W=7, heads=3, d=32, sigma=1.5, dtype="bf16", G=17),
    "bf16-d128-G1": dict(T=3, H=4, W=6, heads=2, d=128, dtype="bf16", G=1),
    "bf16-d64-G100-slabs": dict(T=4, H=12, W=20, heads=2, d=64, sigma=1.0, dtype="bf16", G=100),
    "bf16-d128-G70-blocks": dict(T=5, H=12, W=11, heads=1, d=128, window=(3, 5, 5), sigma=2.0, dtype="bf16",
                                 G=70),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("det", [False, True])
def test_hybrid_whole_grid(name, det):
    _run_whole(_wl(det=det, **CASES[name]), seed=91, det=det)


def test_hybrid_multi_pass_and_bitwise_reproducible():
    """The smallest workspace (one head per pass of the local backward) and the
    default one give the same bits in deterministic mode, against the oracle."""
    wl = _wl(T=4, H=6, W=9, heads=4, d=64, window=(3, 5, 5), sigma=2.0, dtype="bf16", G=48, det=True)
    desc = dsa.make_desc(wl.B, wl.T, wl.H, wl.W, wl.heads, wl.head_dim, wl.window, wl.dilation, torch.bfloat16,
                         0.0, True)
    small = dsa.dsa3d_hybrid_workspace_min(desc, wl.global_tokens, dsa.WS_BACKWARD)
    full = dsa.dsa3d_hybrid_workspace_size(desc, wl.global_tokens, dsa.WS_BACKWARD)
    assert 0 < small < full
    outs = []
    for ws in (full, small, full):
        ch = _run_whole(wl, seed=92, det=True, ws_bytes=ws)
        outs.append([t.clone() for t in (ch.out, ch.lse, ch.dq, ch.dk, ch.dv, ch.doff, ch.dgk, ch.dgv)])
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_hybrid_rejects_bad_global_counts():
    wl = _wl(G=4)
    x = {k: v.to(DEV) for k, v in synth.make_inputs(wl, "cpu", seed=93).items()}
    desc = dsa.desc_like(x["q"], wl.window)
    out, lse = torch.empty_like(x["q"]), torch.empty(x["q"].shape[:5], dtype=torch.float32, device=DEV)
    for G in (0, 1025):
        g = torch.zeros((1, G, wl.heads, wl.head_dim), dtype=torch.float32, device=DEV)
        with pytest.raises(dsa.DSA3DError):
            dsa.dsa3d_forward_hybrid(desc, x["q"], x["k"], x["v"], x["offsets"], G, g, g, out, lse)
    assert dsa.dsa3d_hybrid_workspace_size(desc, 0, dsa.WS_BACKWARD) == 0


@pytest.mark.slow
def test_1080p_p75_hybrid64_workload_full_size_sampled():
    """The 1080p 3x5x5 workload with 64 global tokens per head in the bench's
    launch configuration: queries and keys through the full-size parity driver
    (the oracle's joint softmax), dgk/dgv of the first and last head summed by
    the oracle over all 2,088,960 queries."""
    from test_gpu_parity import _free, _full_size_parity
    wl = synth.WORKLOADS["1080p-bf16-p75-hybrid64"]
    say(f"[full] {synth.describe(wl)}")
    xd = synth.make_inputs(wl, DEV)
    ch = Chain(wl, xd)
    ch.run()
    torch.cuda.synchronize()
    _full_size_parity("1080p-bf16-p75-hybrid64", wl, xd, ch.offsets, ch.out, ch.lse, dq=ch.dq, dk=ch.dk, dv=ch.dv,
                      doff=ch.doff, dout=xd["dout"], seed=17, global_rows=(xd["gk"], xd["gv"]), dgk=ch.dgk,
                      dgv=ch.dgv, k_heads=[0, 9, wl.heads - 1], n_random_k_heads=256)
    del ch, xd
    _free()
