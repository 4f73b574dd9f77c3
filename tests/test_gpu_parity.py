"""GPU parity: libdsa3d on an MI355X against the CPU oracle, element by element.

Acceptance: sample corners bit-exact; float32 runs max |err| <= 1e-4 on every
output; bf16 runs ||gpu - oracle|| / ||oracle|| <= 1e-2 per output tensor
(lse, always float32, within 1e-3 absolute), with the oracle fed the same bf16
values widened exactly. Small grids are checked whole; the full-size
workloads on sampled queries and key tokens, in the same launch configuration
as the benchmark.
"""
import json
import math
import os
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import deformable_local_attention_amd as dsa
from deformable_local_attention_amd import synth
from deformable_local_attention_amd.chain import Chain
from gpu_helpers import (HeadOracle, errors, face_tokens, gather, grid_corner_tokens, interior_tokens,
                         oracle_dkdv_at_keys, oracle_queries, random_tokens, rel_l2, rows_at, sample_queries, to_np,
                         to_np32)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F32_TOL = 1e-4
BF16_TOL = 1e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _wl(name="case", B=1, T=3, H=4, W=5, heads=2, d=32, window=(3, 3, 3), dil=(1, 1, 1), dtype="f32",
        sigma=1.0, backward=True, det=False):
    return synth.Workload(name, B, T, H, W, heads, d, window, dil, dtype, "direct", offset_sigma=sigma,
                          backward=backward, deterministic=det)


def _check(name, gpu, ref, dtype, tol_f32=F32_TOL, tol_bf16=BF16_TOL):
    if dtype == "f32":
        err = float(np.abs(gpu - ref).max()) if gpu.size else 0.0
        say(f"    {name}: max abs err {err:.3e} (tolerance {tol_f32})")
        assert err <= tol_f32, f"{name}: max abs err {err:.3e} > {tol_f32}"
    else:
        err = rel_l2(gpu, ref)
        say(f"    {name}: rel-L2 err {err:.3e} (tolerance {tol_bf16})")
        assert err <= tol_bf16, f"{name}: rel-L2 err {err:.3e} > {tol_bf16}"
    return err


def _run_whole(wl, x, det=None, ws_bytes=None):
    """Run the chain on the GPU and the oracle on the whole grid; compare all."""
    say(f"[parity] {synth.describe(wl)} det={det}")
    xd = {k: v.to(DEV) for k, v in x.items()}
    ch = Chain(wl, xd, bwd_workspace_bytes=ws_bytes, deterministic=det)
    ch.run()
    torch.cuda.synchronize()
    off = (to_np32(ch.offsets) if ch.offsets is not None
           else np.zeros(tuple(x["q"].shape[:5]) + (wl.P, 3), dtype=np.float32))  # fixed window
    o, lse = oracle.forward(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), off, wl.window, wl.dilation)
    _check("o", to_np(ch.out), o, wl.dtype)
    lerr = float(np.abs(to_np(ch.lse) - lse).max())
    assert lerr <= (F32_TOL if wl.dtype == "f32" else 1e-3), f"lse err {lerr}"
    if wl.backward:
        dq, dk, dv, doff = oracle.backward(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), off, to_np(x["dout"]),
                                           wl.window, wl.dilation)
        _check("dq", to_np(ch.dq), dq, wl.dtype)
        _check("dk", to_np(ch.dk), dk, wl.dtype)
        _check("dv", to_np(ch.dv), dv, wl.dtype)
        if ch.doff is not None:
            _check("doff", to_np(ch.doff), doff, wl.dtype)
    return ch


# ---------------------------------------------------------------------------
# whole-grid parity on small and ragged grids
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("det", [False, True])
def test_tiny_f32_workload(det):
    wl = synth.WORKLOADS["tiny-f32"]
    _run_whole(wl, synth.make_inputs(wl, "cpu"), det=det)


CASES = {
    "f32-ragged-b2-h3-d16": dict(B=2, T=3, H=5, W=7, heads=3, d=16, sigma=1.5),
    "bf16-ragged-p75-d128": dict(T=5, H=6, W=9, heads=2, d=128, window=(3, 5, 5), sigma=2.0, dtype="bf16"),
    "bf16-odd-b2-p75-d128": dict(B=2, T=3, H=7, W=5, heads=3, d=128, window=(3, 5, 5), sigma=2.0, dtype="bf16"),
    "bf16-single-token-d128": dict(T=1, H=1, W=1, heads=2, d=128, window=(3, 5, 5), sigma=1.0, dtype="bf16"),
    "f32-p1-d8": dict(T=4, H=5, W=6, heads=2, d=8, window=(1, 1, 1), sigma=0.7),
    "f32-d256-dil": dict(T=2, H=3, W=4, heads=1, d=256, window=(3, 3, 3), dil=(2, 1, 3), sigma=1.0),
    "bf16-d64-513": dict(T=4, H=7, W=6, heads=3, d=64, window=(5, 1, 3), dil=(1, 2, 2), sigma=0.3, dtype="bf16"),
    "bf16-d32-wide": dict(T=3, H=9, W=11, heads=2, d=32, window=(3, 7, 7), sigma=3.0, dtype="bf16"),
    "f32-single-token": dict(T=1, H=1, W=1, heads=2, d=32, sigma=0.4),
    "f32-window-wider-than-grid": dict(T=2, H=2, W=3, heads=1, d=64, window=(5, 5, 7), sigma=0.8),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("det", [False, True])
def test_small_grids(name, det):
    wl = _wl(name, **CASES[name])
    _run_whole(wl, synth.make_inputs(wl, "cpu", seed=7), det=det)


@pytest.mark.parametrize("fill", ["zero", "integer", "huge", "nan", "inf", "beyond2p30", "tiny_negative"])
def test_special_offsets(fill):
    wl = _wl("special-" + fill, T=3, H=4, W=5, heads=2, d=32, sigma=1.0)
    x = synth.make_inputs(wl, "cpu", seed=11)
    off = x["offsets"]
    g = torch.Generator().manual_seed(5)
    if fill == "zero":
        off.zero_()
    elif fill == "integer":
        off.copy_(torch.randint(-3, 4, off.shape, generator=g).float())
    elif fill == "huge":
        off.fill_(1.0e6)
    elif fill == "nan":
        off[..., ::2, :] = float("nan")
    elif fill == "inf":
        off[..., 1::3, 0] = float("inf")
        off[..., 2::3, 2] = -float("inf")
    elif fill == "beyond2p30":
        off[..., ::2, 1] = 3.0e9
    elif fill == "tiny_negative":
        off.fill_(-1e-9)
        off[..., 1::2, :] = 1e-9
    _run_whole(wl, x, det=False)
    _check_geometry(wl, x["offsets"])


def test_every_sample_in_one_cell_deterministic():
    """Offsets that move every sample of every query to the same cell: one
    bucket of T*H*W*P samples per head, which takes the large-bucket sort."""
    wl = _wl("one-cell", T=3, H=4, W=5, heads=2, d=32, window=(3, 3, 3), dtype="f32", det=True)
    x = synth.make_inputs(wl, "cpu", seed=23)
    kt, kh, kw = wl.window
    it, ih, iw = np.meshgrid(np.arange(kt), np.arange(kh), np.arange(kw), indexing="ij")
    win = np.stack([it.ravel() - 1, ih.ravel() - 1, iw.ravel() - 1], 1)          # [P, 3]
    grid = np.stack(np.meshgrid(np.arange(wl.T), np.arange(wl.H), np.arange(wl.W), indexing="ij"), -1)
    ref = grid[:, :, :, None, :] + win[None, None, None]                           # [T,H,W,P,3]
    target = np.array([1.25, 2.5, 2.75])
    off = (target - ref).astype(np.float32)                                        # exact in f32
    x["offsets"].copy_(torch.from_numpy(off)[None, :, :, :, None].expand(x["offsets"].shape))
    say(f"[one-cell] {synth.describe(wl)}: {wl.T * wl.H * wl.W * wl.P} samples per head in one cell")
    ch = _run_whole(wl, x, det=True)
    first = [t.clone() for t in (ch.dk, ch.dv)]
    ch.run()
    torch.cuda.synchronize()
    assert torch.equal(first[0], ch.dk) and torch.equal(first[1], ch.dv)


def test_bucket_sizes_across_the_sort_paths():
    """Buckets of chosen sizes on both sides of each sort path's limit (128
    records: ranked by one wave; 512: bitonic network of one wave; beyond:
    one block per bucket), in deterministic mode, against the oracle and
    bitwise reproducible."""
    wl = _wl("bucket-sizes", T=4, H=5, W=6, heads=1, d=32, window=(3, 3, 3), dtype="f32", det=True)
    x = synth.make_inputs(wl, "cpu", seed=29)
    sizes = [2, 64, 127, 128, 129, 200, 512, 513]
    cells = [(0, 0, 0), (1, 1, 1), (2, 2, 2), (3, 3, 3), (0, 4, 5), (1, 0, 4), (2, 3, 1), (3, 1, 4)]
    kt, kh, kw = wl.window
    it, ih, iw = np.meshgrid(np.arange(kt), np.arange(kh), np.arange(kw), indexing="ij")
    win = np.stack([it.ravel() - 1, ih.ravel() - 1, iw.ravel() - 1], 1)          # [P, 3]
    grid = np.stack(np.meshgrid(np.arange(wl.T), np.arange(wl.H), np.arange(wl.W), indexing="ij"), -1)
    ref = (grid[:, :, :, None, :] + win[None, None, None]).reshape(-1, 3)          # samples in flat order
    off = x["offsets"][0, :, :, :, 0].reshape(-1, 3).numpy().copy()
    s = 0
    for n, cell in zip(sizes, cells):
        for j in range(s, s + n):
            frac = np.array([((j * 37 + a * 11) % 7 + 1) / 8.0 for a in range(3)])
            off[j] = (np.array(cell) + frac - ref[j]).astype(np.float32)           # exact in f32
        s += n
    assert s <= len(off)
    off[s:] = 1.0e6  # the other samples fall outside the grid: the buckets hold exactly these sizes
    x["offsets"][0, :, :, :, 0] = torch.from_numpy(off).reshape(wl.T, wl.H, wl.W, wl.P, 3)
    say(f"[bucket-sizes] {synth.describe(wl)}: buckets of {sizes} samples")
    ch = _run_whole(wl, x, det=True)
    first = [t.clone() for t in (ch.dk, ch.dv)]
    ch.run()
    torch.cuda.synchronize()
    assert torch.equal(first[0], ch.dk) and torch.equal(first[1], ch.dv)


def _check_geometry(wl, off_cpu):
    desc = dsa.desc_like(torch.empty((wl.B, wl.T, wl.H, wl.W, wl.heads, wl.head_dim), dtype=wl.torch_dtype),
                         wl.window, wl.dilation)
    offd = off_cpu.to(DEV)
    base = torch.empty(offd.shape, dtype=torch.int32, device=DEV)
    frac = torch.empty(offd.shape, dtype=torch.float32, device=DEV)
    dsa.dsa3d_debug_geometry(desc, offd, base, frac)
    torch.cuda.synchronize()
    ob, of = oracle.geometry(to_np32(off_cpu), wl.window, wl.dilation)
    assert np.array_equal(base.cpu().numpy(), ob), "sample base corners differ"
    assert np.array_equal(frac.cpu().numpy().view(np.int32), of.view(np.int32)), "sample fractions differ"


@pytest.mark.parametrize("name", ["tiny-f32", "bf16-ragged-p75-d128", "bf16-d64-513"])
def test_geometry_is_bit_exact(name):
    wl = synth.WORKLOADS["tiny-f32"] if name == "tiny-f32" else _wl(name, **CASES[name])
    say(f"[geometry] {synth.describe(wl)}")
    _check_geometry(wl, synth.make_inputs(wl, "cpu", seed=13)["offsets"])


# ---------------------------------------------------------------------------
# determinism of the K/V gradients
# ---------------------------------------------------------------------------

def test_deterministic_mode_is_bitwise_reproducible_across_runs_and_pass_splits():
    wl = _wl("det-p75", T=6, H=12, W=20, heads=4, d=128, window=(3, 5, 5), sigma=2.0, dtype="bf16", det=True)
    say(f"[determinism] {synth.describe(wl)}")
    x = {k: v.to(DEV) for k, v in synth.make_inputs(wl, "cpu", seed=17).items()}
    desc = dsa.desc_like(x["q"], wl.window, wl.dilation, 0.0, True)
    full = dsa.dsa3d_workspace_size(desc, dsa.WS_BACKWARD)
    one = dsa.dsa3d_workspace_min(desc, dsa.WS_BACKWARD)
    assert 3 * one < full <= 4 * one  # one pass of 4 heads; then 1 and 3 heads per pass
    outs = []
    for ws in (full, full, one, 3 * one):
        ch = Chain(wl, x, bwd_workspace_bytes=ws)
        ch.run()
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (ch.out, ch.lse, ch.dq, ch.dk, ch.dv, ch.doff)])
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("det", [False, True])
def test_multi_pass_backward_against_oracle(det):
    """The backward with the smallest workspace it accepts (one head per pass:
    four passes) and with room for two heads (two passes), against the oracle
    on the whole grid."""
    wl = _wl("multi-pass", T=4, H=6, W=9, heads=4, d=64, window=(3, 5, 5), sigma=2.0, dtype="bf16", det=det)
    x = synth.make_inputs(wl, "cpu", seed=53)
    desc = dsa.desc_like(x["q"], wl.window, wl.dilation, 0.0, det)
    one = dsa.dsa3d_workspace_min(desc, dsa.WS_BACKWARD)
    full = dsa.dsa3d_workspace_size(desc, dsa.WS_BACKWARD)
    assert full > 3 * one
    for ws in (one, 2 * one + 256):
        say(f"[multi-pass] workspace {ws} B ({ws / one:.2f} x the one-head minimum)")
        _run_whole(wl, x, det=det, ws_bytes=ws)


# ---------------------------------------------------------------------------
# fixed window (offsets NULL: every offset zero)
# ---------------------------------------------------------------------------

# (dtype, B, T, H, W, heads, d, window, dilation): the pages' 3x7x7 window on
# ragged grids, a dilated 3x3x3 window, a window wider than the grid. bf16
# rows of 32-256 channels with an undilated w axis and k_w <= 17 take the
# matrix-core forward: a row shorter than one wave's 16 tokens, rows of
# 16 + 16 + 5 tokens, the widest band (k_w = 17), k_w = 1 with dilated t and
# h, 256 channels, a window wider than the grid, one token per batch item;
# k_w = 19 and a dilated w axis take the vector kernels.
@pytest.mark.parametrize("case", [("f32", 2, 3, 5, 11, 2, 32, (3, 7, 7), (1, 1, 1)),
                                  ("bf16", 1, 4, 9, 13, 3, 128, (3, 7, 7), (1, 1, 1)),
                                  ("bf16", 2, 3, 4, 37, 2, 128, (3, 7, 7), (1, 1, 1)),
                                  ("bf16", 1, 2, 3, 40, 2, 64, (1, 3, 17), (1, 1, 1)),
                                  ("bf16", 1, 6, 7, 20, 3, 32, (3, 3, 1), (2, 3, 1)),
                                  ("bf16", 1, 2, 3, 18, 1, 256, (1, 3, 5), (1, 1, 1)),
                                  ("bf16", 1, 2, 3, 25, 2, 64, (1, 1, 19), (1, 1, 1)),
                                  ("bf16", 1, 2, 2, 3, 2, 64, (5, 5, 7), (1, 1, 1)),
                                  ("bf16", 2, 1, 1, 1, 3, 128, (3, 7, 7), (1, 1, 1)),
                                  ("bf16", 1, 5, 8, 10, 2, 64, (3, 3, 3), (1, 2, 2)),
                                  ("f32", 1, 2, 3, 4, 1, 8, (3, 7, 7), (2, 1, 1))])
def test_fixed_window_whole(case):
    dt, B, T, H, W, nh, d, win, dil = case
    wl = synth.Workload("fixed", B, T, H, W, nh, d, win, dil, dt, "none", backward=True)
    _run_whole(wl, synth.make_inputs(wl, "cpu", seed=41))


@pytest.mark.parametrize("d", [64, 128])
def test_fixed_window_matrix_core_path_is_bitwise_reproducible(d):
    """Every sum of the matrix-core kernels runs over the window in a fixed
    order: two runs give the same bits, and the backward leaves the forward's
    outputs untouched."""
    wl = synth.Workload("fixed", 1, 4, 9, 37, 2, d, (3, 7, 7), (1, 1, 1), "bf16", "none", backward=True)
    x = {k: v.to(DEV) for k, v in synth.make_inputs(wl, "cpu", seed=47).items()}
    outs = []
    for _ in range(2):
        ch = Chain(wl, x)
        ch.run()
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (ch.out, ch.lse, ch.dq, ch.dk, ch.dv)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fixed_window_equals_general_path_at_zero_offsets(dtype):
    """offsets NULL and a zero offsets tensor. The vector kernels (f32) give
    the same forward and dq bits; the matrix-core forward (bf16) sums in
    another order and agrees within the tolerance; dk/dv are summed in another
    order (per key window instead of per cell)."""
    wl = synth.Workload("fixed", 1, 4, 6, 9, 2, 64, (3, 7, 7), (1, 1, 1), dtype, "none", backward=True)
    x = {k: v.to(DEV) for k, v in synth.make_inputs(wl, "cpu", seed=43).items()}
    zeros = torch.zeros(tuple(x["q"].shape[:5]) + (wl.P, 3), dtype=x["q"].dtype, device=DEV)
    o_f, lse_f = dsa.forward(x["q"], x["k"], x["v"], None, wl.window)
    o_g, lse_g = dsa.forward(x["q"], x["k"], x["v"], zeros, wl.window)
    dq_f, dk_f, dv_f, doff_f = dsa.backward(x["q"], x["k"], x["v"], None, o_f, lse_f, x["dout"], wl.window)
    dq_g, dk_g, dv_g, _ = dsa.backward(x["q"], x["k"], x["v"], zeros, o_g, lse_g, x["dout"], wl.window)
    torch.cuda.synchronize()
    assert doff_f is None
    if dtype == "f32":
        assert torch.equal(o_f, o_g)
        assert torch.equal(lse_f, lse_g)
        assert torch.equal(dq_f, dq_g)
        assert float((dk_f - dk_g).abs().max()) <= F32_TOL and float((dv_f - dv_g).abs().max()) <= F32_TOL
    else:
        assert rel_l2(to_np(o_f), to_np(o_g)) <= BF16_TOL
        assert float((lse_f - lse_g).abs().max()) <= 1e-3
        assert rel_l2(to_np(dq_f), to_np(dq_g)) <= BF16_TOL
        assert rel_l2(to_np(dk_f), to_np(dk_g)) <= BF16_TOL and rel_l2(to_np(dv_f), to_np(dv_g)) <= BF16_TOL
    # NULL offsets need NULL doffsets
    desc = dsa.desc_like(x["q"], wl.window)
    ws = dsa._workspace(desc, dsa.WS_BACKWARD_FIXED, DEV)
    with pytest.raises(dsa.DSA3DError):
        dsa.dsa3d_backward(desc, x["q"], x["k"], x["v"], None, o_f, lse_f, x["dout"], dq_f, dk_f, dv_f, zeros, ws)


# ---------------------------------------------------------------------------
# offset projection
# ---------------------------------------------------------------------------

# (heads, head_dim, grid): 3 heads give F = 243, which takes the 128x128 kernel
# for every product; 8 heads (F = 648, C = 512) take the bf16 256x256 kernel
# for all three, with ragged M, N and K tiles (1,380 tokens; 648 = 2.5 tiles;
# K = 648 = 10.1 slices for dq; a short last split for dW).
@pytest.mark.parametrize("dtype,shape", [("bf16", (3, 32, (3, 10, 13))), ("f32", (3, 32, (3, 10, 13))),
                                         ("bf16", (8, 64, (3, 20, 23)))])
def test_projection_forward_and_backward(dtype, shape):
    heads, hd, (T, H, W) = shape
    wl = synth.Workload("proj-" + dtype, 1, T, H, W, heads, hd, (3, 3, 3), (1, 1, 1), dtype, "proj", backward=True)
    say(f"[projection] {synth.describe(wl)}")
    x = synth.make_inputs(wl, "cpu", seed=19)
    x["proj_b"].normal_(0, 0.1, generator=torch.Generator().manual_seed(2))
    xd = {k: v.to(DEV) for k, v in x.items()}
    N, C, F = wl.tokens, wl.C, wl.F
    off = dsa.offset_proj(xd["q"], xd["proj_w"], xd["proj_b"], wl.window)
    g = torch.randn(off.shape, generator=torch.Generator().manual_seed(3)).to(wl.torch_dtype)
    dq0 = torch.randn(x["q"].shape, generator=torch.Generator().manual_seed(4)).to(wl.torch_dtype)
    dq = dq0.to(DEV).clone()
    dw, db = dsa.offset_proj_backward(xd["q"], xd["proj_w"], g.to(DEV), dq, wl.window)
    torch.cuda.synchronize()
    q2 = to_np(x["q"]).reshape(N, C)
    ref = oracle.offset_proj(q2, to_np(x["proj_w"]), to_np(x["proj_b"]))
    tol = 1e-4 if dtype == "f32" else BF16_TOL
    _check("offsets", to_np(off).reshape(N, F), ref, dtype, tol_f32=1e-4)
    add, dw_ref, db_ref = oracle.offset_proj_backward(q2, to_np(x["proj_w"]), to_np(g).reshape(N, F))
    _check("dq_accum", to_np(dq).reshape(N, C), to_np(dq0).reshape(N, C) + add, dtype)
    # dW and db are float32 sums of exactly widened inputs: tight for both dtypes
    assert rel_l2(to_np(dw), dw_ref) <= 1e-5, rel_l2(to_np(dw), dw_ref)
    assert rel_l2(to_np(db), db_ref) <= 1e-5
    assert tol > 0


# ---------------------------------------------------------------------------
# depthwise convolution of the offset network
# ---------------------------------------------------------------------------

# (B, T, H, W, heads, head_dim): 24 channels (part of one wave), W under one
# run; 512 channels with ragged runs along w (30 = 12 + 12 + 6); 640 channels
# (a second, partial block of channels), single-token rows and frames. bf16
# with a multiple of 64 channels takes the LDS-tiled kernels (8 x 16 tiles of
# the (h, w) plane, runs of 16 frames): ragged tiles in h (11 = 8 + 3) and w
# (37 = 16 + 16 + 5) over two batch items, and frame runs 35 = 12 + 12 + 11;
# 256 x 512 frames: 32 x 32 tiles per frame, 1,024 partials of the
# weight-gradient sums.
@pytest.mark.parametrize("dtype,shape", [("f32", (2, 3, 5, 7, 3, 8)), ("bf16", (2, 3, 5, 7, 3, 8)),
                                         ("bf16", (1, 4, 6, 30, 8, 64)), ("f32", (1, 1, 1, 5, 5, 128)),
                                         ("bf16", (1, 3, 2, 1, 5, 128)), ("bf16", (2, 5, 11, 37, 2, 64)),
                                         ("bf16", (1, 35, 9, 17, 1, 64)), ("bf16", (1, 2, 256, 512, 1, 64))])
def test_dwconv_forward_and_backward(dtype, shape):
    B, T, H, W, heads, hd = shape
    C = heads * hd
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    say(f"[dwconv] {dtype} B={B} T={T} H={H} W={W} C={C}")
    gen = torch.Generator().manual_seed(31)
    q = torch.randn((B, T, H, W, heads, hd), generator=gen).to(tdt)
    wt = (torch.randn((C, 3, 3, 3), generator=gen) * 0.2).to(tdt)
    bias = (torch.randn(C, generator=gen) * 0.1).to(tdt)
    dy = torch.randn(q.shape, generator=gen).to(tdt)
    dq0 = torch.randn(q.shape, generator=gen).to(tdt)
    qd, wd, bd, gd = q.to(DEV), wt.to(DEV), bias.to(DEV), dy.to(DEV)
    y = dsa.dwconv(qd, wd, bd)
    dq = dq0.to(DEV).clone()
    dwt, db = dsa.dwconv_backward(qd, wd, gd, dq)
    torch.cuda.synchronize()
    q5, g5 = to_np(q).reshape(B, T, H, W, C), to_np(dy).reshape(B, T, H, W, C)
    ref = oracle.dwconv3d(q5, to_np(wt), to_np(bias))
    _check("dwconv y", to_np(y).reshape(-1, C), ref.reshape(-1, C), dtype)
    dq_ref, dw_ref, db_ref = oracle.dwconv3d_backward(q5, to_np(wt), g5)
    _check("dwconv dq_accum", to_np(dq).reshape(-1, C), (to_np(dq0).reshape(B, T, H, W, C) + dq_ref).reshape(-1, C),
           dtype)
    # dwt and dbias are float32 sums of exactly widened inputs: tight for both dtypes
    assert rel_l2(to_np(dwt), dw_ref) <= 1e-5, rel_l2(to_np(dwt), dw_ref)
    assert rel_l2(to_np(db), db_ref) <= 1e-5


def test_conv_offset_network_chain():
    """The whole chain with the depthwise convolution in the offset network:
    offsets = Linear(dwconv(q)), then attention forward and backward, then the
    projection and convolution backward into dq."""
    wl = synth.Workload("conv-chain", 1, 4, 6, 10, 8, 32, (3, 3, 3), (1, 2, 2), "bf16", "conv", backward=True)
    say(f"[conv chain] {synth.describe(wl)}")
    x = synth.make_inputs(wl, "cpu", seed=5)
    xd = {k: v.to(DEV) for k, v in x.items()}
    ch = Chain(wl, xd)
    desc = ch.desc
    dsa.dsa3d_dwconv_forward(desc, xd["q"], xd["conv_w"], xd["conv_b"], ch.pin)
    dsa.dsa3d_offset_proj_forward(desc, ch.pin, xd["proj_w"], xd["proj_b"], ch.offsets)
    dsa.dsa3d_forward(desc, xd["q"], xd["k"], xd["v"], ch.offsets, ch.out, ch.lse)
    dsa.dsa3d_backward(desc, xd["q"], xd["k"], xd["v"], ch.offsets, ch.out, ch.lse, xd["dout"], ch.dq, ch.dk, ch.dv,
                       ch.doff, ch.ws)
    torch.cuda.synchronize()
    dq_attn = ch.dq.clone()
    ch.dpin.zero_()
    dsa.dsa3d_offset_proj_backward(desc, ch.pin, xd["proj_w"], ch.doff, ch.dpin, ch.dw, ch.db, ch.pws)
    dsa.dsa3d_dwconv_backward(desc, xd["q"], xd["conv_w"], ch.dpin, ch.dq, ch.dcw, ch.dcb, ch.cws)
    torch.cuda.synchronize()
    N, C, F = wl.tokens, wl.C, wl.F
    q5 = to_np(x["q"]).reshape(1, wl.T, wl.H, wl.W, C)
    y_ref = oracle.dwconv3d(q5, to_np(x["conv_w"]), to_np(x["conv_b"]))
    _check("conv output", to_np(ch.pin).reshape(N, C), y_ref.reshape(N, C), "bf16")
    off_ref = oracle.offset_proj(to_np(ch.pin).reshape(N, C), to_np(x["proj_w"]), to_np(x["proj_b"]))
    _check("offsets", to_np(ch.offsets).reshape(N, F), off_ref, "bf16")
    # the attention on the GPU's offsets
    ref = oracle.forward(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), to_np(ch.offsets), wl.window, wl.dilation)
    _check("out", to_np(ch.out), ref[0], "bf16")
    # projection and convolution backward on the GPU's doffsets and convolution-output gradient
    g = to_np(ch.doff).reshape(N, F)
    _check("d(conv output)", to_np(ch.dpin).reshape(N, C), g @ to_np(x["proj_w"]), "bf16")
    dq_conv, dcw_ref, dcb_ref = oracle.dwconv3d_backward(q5, to_np(x["conv_w"]), to_np(ch.dpin).reshape(q5.shape))
    _check("dq total", to_np(ch.dq).reshape(N, C), to_np(dq_attn).reshape(N, C) + dq_conv.reshape(N, C), "bf16")
    assert rel_l2(to_np(ch.dcw), dcw_ref) <= 1e-5
    assert rel_l2(to_np(ch.dcb), dcb_ref) <= 1e-5
    assert rel_l2(to_np(ch.dw), g.T @ to_np(ch.pin).reshape(N, C)) <= 1e-5
    # the chain's own run() gives the same bits
    dq_once = ch.dq.clone()
    ch.run()
    torch.cuda.synchronize()
    assert torch.equal(ch.dq.view(torch.int16), dq_once.view(torch.int16))


# ---------------------------------------------------------------------------
# the named workloads: small one whole, full-size ones sampled
# ---------------------------------------------------------------------------

def test_small_bf16_projection_workload_whole():
    wl = synth.WORKLOADS["small-bf16-proj"]
    x = synth.make_inputs(wl, "cpu")
    ch = _run_whole(wl, x)
    N = wl.tokens
    ref = oracle.offset_proj(to_np(x["q"]).reshape(N, wl.C), to_np(x["proj_w"]), to_np(x["proj_b"]))
    _check("offsets", to_np(ch.offsets).reshape(N, wl.F), ref, "bf16")


def _free():
    import gc
    gc.collect()
    torch.cuda.empty_cache()


PARITY_LOG = os.environ.get("DSA3D_PARITY_LOG")


def _log_errors(test: str, rows):
    """Per-tensor error figures of a full-size test, one JSON line each, to the
    file named by DSA3D_PARITY_LOG (if set)."""
    for r in rows:
        say(f"    {r['tensor']:8s} head {str(r['head']):>4s}: rel-L2 {r['rel_l2']:.3e}  max|err| {r['max_abs']:.3e}"
            f"  (max|ref| {r['ref_max_abs']:.3e}, {r['n']} rows)")
    if PARITY_LOG:
        os.makedirs(os.path.dirname(os.path.abspath(PARITY_LOG)), exist_ok=True)
        with open(PARITY_LOG, "a") as f:
            for r in rows:
                f.write(json.dumps(dict(test=test, **r)) + "\n")


def _full_size_parity(test, wl, xd, offsets, out, lse, dq=None, dk=None, dv=None, doff=None, dout=None,
                      q_heads=None, k_heads=None, n_random=4096, n_random_k_heads=512, n_interior_keys=12, seed=0,
                      b=0, global_rows=None, dgk=None, dgv=None):
    """Oracle parity of a full-size run on sampled outputs.

    Queries: every token on the six faces of the grid plus n_random random
    tokens, for each head of q_heads (default: the first and the last head);
    n_random_k_heads random tokens for every other head of k_heads. Keys (when
    the run has a backward): the 8 grid corners, n_interior_keys random
    interior keys and 4 random face keys of every head of k_heads (default:
    every third head and the last one, so that every backward pass over a
    range of heads is covered). Each tensor is compared per head and over all
    the heads together. Hybrid attention: global_rows = (gk, gv) join each
    query's softmax, and dgk/dgv of the q_heads are compared with the oracle's
    sums over every query of the head."""
    rng = np.random.default_rng(seed)
    T, H, W = wl.T, wl.H, wl.W
    heads = wl.heads
    q_heads = sorted(set(q_heads if q_heads is not None else [0, heads - 1]))
    k_heads = sorted(set(k_heads if k_heads is not None else list(range(0, heads, 3)) + [heads - 1]))
    bwd = dq is not None
    tol = F32_TOL if wl.dtype == "f32" else BF16_TOL
    acc = {}   # tensor -> ([gpu rows], [ref rows])
    rows = []

    def compare(name, head, gpu, ref):
        e = errors(gpu, ref)
        rows.append(dict(tensor=name, head=str(head), **e))
        acc.setdefault(name, ([], []))
        acc[name][0].append(gpu.reshape(len(gpu), -1))
        acc[name][1].append(ref.reshape(len(ref), -1))

    for e in sorted(set(q_heads) | set(k_heads if bwd else [])):
        t0 = time.time()
        ho = HeadOracle(wl, xd, b, e, offsets, dout, global_rows=global_rows)
        if e in q_heads:
            pos = np.unique(np.concatenate([face_tokens(T, H, W), random_tokens(T, H, W, n_random, rng)]), axis=0)
        else:
            pos = random_tokens(T, H, W, n_random_k_heads, rng)
        o_ref, lse_ref = ho.forward(pos)
        compare("o", e, rows_at(out, b, e, pos), o_ref)
        compare("lse", e, rows_at(lse.unsqueeze(-1), b, e, pos), lse_ref[:, None])
        nk = 0
        if bwd:
            dq_ref, doff_ref = ho.backward_queries(pos)
            compare("dq", e, rows_at(dq, b, e, pos), dq_ref)
            if doff is not None:
                compare("doff", e, rows_at(doff, b, e, pos), doff_ref)
            if e in k_heads:
                keys = np.unique(np.concatenate([grid_corner_tokens(T, H, W),
                                                 interior_tokens(T, H, W, n_interior_keys, rng),
                                                 face_tokens(T, H, W)[rng.choice(len(face_tokens(T, H, W)), 4)]]),
                                 axis=0)
                kk, vv = ho.dkdv_at(keys)
                compare("dk", e, rows_at(dk, b, e, keys), kk)
                compare("dv", e, rows_at(dv, b, e, keys), vv)
                nk = len(keys)
            if dgk is not None and e in q_heads:
                gk_ref, gv_ref = ho.global_grads()
                compare("dgk", e, to_np(dgk[b, :, e]), gk_ref)
                compare("dgv", e, to_np(dgv[b, :, e]), gv_ref)
        say(f"[full] head {e}: {len(pos)} queries, {nk} keys in {time.time() - t0:.1f} s")
        del ho
    for name, (g, r) in acc.items():
        g, r = np.concatenate(g), np.concatenate(r)
        rows.append(dict(tensor=name, head="all", **errors(g, r)))
    _log_errors(test, rows)
    for r in rows:
        if r["tensor"] == "lse":
            assert r["max_abs"] <= (F32_TOL if wl.dtype == "f32" else 1e-3), r
        elif wl.dtype == "f32":
            assert r["max_abs"] <= tol, r
        else:
            assert r["rel_l2"] <= tol, r
    return rows


@pytest.mark.slow
def test_720p_dil2_workload_full_size_sampled():
    wl = synth.WORKLOADS["720p-bf16-proj-dil2"]
    say(f"[full] {synth.describe(wl)}")
    xd = synth.make_inputs(wl, DEV)
    ch = Chain(wl, xd)
    # run the pieces so that the attention's dq can be checked before the projection adds to it
    desc = ch.desc
    dsa.dsa3d_offset_proj_forward(desc, xd["q"], xd["proj_w"], xd["proj_b"], ch.offsets)
    dsa.dsa3d_forward(desc, xd["q"], xd["k"], xd["v"], ch.offsets, ch.out, ch.lse)
    dsa.dsa3d_backward(desc, xd["q"], xd["k"], xd["v"], ch.offsets, ch.out, ch.lse, xd["dout"], ch.dq, ch.dk, ch.dv,
                       ch.doff, ch.ws)
    torch.cuda.synchronize()
    dq_attn = ch.dq.clone()
    dsa.dsa3d_offset_proj_backward(desc, xd["q"], xd["proj_w"], ch.doff, ch.dq, ch.dw, ch.db, ch.pws)
    torch.cuda.synchronize()
    N, C, F = wl.tokens, wl.C, wl.F
    rows = np.random.default_rng(0).choice(N, 512, replace=False)
    q2 = xd["q"].view(N, C)
    ref = oracle.offset_proj(to_np(q2[rows]), to_np(xd["proj_w"]), to_np(xd["proj_b"]))
    _check("offsets rows", to_np(ch.offsets.view(N, F)[rows]), ref, "bf16")
    _full_size_parity("720p-bf16-proj-dil2", wl, xd, ch.offsets, ch.out, ch.lse, dq=dq_attn, dk=ch.dk, dv=ch.dv,
                      doff=ch.doff, dout=xd["dout"], seed=1)
    # projection backward on the GPU's doffsets (its input)
    g = to_np(ch.doff.view(N, F))
    add = g[rows] @ to_np(xd["proj_w"])
    _check("dq total rows", to_np(ch.dq.view(N, C)[rows]), to_np(dq_attn.view(N, C)[rows]) + add, "bf16")
    cols = np.random.default_rng(1).choice(C, 64, replace=False)
    dw_ref = g.T @ to_np(q2[:, torch.tensor(cols)])
    assert rel_l2(to_np(ch.dw)[:, cols], dw_ref) <= 1e-5
    assert rel_l2(to_np(ch.db), g.sum(0)) <= 1e-5
    del ch, xd
    _free()


@pytest.mark.slow
def test_720p_conv_workload_full_size_sampled():
    """The 720p chain with the depthwise convolution in the offset network, at full size:
    the convolution and its gradients on a subset of channels over the whole grid, the
    offsets and attention on sampled tokens."""
    wl = synth.WORKLOADS["720p-bf16-conv-dil2"]
    say(f"[full] {synth.describe(wl)}")
    xd = synth.make_inputs(wl, DEV)
    ch = Chain(wl, xd)
    desc = ch.desc
    dsa.dsa3d_dwconv_forward(desc, xd["q"], xd["conv_w"], xd["conv_b"], ch.pin)
    dsa.dsa3d_offset_proj_forward(desc, ch.pin, xd["proj_w"], xd["proj_b"], ch.offsets)
    dsa.dsa3d_forward(desc, xd["q"], xd["k"], xd["v"], ch.offsets, ch.out, ch.lse)
    dsa.dsa3d_backward(desc, xd["q"], xd["k"], xd["v"], ch.offsets, ch.out, ch.lse, xd["dout"], ch.dq, ch.dk, ch.dv,
                       ch.doff, ch.ws)
    torch.cuda.synchronize()
    dq_attn = ch.dq.clone()
    ch.dpin.zero_()
    dsa.dsa3d_offset_proj_backward(desc, ch.pin, xd["proj_w"], ch.doff, ch.dpin, ch.dw, ch.db, ch.pws)
    dsa.dsa3d_dwconv_backward(desc, xd["q"], xd["conv_w"], ch.dpin, ch.dq, ch.dcw, ch.dcb, ch.cws)
    torch.cuda.synchronize()
    N, C, F = wl.tokens, wl.C, wl.F
    g5 = (1, wl.T, wl.H, wl.W, C)
    cols = torch.tensor(np.sort(np.random.default_rng(3).choice(C, 16, replace=False)), device=DEV)
    sub = lambda t: to_np(t.view(g5).index_select(4, cols))
    cw = to_np(xd["conv_w"].index_select(0, cols))
    q_c = sub(xd["q"])
    _check("conv output (16 channels)", sub(ch.pin).reshape(-1, 16),
           oracle.dwconv3d(q_c, cw, to_np(xd["conv_b"].index_select(0, cols))).reshape(-1, 16), "bf16")
    rows = np.random.default_rng(0).choice(N, 512, replace=False)
    pin2 = ch.pin.view(N, C)
    ref = oracle.offset_proj(to_np(pin2[rows]), to_np(xd["proj_w"]), to_np(xd["proj_b"]))
    _check("offsets rows", to_np(ch.offsets.view(N, F)[rows]), ref, "bf16")
    _full_size_parity("720p-bf16-conv-dil2", wl, xd, ch.offsets, ch.out, ch.lse, dq=dq_attn, dk=ch.dk, dv=ch.dv,
                      doff=ch.doff, dout=xd["dout"], seed=9)
    g = to_np(ch.doff.view(N, F)[rows])
    _check("d(conv output) rows", to_np(ch.dpin.view(N, C)[rows]), g @ to_np(xd["proj_w"]), "bf16")
    dq_c, dcw_ref, dcb_ref = oracle.dwconv3d_backward(q_c, cw, sub(ch.dpin))
    _check("dq total (16 channels)", sub(ch.dq).reshape(-1, 16), (sub(dq_attn) + dq_c).reshape(-1, 16), "bf16")
    assert rel_l2(to_np(ch.dcw.index_select(0, cols)), dcw_ref) <= 1e-5
    assert rel_l2(to_np(ch.dcb.index_select(0, cols)), dcb_ref) <= 1e-5
    del ch, xd
    _free()


@pytest.mark.slow
def test_1080p_projection_workload_full_size_sampled():
    wl = synth.WORKLOADS["1080p-bf16-proj"]
    say(f"[full] {synth.describe(wl)}")
    xd = synth.make_inputs(wl, DEV)
    ch = Chain(wl, xd)
    ch.run()
    torch.cuda.synchronize()
    N, C, F = wl.tokens, wl.C, wl.F
    rows = np.random.default_rng(0).choice(N, 256, replace=False)
    ref = oracle.offset_proj(to_np(xd["q"].view(N, C)[rows]), to_np(xd["proj_w"]), to_np(xd["proj_b"]))
    _check("offsets rows", to_np(ch.offsets.view(N, F)[rows]), ref, "bf16")
    _full_size_parity("1080p-bf16-proj", wl, xd, ch.offsets, ch.out, ch.lse, q_heads=[0, 11, wl.heads - 1],
                      seed=3)
    del ch, xd
    _free()


@pytest.mark.slow
def test_1080p_fixed_377_workload_full_size_sampled():
    """The fixed 3x7x7 window at 1080p, in the bench's launch configuration."""
    wl = synth.WORKLOADS["1080p-bf16-fixed377"]
    say(f"[full] {synth.describe(wl)}")
    xd = synth.make_inputs(wl, DEV)
    ch = Chain(wl, xd)
    ch.run()
    torch.cuda.synchronize()
    _full_size_parity("1080p-bf16-fixed377", wl, xd, None, ch.out, ch.lse, dq=ch.dq, dk=ch.dk, dv=ch.dv,
                      dout=xd["dout"], seed=7)
    del ch, xd
    _free()


@pytest.mark.slow
def test_1080p_p75_deterministic_workload_full_size_sampled():
    """The benchmark's workload and launch configuration (default workspace)."""
    wl = synth.WORKLOADS[synth.HEADLINE]
    say(f"[full] {synth.describe(wl)}")
    xd = synth.make_inputs(wl, DEV)
    ch = Chain(wl, xd)
    ch.run()
    torch.cuda.synchronize()
    _full_size_parity("1080p-bf16-p75-det", wl, xd, ch.offsets, ch.out, ch.lse, dq=ch.dq, dk=ch.dk, dv=ch.dv,
                      doff=ch.doff, dout=xd["dout"], seed=5)
    # bitwise reproducibility of the whole chain at full size
    ref = [t.clone() for t in (ch.dk, ch.dv)]
    ch.run()
    torch.cuda.synchronize()
    assert torch.equal(ref[0].view(torch.int16), ch.dk.view(torch.int16))
    assert torch.equal(ref[1].view(torch.int16), ch.dv.view(torch.int16))
    del ch, xd, ref
    _free()
