"""GPU parity of the transformer block around the operator: layer
normalisation, linear layers (with bias and residual) and the whole block,
through the C ABI, against the oracle's float64 definitions.

Acceptance as for the operator: float32 runs max |err| <= 1e-4 on
activations; bf16 runs rel-L2 <= 1e-2 per tensor with the oracle fed the same
bf16 inputs widened exactly; float32 parameter gradients (dgamma, dbeta, dW,
db: float32 sums of exactly widened inputs) rel-L2 <= 1e-5. The bf16 block is
checked stage by stage, each stage on the GPU's own inputs to it; the float32
block also end to end.
"""
import os
import sys

import numpy as np
import pytest
import torch

import deformable_local_attention_amd as dsa
import oracle
from deformable_local_attention_amd import synth
from deformable_local_attention_amd.chain import BlockChain
from gpu_helpers import rel_l2, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _close(name, gpu, ref, dtype, kind="act"):
    gpu, ref = np.asarray(gpu, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    if kind == "param":
        err = rel_l2(gpu, ref)
        say(f"    {name}: rel-L2 {err:.3e} (float32 sums, tolerance 1e-5)")
        assert err <= 1e-5, f"{name}: rel-L2 {err:.3e}"
    elif dtype == torch.float32:
        err = float(np.abs(gpu - ref).max()) if gpu.size else 0.0
        say(f"    {name}: max abs err {err:.3e} (tolerance 1e-4)")
        assert err <= 1e-4, f"{name}: max abs err {err:.3e}"
    else:
        err = rel_l2(gpu, ref)
        say(f"    {name}: rel-L2 {err:.3e} (tolerance 1e-2)")
        assert err <= 1e-2, f"{name}: rel-L2 {err:.3e}"


# ---------------------------------------------------------------------------
# layer normalisation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M,N", [(1, 8), (37, 64), (1000, 1024), (513, 3072), (130, 4096), (7, 2056)])
@pytest.mark.parametrize("with_res", [False, True])
def test_layernorm_forward_backward(dtype, M, N, with_res):
    say(f"[layernorm] {dtype} M={M} N={N} dres={with_res}")
    g = torch.Generator().manual_seed(M * 7 + N)
    x = (torch.randn((M, N), generator=g) * 2.0 + 0.5).to(dtype)
    gam = (1.0 + 0.2 * torch.randn(N, generator=g)).to(dtype)
    bet = (0.1 * torch.randn(N, generator=g)).to(dtype)
    dy = torch.randn((M, N), generator=g).to(dtype)
    dres = torch.randn((M, N), generator=g).to(dtype) if with_res else None
    xd, gd, bd, dyd = x.to(DEV), gam.to(DEV), bet.to(DEV), dy.to(DEV)
    y, stats = dsa.layernorm(xd, gd, bd, 1e-6)
    dx = torch.empty_like(xd)
    dg = torch.empty(N, dtype=torch.float32, device=DEV)
    db = torch.empty(N, dtype=torch.float32, device=DEV)
    ws = torch.empty(dsa.dsa3d_layernorm_workspace_size(M, N), dtype=torch.uint8, device=DEV)
    dsa.dsa3d_layernorm_backward(dsa.dtype_code(dtype), M, N, xd, gd, stats, dyd,
                                 None if dres is None else dres.to(DEV), dx, dg, db, ws)
    torch.cuda.synchronize()
    y_ref, mean, rstd = oracle.layernorm(to_np(x), to_np(gam), to_np(bet), 1e-6)
    _close("y", to_np(y), y_ref, dtype)
    st = stats.cpu().numpy().astype(np.float64)
    assert np.abs(st[:, 0] - mean).max() <= 1e-5 * max(1.0, np.abs(mean).max())
    assert np.abs(st[:, 1] - rstd).max() <= 1e-5 * np.abs(rstd).max()
    dx_ref, dg_ref, db_ref = oracle.layernorm_backward(to_np(x), to_np(gam), to_np(dy), 1e-6)
    if with_res:
        dx_ref = dx_ref + to_np(dres)
    _close("dx", to_np(dx), dx_ref, dtype)
    _close("dgamma", to_np(dg), dg_ref, dtype, "param")
    _close("dbeta", to_np(db), db_ref, dtype, "param")


def test_layernorm_rejects_unsupported_widths():
    x = torch.zeros((4, 12), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dsa.DSA3DError):
        dsa.layernorm(x, None, None)
    x = torch.zeros((4, 4104), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dsa.DSA3DError):
        dsa.layernorm(x, None, None)


# ---------------------------------------------------------------------------
# linear layers
# ---------------------------------------------------------------------------

# (M, N, K): the 256x256 DMA-fed kernel (K, N multiples of 8; 64-deep K
# slices, the last one ragged at K = 72 and 200), ragged tiles, shapes only
# the 128x128 kernel takes (N odd), tiny ones
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M,N,K", [(2048, 1024, 1024), (1000, 264, 72), (1536, 512, 200), (333, 77, 40),
                                   (5, 8, 16)])
@pytest.mark.parametrize("with_res", [False, True])
def test_linear_forward_backward(dtype, M, N, K, with_res):
    say(f"[linear] {dtype} M={M} N={N} K={K} residual={with_res}")
    g = torch.Generator().manual_seed(M + 3 * N + 5 * K)
    x = torch.randn((M, K), generator=g).to(dtype)
    w = (torch.randn((N, K), generator=g) * K ** -0.5).to(dtype)
    b = (0.1 * torch.randn(N, generator=g)).to(dtype)
    r = torch.randn((M, N), generator=g).to(dtype) if with_res else None
    dy = torch.randn((M, N), generator=g).to(dtype)
    dres = torch.randn((M, K), generator=g).to(dtype) if with_res else None
    xd, wd, bd, dyd = x.to(DEV), w.to(DEV), b.to(DEV), dy.to(DEV)
    y = dsa.linear(xd, wd, bd, None if r is None else r.to(DEV))
    code = dsa.dtype_code(dtype)
    dx = torch.empty_like(xd)
    dw = torch.empty((N, K), dtype=torch.float32, device=DEV)
    db = torch.empty(N, dtype=torch.float32, device=DEV)
    ws = torch.empty(dsa.dsa3d_linear_workspace_size(code, M, N, K), dtype=torch.uint8, device=DEV)
    dsa.dsa3d_linear_backward(code, M, N, K, xd, wd, dyd, None if dres is None else dres.to(DEV), dx, dw, db, ws)
    torch.cuda.synchronize()
    y_ref = oracle.linear(to_np(x), to_np(w), to_np(b)) + (to_np(r) if with_res else 0.0)
    _close("y", to_np(y), y_ref, dtype)
    dx_ref, dw_ref, db_ref = oracle.linear_backward(to_np(x), to_np(w), to_np(dy))
    if with_res:
        dx_ref = dx_ref + to_np(dres)
    _close("dx", to_np(dx), dx_ref, dtype)
    _close("dw", to_np(dw), dw_ref, dtype, "param")
    _close("db", to_np(db), db_ref, dtype, "param")


def test_linear_residual_in_place():
    """residual == y: the product is added to y in place (one rounding)."""
    g = torch.Generator().manual_seed(9)
    M, N, K = 512, 256, 128
    x = torch.randn((M, K), generator=g).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g) * K ** -0.5).to(torch.bfloat16)
    y0 = torch.randn((M, N), generator=g).to(torch.bfloat16)
    yd = y0.to(DEV)
    dsa.dsa3d_linear_forward(dsa.DSA3D_BF16, M, N, K, x.to(DEV), w.to(DEV), None, yd, yd)
    torch.cuda.synchronize()
    _close("y += x.w^T", to_np(yd), to_np(y0) + oracle.linear(to_np(x), to_np(w)), torch.bfloat16)


# ---------------------------------------------------------------------------
# the whole block
# ---------------------------------------------------------------------------

def _block_wl(dtype, T=3, H=5, W=7, heads=2, d=32, window=(3, 3, 3), dil=(1, 1, 1), name="block", det=False):
    return synth.Workload(name, 1, T, H, W, heads, d, window, dil, dtype, "proj", weight_sigma=0.05,
                          backward=True, deterministic=det, block=True)


def _params64(x):
    return {"ln_g": to_np(x["ln_g"]), "ln_b": to_np(x["ln_b"]), "w_qkv": to_np(x["w_qkv"]),
            "b_qkv": to_np(x["b_qkv"]), "w_off": to_np(x["proj_w"]), "b_off": to_np(x["proj_b"]),
            "w_out": to_np(x["w_out"]), "b_out": to_np(x["b_out"])}


def test_block_f32_end_to_end():
    """The float32 block, forward and backward, against the oracle's block
    composed in float64 from the same inputs."""
    wl = _block_wl("f32")
    say(f"[block] {synth.describe(wl)}")
    x = synth.make_inputs(wl, "cpu", seed=81)
    xd = {k: v.to(DEV) for k, v in x.items()}
    ch = BlockChain(wl, xd)
    ch.run()
    torch.cuda.synchronize()
    p = _params64(x)
    f = oracle.block_forward(to_np(x["x"]), p, wl.heads, wl.window, wl.dilation, wl.ln_eps)
    _close("offsets", to_np(ch.offsets), f["offsets"], torch.float32)
    _close("o", to_np(ch.out), f["o"], torch.float32)
    _close("y", to_np(ch.y), f["y"], torch.float32)
    g = oracle.block_backward(to_np(x["x"]), p, to_np(x["dout"]), wl.heads, wl.window, wl.dilation, wl.ln_eps)
    _close("dx", to_np(ch.dx), g["dx"], torch.float32)
    for name, t in (("dln_g", ch.dln_g), ("dln_b", ch.dln_b), ("dw_qkv", ch.dw_qkv), ("db_qkv", ch.db_qkv),
                    ("dw_off", ch.dw_off), ("db_off", ch.db_off), ("dw_out", ch.dw_out), ("db_out", ch.db_out)):
        err = rel_l2(to_np(t), g[name])
        say(f"    {name}: rel-L2 {err:.3e} (tolerance 1e-4)")
        assert err <= 1e-4, (name, err)


def _check_block_stages(wl, x, ch, rows=None):
    """Each stage of a bf16 block run against the oracle on the GPU's own
    inputs to that stage (rows: a sample of token rows, or all)."""
    C, M = wl.C, wl.tokens
    sel = np.arange(M) if rows is None else np.asarray(rows)
    r = lambda t: to_np(t.reshape(M, -1)[torch.as_tensor(sel, device=t.device)])
    xx = r(x["x"])
    h_ref, _, _ = oracle.layernorm(xx, to_np(x["ln_g"]), to_np(x["ln_b"]), wl.ln_eps)
    _close("h", r(ch.h), h_ref, torch.bfloat16)
    wqkv, bqkv = to_np(x["w_qkv"]), to_np(x["b_qkv"])
    hh = r(ch.h)
    for i, t in enumerate((ch.q, ch.k, ch.v)):
        _close("qkv"[i], r(t), oracle.linear(hh, wqkv[i * C:(i + 1) * C], bqkv[i * C:(i + 1) * C]), torch.bfloat16)
    _close("offsets", r(ch.offsets), oracle.linear(r(ch.q), to_np(x["proj_w"]), to_np(x["proj_b"])), torch.bfloat16)
    _close("y", r(ch.y), xx + oracle.linear(r(ch.out), to_np(x["w_out"]), to_np(x["b_out"])), torch.bfloat16)
    dy = r(x["dout"])
    _close("do", r(ch.do), dy @ to_np(x["w_out"]), torch.bfloat16)
    dqt = r(ch.dq)
    dh_ref = dqt @ wqkv[:C] + r(ch.dk) @ wqkv[C:2 * C] + r(ch.dv) @ wqkv[2 * C:]
    _close("dh", r(ch.dh), dh_ref, torch.bfloat16)
    dx_ref, _, _ = oracle.layernorm_backward(xx, to_np(x["ln_g"]), r(ch.dh), wl.ln_eps)
    _close("dx", r(ch.dx), dx_ref + dy, torch.bfloat16)


def test_block_bf16_stages_whole_grid():
    """The bf16 block, stage by stage on every token, plus the attention stage
    and the parameter gradients against the oracle on the GPU's inputs."""
    wl = _block_wl("bf16", T=4, H=6, W=9, heads=2, d=64, window=(3, 5, 5), det=True)
    say(f"[block] {synth.describe(wl)}")
    x = synth.make_inputs(wl, "cpu", seed=82)
    xd = {k: v.to(DEV) for k, v in x.items()}
    ch = BlockChain(wl, xd)
    ch.run()
    torch.cuda.synchronize()
    _check_block_stages(wl, xd, ch)
    # the attention on the GPU's q, k, v and offsets
    o, _ = oracle.forward(to_np(ch.q), to_np(ch.k), to_np(ch.v), to_np(ch.offsets), wl.window, wl.dilation)
    _close("attention o", to_np(ch.out), o, torch.bfloat16)
    dq, dk, dv, doff = oracle.backward(to_np(ch.q), to_np(ch.k), to_np(ch.v), to_np(ch.offsets), to_np(ch.do),
                                       wl.window, wl.dilation)
    C, M = wl.C, wl.tokens
    add, dw_off, db_off = oracle.offset_proj_backward(to_np(ch.q).reshape(M, C), to_np(x["proj_w"]),
                                                      to_np(ch.doff).reshape(M, -1))
    _close("dq (attention + offset projection)", to_np(ch.dq).reshape(M, C), dq.reshape(M, C) + add,
           torch.bfloat16)
    _close("dk", to_np(ch.dk), dk, torch.bfloat16)
    _close("doffsets", to_np(ch.doff), doff, torch.bfloat16)
    # parameter gradients on the GPU's inputs to each product
    h2, o2, dy2 = to_np(ch.h).reshape(M, C), to_np(ch.out).reshape(M, C), to_np(x["dout"]).reshape(M, C)
    _close("dw_out", to_np(ch.dw_out), dy2.T @ o2, torch.bfloat16, "param")
    _close("db_out", to_np(ch.db_out), dy2.sum(0), torch.bfloat16, "param")
    _close("dw_qkv[v]", to_np(ch.dw_qkv)[2 * C:], to_np(ch.dv).reshape(M, C).T @ h2, torch.bfloat16, "param")
    _close("dw_off", to_np(ch.dw_off), dw_off, torch.bfloat16, "param")
    _, dg_ref, db_ref = oracle.layernorm_backward(to_np(x["x"]).reshape(M, C), to_np(x["ln_g"]),
                                                  to_np(ch.dh).reshape(M, C), wl.ln_eps)
    _close("dln_g", to_np(ch.dln_g), dg_ref, torch.bfloat16, "param")
    _close("dln_b", to_np(ch.dln_b), db_ref, torch.bfloat16, "param")
    # deterministic mode: a second run gives the same bits (every sum in a fixed order)
    first = [t.clone() for t in (ch.y, ch.dx, ch.dw_qkv, ch.dln_g)]
    ch.run()
    torch.cuda.synchronize()
    for a, b in zip(first, (ch.y, ch.dx, ch.dw_qkv, ch.dln_g)):
        assert torch.equal(a, b) if a.dtype == torch.float32 else torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.slow
def test_720p_block_workload_full_size_sampled():
    """The 720p block (64x45x80 tokens, 16 x 64 heads, 3x3x3 window with
    dilation (1,2,2)) at full size in the bench's launch configuration: every
    stage on 2,048 sampled token rows, the attention through the operator's
    full-size parity driver, and the parameter gradients on sampled columns."""
    wl = synth.WORKLOADS["720p-bf16-block"]
    say(f"[full] {synth.describe(wl)}")
    xd = synth.make_inputs(wl, DEV)
    ch = BlockChain(wl, xd)
    ch.run()
    torch.cuda.synchronize()
    M, C = wl.tokens, wl.C
    rows = np.sort(np.random.default_rng(0).choice(M, 2048, replace=False))
    _check_block_stages(wl, xd, ch, rows)
    from test_gpu_parity import _full_size_parity
    # the attention's dq here includes the offset projection's share, so only
    # o, lse, dk, dv are compared (dq and doffsets are covered by the operator's tests)
    _full_size_parity("720p-bf16-block", wl, {"q": ch.q, "k": ch.k, "v": ch.v}, ch.offsets, ch.out, ch.lse,
                      q_heads=[0, wl.heads - 1], k_heads=[], n_random=2048, seed=11)
    cols = torch.as_tensor(np.sort(np.random.default_rng(1).choice(C, 32, replace=False)), device=DEV)
    dy2 = to_np(xd["dout"].reshape(M, C))
    o_cols = to_np(ch.out.reshape(M, C).index_select(1, cols))
    _close("dw_out (32 columns)", to_np(ch.dw_out.index_select(1, cols)), dy2.T @ o_cols, torch.bfloat16, "param")
    _close("db_out", to_np(ch.db_out), dy2.sum(0), torch.bfloat16, "param")
    del ch, xd
    import gc
    gc.collect()
    torch.cuda.empty_cache()
