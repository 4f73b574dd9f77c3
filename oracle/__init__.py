"""CPU oracle for 3D Deformable Slide Attention (3D-DSA) -- test infrastructure.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. It shares no code with the GPU library.

The attention itself lives in `dsa3d_oracle.c` (plain fp64 C, one query at a
time; see that file's header for the operator's steps and the passages they
follow). This module loads it with ctypes, splits whole tensors into one call
per (batch item, head) -- heads are independent given the offsets -- and runs
those calls on a thread pool. The offset projection is a textbook fp64 GEMM
done with numpy: the offset network ends in a pointwise convolution / linear
layer [MegaSlide-DiT, §5.3 Implementation considerations; Dutch and French
summaries, "3D Deformable Slide Attention", Implementation], read here as a
Linear layer of the token's full query row.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence, Tuple

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "dsa3d_oracle.c")
_LIB_PATH = os.path.join(_DIR, "libdsa3d_oracle.so")
_lib = None
_lock = threading.Lock()

OUTSIDE = np.iinfo(np.int32).min  # base coordinate of a sample that is entirely outside


class _Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("d", ctypes.c_int32),
                ("kt", ctypes.c_int32), ("kh", ctypes.c_int32), ("kw", ctypes.c_int32),
                ("dil_t", ctypes.c_int32), ("dil_h", ctypes.c_int32), ("dil_w", ctypes.c_int32),
                ("scale", ctypes.c_double),
                ("bt0", ctypes.c_int32), ("bh0", ctypes.c_int32), ("bw0", ctypes.c_int32),
                ("BT", ctypes.c_int32), ("BH", ctypes.c_int32), ("BW", ctypes.c_int32)]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    """The loaded oracle library (built first if it is not there)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            L = ctypes.CDLL(_LIB_PATH)
            P = ctypes.POINTER
            L.orc_geometry.argtypes = [P(_Problem), ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
            L.orc_forward.argtypes = [P(_Problem), ctypes.c_long] + [ctypes.c_void_p] * 8
            L.orc_backward.argtypes = [P(_Problem), ctypes.c_long] + [ctypes.c_void_p] * 10
            L.orc_forward_hybrid.argtypes = ([P(_Problem), ctypes.c_long] + [ctypes.c_void_p] * 5 + [ctypes.c_int] +
                                             [ctypes.c_void_p] * 4)
            L.orc_backward_hybrid.argtypes = ([P(_Problem), ctypes.c_long] + [ctypes.c_void_p] * 5 + [ctypes.c_int] +
                                              [ctypes.c_void_p] * 9)
            for f in (L.orc_geometry, L.orc_forward, L.orc_backward, L.orc_forward_hybrid, L.orc_backward_hybrid):
                f.restype = ctypes.c_int
            _lib = L
    return _lib


def _use_library(path: Optional[str]):
    """Test hook: load the oracle from another build (e.g. a planted mistake)
    and return the previously loaded library handle; None restores the default."""
    global _lib
    prev = _lib
    with _lock:
        _lib = None
    if path is not None:
        global _LIB_PATH
        saved = _LIB_PATH
        _LIB_PATH = path
        try:
            lib()
        finally:
            _LIB_PATH = saved
    return prev


def _restore_library(handle):
    global _lib
    with _lock:
        _lib = handle


def build_variant(src_text: str, out_path: str) -> str:
    """Compile C source text with the oracle's flags into out_path (tests only)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    "-w", "-o", out_path, src, "-lm"], check=True)
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def default_scale(d: int) -> float:
    """Logit scale 1/sqrt(d)."""
    return 1.0 / math.sqrt(d)


def _problem(grid, d, window, dilation, scale, box_origin, box_shape) -> _Problem:
    T, H, W = grid
    kt, kh, kw = window
    if kt % 2 == 0 or kh % 2 == 0 or kw % 2 == 0:
        raise ValueError("window sizes must be odd")
    return _Problem(T, H, W, d, kt, kh, kw, dilation[0], dilation[1], dilation[2], float(scale),
                    box_origin[0], box_origin[1], box_origin[2], box_shape[0], box_shape[1], box_shape[2])


def _check(rc: int, what: str):
    if rc == -1:
        raise RuntimeError(f"oracle {what}: a sampled corner lies in the grid but outside the K/V box")
    if rc != 0:
        raise RuntimeError(f"oracle {what}: error {rc}")


# ----------------------------------------------------------------------------
# One (batch item, head): explicit query list and K/V box.
# ----------------------------------------------------------------------------

def forward_queries(grid, window, dilation, scale, qpos, q, off, box_origin, K, V,
                    want_attn=False, threads=1):
    """Forward of listed queries of one head.

    grid (T,H,W); qpos [n,3] int absolute coordinates; q [n,d]; off [n,P,3]
    (rounded to single precision first); K, V [BT,BH,BW,d] the box at
    box_origin. Returns o [n,d], lse [n] (and attn [n,P]). With threads > 1
    the queries are split into that many runs of consecutive queries, each a
    call of its own on a thread pool (the calls share only read-only inputs).
    """
    qpos = np.ascontiguousarray(qpos, dtype=np.int32)
    q, K, V, off = _f64(q), _f64(K), _f64(V), _f32(off)
    n, d = q.shape
    P = window[0] * window[1] * window[2]
    pr = _problem(grid, d, window, dilation, scale, box_origin, K.shape[:3])
    o = np.zeros((n, d)); lse = np.zeros(n)
    attn = np.zeros((n, P)) if want_attn else None

    def run(r):
        i0, i1 = r
        if i1 <= i0:
            return 0
        return lib().orc_forward(ctypes.byref(pr), i1 - i0, _ptr(qpos[i0:i1]), _ptr(q[i0:i1]), _ptr(off[i0:i1]),
                                 _ptr(K), _ptr(V), _ptr(o[i0:i1]), _ptr(lse[i0:i1]),
                                 None if attn is None else _ptr(attn[i0:i1]))

    for rc in _pool_map(run, _runs(n, threads), threads):
        _check(rc, "forward")
    return (o, lse, attn) if want_attn else (o, lse)


def _runs(n: int, parts: int):
    parts = max(1, min(int(parts or 1), n)) if n else 1
    edges = [n * i // parts for i in range(parts + 1)]
    return list(zip(edges[:-1], edges[1:]))


def backward_queries(grid, window, dilation, scale, qpos, q, off, box_origin, K, V, dout,
                     dK=None, dV=None, want_kv=True, threads=1):
    """Backward of listed queries of one head.

    Returns dq [n,d], doff [n,P,3], and dK, dV [BT,BH,BW,d] holding the
    contributions of these queries only (accumulated into dK/dV if given).
    With want_kv False no key/value gradient is formed (dK, dV returned as
    None) and, with threads > 1, runs of consecutive queries are computed by
    concurrent calls.
    """
    qpos = np.ascontiguousarray(qpos, dtype=np.int32)
    q, K, V, off, dout = _f64(q), _f64(K), _f64(V), _f32(off), _f64(dout)
    n, d = q.shape
    P = window[0] * window[1] * window[2]
    pr = _problem(grid, d, window, dilation, scale, box_origin, K.shape[:3])
    dq = np.zeros((n, d)); doff = np.zeros((n, P, 3))
    if want_kv:
        dK = np.zeros(K.shape) if dK is None else dK
        dV = np.zeros(V.shape) if dV is None else dV
        assert dK.dtype == np.float64 and dK.flags.c_contiguous and dV.flags.c_contiguous
        threads = 1
    else:
        dK = dV = None

    def run(r):
        i0, i1 = r
        if i1 <= i0:
            return 0
        return lib().orc_backward(ctypes.byref(pr), i1 - i0, _ptr(qpos[i0:i1]), _ptr(q[i0:i1]), _ptr(off[i0:i1]),
                                  _ptr(K), _ptr(V), _ptr(dout[i0:i1]), _ptr(dq[i0:i1]), _ptr(doff[i0:i1]),
                                  _ptr(dK), _ptr(dV))

    for rc in _pool_map(run, _runs(n, threads), threads):
        _check(rc, "backward")
    return dq, doff, dK, dV


def geometry_queries(grid, window, dilation, qpos, off):
    """Base corner [n,P,3] int32 and fraction [n,P,3] float32 of listed queries."""
    qpos = np.ascontiguousarray(qpos, dtype=np.int32)
    off = _f32(off)
    n = qpos.shape[0]
    P = window[0] * window[1] * window[2]
    pr = _problem(grid, 1, window, dilation, 1.0, (0, 0, 0), (0, 0, 0))
    base = np.zeros((n, P, 3), dtype=np.int32); frac = np.zeros((n, P, 3), dtype=np.float32)
    rc = lib().orc_geometry(ctypes.byref(pr), n, _ptr(qpos), _ptr(off), _ptr(base), _ptr(frac))
    _check(rc, "geometry")
    return base, frac


# ----------------------------------------------------------------------------
# Whole tensors in the [B,T,H,W,heads,d] layout.
# ----------------------------------------------------------------------------

def grid_positions(T: int, H: int, W: int) -> np.ndarray:
    """All token coordinates of a T x H x W grid in row-major order, [N,3]."""
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1).astype(np.int32)


def _pool_map(fn, items, threads):
    threads = threads or min(len(items), os.cpu_count() or 1)
    if threads <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))


def forward(q, k, v, off, window, dilation=(1, 1, 1), scale=None, want_attn=False,
            threads=None):
    """Forward over whole tensors: q,k,v [B,T,H,W,heads,d], off [B,T,H,W,heads,P,3].

    Returns o [B,T,H,W,heads,d] and lse [B,T,H,W,heads] (and attn [..,heads,P]).
    """
    q, k, v, off = _f64(q), _f64(k), _f64(v), _f32(off)
    B, T, H, W, nh, d = q.shape
    P = window[0] * window[1] * window[2]
    if off.shape != (B, T, H, W, nh, P, 3):
        raise ValueError(f"offsets shape {off.shape} != {(B, T, H, W, nh, P, 3)}")
    scale = default_scale(d) if scale is None else scale
    pos = grid_positions(T, H, W)
    N = T * H * W
    o = np.zeros_like(q); lse = np.zeros((B, T, H, W, nh))
    attn = np.zeros((B, T, H, W, nh, P)) if want_attn else None

    def one(bh):
        b, h = bh
        res = forward_queries((T, H, W), window, dilation, scale, pos,
                              q[b, :, :, :, h].reshape(N, d), off[b, :, :, :, h].reshape(N, P, 3),
                              (0, 0, 0), k[b, :, :, :, h], v[b, :, :, :, h], want_attn)
        o[b, :, :, :, h] = res[0].reshape(T, H, W, d)
        lse[b, :, :, :, h] = res[1].reshape(T, H, W)
        if want_attn:
            attn[b, :, :, :, h] = res[2].reshape(T, H, W, P)

    _pool_map(one, [(b, h) for b in range(B) for h in range(nh)], threads)
    return (o, lse, attn) if want_attn else (o, lse)


def backward(q, k, v, off, dout, window, dilation=(1, 1, 1), scale=None, threads=None):
    """Backward over whole tensors. Returns dq, dk, dv [B,T,H,W,heads,d] and
    doff [B,T,H,W,heads,P,3] (all float64)."""
    q, k, v, off, dout = _f64(q), _f64(k), _f64(v), _f32(off), _f64(dout)
    B, T, H, W, nh, d = q.shape
    P = window[0] * window[1] * window[2]
    scale = default_scale(d) if scale is None else scale
    pos = grid_positions(T, H, W)
    N = T * H * W
    dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
    doff = np.zeros(off.shape)

    def one(bh):
        b, h = bh
        r = backward_queries((T, H, W), window, dilation, scale, pos,
                             q[b, :, :, :, h].reshape(N, d), off[b, :, :, :, h].reshape(N, P, 3),
                             (0, 0, 0), k[b, :, :, :, h], v[b, :, :, :, h],
                             dout[b, :, :, :, h].reshape(N, d))
        dq[b, :, :, :, h] = r[0].reshape(T, H, W, d)
        doff[b, :, :, :, h] = r[1].reshape(T, H, W, P, 3)
        dk[b, :, :, :, h] = r[2]
        dv[b, :, :, :, h] = r[3]

    _pool_map(one, [(b, h) for b in range(B) for h in range(nh)], threads)
    return dq, dk, dv, doff


def geometry(off, window, dilation=(1, 1, 1)):
    """Base corner and fraction of every sample: off [B,T,H,W,heads,P,3] ->
    base int32 and frac float32 of the same shape."""
    off = _f32(off)
    B, T, H, W, nh, P, _ = off.shape
    pos = grid_positions(T, H, W)
    base = np.zeros(off.shape, dtype=np.int32); frac = np.zeros(off.shape, dtype=np.float32)
    for b in range(B):
        for h in range(nh):
            bb, ff = geometry_queries((T, H, W), window, dilation, pos,
                                      off[b, :, :, :, h].reshape(-1, P, 3))
            base[b, :, :, :, h] = bb.reshape(T, H, W, P, 3)
            frac[b, :, :, :, h] = ff.reshape(T, H, W, P, 3)
    return base, frac


# ----------------------------------------------------------------------------
# Offset projection: Linear(C -> heads*P*3) of each token's query row.
# ----------------------------------------------------------------------------

def offset_proj(q2d, w, b=None) -> np.ndarray:
    """offsets[N, F] = q[N, C] @ w[F, C]^T + b[F], in float64."""
    out = _f64(q2d) @ _f64(w).T
    if b is not None:
        out += _f64(b)[None, :]
    return out


def offset_proj_backward(q2d, w, doff2d) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of the projection, in float64: (dq share = doff @ w,
    dW = doff^T @ q, db = column sums of doff)."""
    g = _f64(doff2d)
    return g @ _f64(w), g.T @ _f64(q2d), g.sum(axis=0)


# ----------------------------------------------------------------------------
# Depthwise 3-D convolution of the offset network, before the pointwise layer
# [MegaSlide-DiT, §5.3 Implementation considerations: nn.Conv3d with groups equal
# to the hidden size, followed by pointwise convolutions; Dutch and French
# summaries, "3D Deformable Slide Attention", Implementation: a lightweight
# depthwise 3-D convolution and a linear layer]. The pages give no kernel size;
# the reading here is 3x3x3, stride 1, zero padding 1 (output the size of the
# input), with a bias, applied to the query tensor [B,T,H,W,C] channel by
# channel, C = heads*head_dim, weight [C, 3, 3, 3] (torch's Conv3d weight
# [C, 1, 3, 3, 3] without its unit axis). Conv3d is a cross-correlation: tap
# (i, j, k) reads the input at offset (i-1, j-1, k-1).
# ----------------------------------------------------------------------------

def _pad1(x: np.ndarray) -> np.ndarray:
    B, T, H, W, C = x.shape
    xp = np.zeros((B, T + 2, H + 2, W + 2, C))
    xp[:, 1:-1, 1:-1, 1:-1] = x
    return xp


def dwconv3d(q, w, b=None) -> np.ndarray:
    """y[b,t,h,x,c] = bias[c] + sum over taps (i,j,k) in {0,1,2}^3 of
    w[c,i,j,k] * q[b, t+i-1, h+j-1, x+k-1, c], zero outside the grid; float64."""
    x = _f64(q)
    wt = _f64(w)
    B, T, H, W, C = x.shape
    xp = _pad1(x)
    y = np.zeros_like(x)
    for i in range(3):
        for j in range(3):
            for k in range(3):
                y += wt[:, i, j, k] * xp[:, i:i + T, j:j + H, k:k + W]
    if b is not None:
        y += _f64(b)
    return y


def dwconv3d_backward(q, w, dy) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of dwconv3d for an output gradient dy, float64:
    dq[b,t,h,x,c] = sum over taps of w[c,i,j,k] * dy[b, t-i+1, h-j+1, x-k+1, c]
    (zero outside), dw[c,i,j,k] = sum over all tokens of dy * q shifted by the
    tap, db[c] = sum over all tokens of dy."""
    g = _f64(dy)
    x = _f64(q)
    wt = _f64(w)
    B, T, H, W, C = g.shape
    gp = _pad1(g)
    xp = _pad1(x)
    dq = np.zeros_like(g)
    dw = np.zeros((C, 3, 3, 3))
    for i in range(3):
        for j in range(3):
            for k in range(3):
                dq += wt[:, i, j, k] * gp[:, 2 - i:2 - i + T, 2 - j:2 - j + H, 2 - k:2 - k + W]
                dw[:, i, j, k] = (g * xp[:, i:i + T, j:j + H, k:k + W]).sum(axis=(0, 1, 2, 3))
    return dq, dw, g.sum(axis=(0, 1, 2, 3))


# ----------------------------------------------------------------------------
# The transformer block around the operator. The pages keep layer normalisation
# and residual connections around their attention as usual, with dense
# projections for the queries, keys, values and output [MegaSlide-DiT, §5.3
# Implementation considerations]. Read as the plain pre-norm block:
#   h = LayerNorm(x); q, k, v = h W_q^T + b_q, h W_k^T + b_k, h W_v^T + b_v;
#   offsets = q W_off^T + b_off; o = 3D-DSA(q, k, v, offsets); y = x + o W_out^T + b_out
# over each token's C channels, all in float64 (the attention's offsets are
# rounded to single precision by the attention oracle, as everywhere).
# ----------------------------------------------------------------------------

def layernorm(x, gamma=None, beta=None, eps: float = 1e-6):
    """Over the last axis: (x - mean) / sqrt(var + eps) * gamma + beta, with the
    population variance. Returns (y, mean, rstd), float64."""
    x = _f64(x)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    y = (x - mean) * rstd
    if gamma is not None:
        y = y * _f64(gamma)
    if beta is not None:
        y = y + _f64(beta)
    return y, mean[..., 0], rstd[..., 0]


def layernorm_backward(x, gamma, dy, eps: float = 1e-6):
    """Gradients of layernorm for dL/dy = dy: (dx, dgamma, dbeta), float64.
    With xh the normalised input and g = dy * gamma:
    dx = rstd * (g - mean(g) - xh * mean(g * xh)); dgamma = sum of dy * xh and
    dbeta = sum of dy over every axis but the last."""
    x, dy = _f64(x), _f64(dy)
    _, mean, rstd = layernorm(x, None, None, eps)
    xh = (x - mean[..., None]) * rstd[..., None]
    g = dy * (_f64(gamma) if gamma is not None else 1.0)
    dx = rstd[..., None] * (g - g.mean(axis=-1, keepdims=True) - xh * (g * xh).mean(axis=-1, keepdims=True))
    axes = tuple(range(x.ndim - 1))
    return dx, (dy * xh).sum(axis=axes), dy.sum(axis=axes)


def linear(x2d, w, b=None) -> np.ndarray:
    """y[M, N] = x[M, K] @ w[N, K]^T + b[N], float64."""
    return offset_proj(x2d, w, b)


def linear_backward(x2d, w, dy2d) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dx = dy @ w, dw = dy^T @ x, db = column sums of dy), float64."""
    return offset_proj_backward(x2d, w, dy2d)


BLOCK_PARAMS = ("ln_g", "ln_b", "w_qkv", "b_qkv", "w_off", "b_off", "w_out", "b_out")


def block_forward(x, p, heads: int, window, dilation=(1, 1, 1), eps: float = 1e-6):
    """The block on x [B,T,H,W,C] with parameters p (BLOCK_PARAMS: ln_g/ln_b [C],
    w_qkv [3C, C], b_qkv [3C], w_off [heads*P*3, C], b_off [heads*P*3],
    w_out [C, C], b_out [C]). Returns a dict of every intermediate: h, q, k, v
    ([B,T,H,W,heads,d]), offsets, o, lse and the output y [B,T,H,W,C]."""
    x = _f64(x)
    B, T, H, W, C = x.shape
    d = C // heads
    P = window[0] * window[1] * window[2]
    x2 = x.reshape(-1, C)
    h, _, _ = layernorm(x2, p["ln_g"], p["ln_b"], eps)
    wqkv, bqkv = _f64(p["w_qkv"]), _f64(p["b_qkv"])
    q2, k2, v2 = (linear(h, wqkv[i * C:(i + 1) * C], bqkv[i * C:(i + 1) * C]) for i in range(3))
    act = lambda a: a.reshape(B, T, H, W, heads, d)
    off = linear(q2, p["w_off"], p["b_off"]).reshape(B, T, H, W, heads, P, 3)
    o, lse = forward(act(q2), act(k2), act(v2), off, window, dilation)
    y = x2 + linear(o.reshape(-1, C), p["w_out"], p["b_out"])
    return {"h": h.reshape(B, T, H, W, C), "q": act(q2), "k": act(k2), "v": act(v2), "offsets": off, "o": o,
            "lse": lse, "y": y.reshape(B, T, H, W, C)}


def block_backward(x, p, dy, heads: int, window, dilation=(1, 1, 1), eps: float = 1e-6):
    """Gradients of block_forward for dL/dy = dy: a dict with dx and the
    gradient of every parameter (d<name>), plus the attention's inputs'
    gradients dq, dk, dv, doffsets and do, all float64. The chain rule through
    the block: the output projection, the attention (its offsets depend on q
    through the offset projection), the q/k/v projections and the layer
    normalisation, plus the residual path dx += dy."""
    x, dy = _f64(x), _f64(dy)
    B, T, H, W, C = x.shape
    d = C // heads
    f = block_forward(x, p, heads, window, dilation, eps)
    x2, dy2 = x.reshape(-1, C), dy.reshape(-1, C)
    do2, dw_out, db_out = linear_backward(f["o"].reshape(-1, C), p["w_out"], dy2)
    dq, dk, dv, doff = backward(f["q"], f["k"], f["v"], f["offsets"], do2.reshape(B, T, H, W, heads, d), window,
                                dilation)
    q2 = f["q"].reshape(-1, C)
    dq_off, dw_off, db_off = linear_backward(q2, p["w_off"], doff.reshape(q2.shape[0], -1))
    dq2 = dq.reshape(-1, C) + dq_off
    h2 = f["h"].reshape(-1, C)
    wqkv = _f64(p["w_qkv"])
    dh = np.zeros_like(h2)
    dw_qkv = np.zeros_like(wqkv)
    db_qkv = np.zeros(3 * C)
    for i, g in enumerate((dq2, dk.reshape(-1, C), dv.reshape(-1, C))):
        a, b, c = linear_backward(h2, wqkv[i * C:(i + 1) * C], g)
        dh += a
        dw_qkv[i * C:(i + 1) * C] = b
        db_qkv[i * C:(i + 1) * C] = c
    dx_ln, dln_g, dln_b = layernorm_backward(x2, p["ln_g"], dh, eps)
    dx = dy2 + dx_ln
    return {"dx": dx.reshape(x.shape), "dln_g": dln_g, "dln_b": dln_b, "dw_qkv": dw_qkv, "db_qkv": db_qkv,
            "dw_off": dw_off, "db_off": db_off, "dw_out": dw_out, "db_out": db_out, "dq": dq, "dk": dk, "dv": dv,
            "doffsets": doff, "do": do2.reshape(B, T, H, W, heads, d), "dh": dh.reshape(x.shape)}


# ----------------------------------------------------------------------------
# Hybrid attention: sparse global tokens with local 3D-DSA [MegaSlide-DiT, §11
# Limitations and Discussion, future work (i)]: each query's P samples and the
# G global tokens of its (batch item, head) share one softmax (see the C file).
# ----------------------------------------------------------------------------

def forward_hybrid(q, k, v, off, gk, gv, window, dilation=(1, 1, 1), scale=None, threads=None):
    """q, k, v [B,T,H,W,heads,d], off [B,T,H,W,heads,P,3], gk, gv [B,G,heads,d].
    Returns o [B,T,H,W,heads,d] and lse [B,T,H,W,heads], float64."""
    q, k, v, off, gk, gv = _f64(q), _f64(k), _f64(v), _f32(off), _f64(gk), _f64(gv)
    B, T, H, W, nh, d = q.shape
    G = gk.shape[1]
    P = window[0] * window[1] * window[2]
    scale = default_scale(d) if scale is None else scale
    pos = grid_positions(T, H, W)
    N = T * H * W
    o = np.zeros_like(q); lse = np.zeros((B, T, H, W, nh))

    def one(bh):
        b, h = bh
        pr = _problem((T, H, W), d, window, dilation, scale, (0, 0, 0), (T, H, W))
        oo = np.zeros((N, d)); ll = np.zeros(N)
        # every array handed to the C call is held by a name for the call's duration
        qq = np.ascontiguousarray(q[b, :, :, :, h].reshape(N, d))
        ff = np.ascontiguousarray(off[b, :, :, :, h].reshape(N, P, 3))
        kk = np.ascontiguousarray(k[b, :, :, :, h])
        vv = np.ascontiguousarray(v[b, :, :, :, h])
        gkk = np.ascontiguousarray(gk[b, :, h])
        gvv = np.ascontiguousarray(gv[b, :, h])
        rc = lib().orc_forward_hybrid(ctypes.byref(pr), N, _ptr(pos), _ptr(qq), _ptr(ff), _ptr(kk), _ptr(vv), G,
                                      _ptr(gkk), _ptr(gvv), _ptr(oo), _ptr(ll))
        _check(rc, "forward_hybrid")
        o[b, :, :, :, h] = oo.reshape(T, H, W, d)
        lse[b, :, :, :, h] = ll.reshape(T, H, W)

    _pool_map(one, [(b, h) for b in range(B) for h in range(nh)], threads)
    return o, lse


def backward_hybrid(q, k, v, off, gk, gv, dout, window, dilation=(1, 1, 1), scale=None, threads=None):
    """Gradients of forward_hybrid: dq, dk, dv [B,T,H,W,heads,d], doff
    [B,T,H,W,heads,P,3], dgk, dgv [B,G,heads,d], float64."""
    q, k, v, off, gk, gv, dout = _f64(q), _f64(k), _f64(v), _f32(off), _f64(gk), _f64(gv), _f64(dout)
    B, T, H, W, nh, d = q.shape
    G = gk.shape[1]
    P = window[0] * window[1] * window[2]
    scale = default_scale(d) if scale is None else scale
    pos = grid_positions(T, H, W)
    N = T * H * W
    dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v); doff = np.zeros(off.shape)
    dgk = np.zeros_like(gk); dgv = np.zeros_like(gv)

    def one(bh):
        b, h = bh
        pr = _problem((T, H, W), d, window, dilation, scale, (0, 0, 0), (T, H, W))
        dqq = np.zeros((N, d)); dff = np.zeros((N, P, 3))
        dK = np.zeros((T, H, W, d)); dV = np.zeros((T, H, W, d))
        dGK = np.zeros((G, d)); dGV = np.zeros((G, d))
        qq = np.ascontiguousarray(q[b, :, :, :, h].reshape(N, d))
        ff = np.ascontiguousarray(off[b, :, :, :, h].reshape(N, P, 3))
        kk = np.ascontiguousarray(k[b, :, :, :, h])
        vv = np.ascontiguousarray(v[b, :, :, :, h])
        gkk = np.ascontiguousarray(gk[b, :, h])
        gvv = np.ascontiguousarray(gv[b, :, h])
        gg = np.ascontiguousarray(dout[b, :, :, :, h].reshape(N, d))
        rc = lib().orc_backward_hybrid(ctypes.byref(pr), N, _ptr(pos), _ptr(qq), _ptr(ff), _ptr(kk), _ptr(vv), G,
                                       _ptr(gkk), _ptr(gvv), _ptr(gg), _ptr(dqq), _ptr(dff), _ptr(dK), _ptr(dV),
                                       _ptr(dGK), _ptr(dGV))
        _check(rc, "backward_hybrid")
        dq[b, :, :, :, h] = dqq.reshape(T, H, W, d)
        doff[b, :, :, :, h] = dff.reshape(T, H, W, P, 3)
        dk[b, :, :, :, h] = dK
        dv[b, :, :, :, h] = dV
        dgk[b, :, h] = dGK
        dgv[b, :, h] = dGV

    _pool_map(one, [(b, h) for b in range(B) for h in range(nh)], threads)
    return dq, dk, dv, doff, dgk, dgv


def forward_hybrid_queries(grid, window, dilation, scale, qpos, q, off, box_origin, K, V, GK, GV, threads=1):
    """forward_queries with the G global rows GK, GV [G, d] of the head joining
    the softmax. Returns o [n,d], lse [n]."""
    qpos = np.ascontiguousarray(qpos, dtype=np.int32)
    q, K, V, off, GK, GV = _f64(q), _f64(K), _f64(V), _f32(off), _f64(GK), _f64(GV)
    n, d = q.shape
    G = GK.shape[0]
    pr = _problem(grid, d, window, dilation, scale, box_origin, K.shape[:3])
    o = np.zeros((n, d)); lse = np.zeros(n)

    def run(r):
        i0, i1 = r
        if i1 <= i0:
            return 0
        return lib().orc_forward_hybrid(ctypes.byref(pr), i1 - i0, _ptr(qpos[i0:i1]), _ptr(q[i0:i1]),
                                        _ptr(off[i0:i1]), _ptr(K), _ptr(V), G, _ptr(GK), _ptr(GV), _ptr(o[i0:i1]),
                                        _ptr(lse[i0:i1]))

    for rc in _pool_map(run, _runs(n, threads), threads):
        _check(rc, "forward_hybrid")
    return o, lse


def backward_hybrid_queries(grid, window, dilation, scale, qpos, q, off, box_origin, K, V, GK, GV, dout,
                            want_kv=False, threads=1):
    """Gradients of listed queries with the global rows: dq [n,d], doff
    [n,P,3], their contributions dGK, dGV [G,d] to the global rows' gradients
    (with threads > 1, the runs' sums added in run order) and, with want_kv
    (one run), dK, dV over the box; else those two are None."""
    qpos = np.ascontiguousarray(qpos, dtype=np.int32)
    q, K, V, off, GK, GV, dout = _f64(q), _f64(K), _f64(V), _f32(off), _f64(GK), _f64(GV), _f64(dout)
    n, d = q.shape
    G = GK.shape[0]
    P = window[0] * window[1] * window[2]
    pr = _problem(grid, d, window, dilation, scale, box_origin, K.shape[:3])
    dq = np.zeros((n, d)); doff = np.zeros((n, P, 3))
    dK = np.zeros(K.shape) if want_kv else None
    dV = np.zeros(V.shape) if want_kv else None
    runs = _runs(n, 1 if want_kv else threads)
    dgk = [np.zeros((G, d)) for _ in runs]
    dgv = [np.zeros((G, d)) for _ in runs]

    def run(i):
        i0, i1 = runs[i]
        if i1 <= i0:
            return 0
        return lib().orc_backward_hybrid(ctypes.byref(pr), i1 - i0, _ptr(qpos[i0:i1]), _ptr(q[i0:i1]),
                                         _ptr(off[i0:i1]), _ptr(K), _ptr(V), G, _ptr(GK), _ptr(GV),
                                         _ptr(dout[i0:i1]), _ptr(dq[i0:i1]), _ptr(doff[i0:i1]), _ptr(dK), _ptr(dV),
                                         _ptr(dgk[i]), _ptr(dgv[i]))

    for rc in _pool_map(run, list(range(len(runs))), len(runs)):
        _check(rc, "backward_hybrid")
    return dq, doff, sum(dgk), sum(dgv), dK, dV
