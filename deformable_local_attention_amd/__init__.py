"""Python binding of libdsa3d -- 3D Deformable Slide Attention on MI355X.

Argument marshalling only: every step of the operator runs in the HIP kernels
of libdsa3d.so (built by `python -m deformable_local_attention_amd.build`).
torch supplies device memory and the current stream. There is no CPU or
PyTorch fallback: if the library is missing, every call raises.

Low-level functions carry the C names (dsa3d_forward, dsa3d_backward, ...)
and take a `Desc` plus torch tensors; `forward`, `backward`, `offset_proj`
and `offset_proj_backward` are conveniences that build the descriptor and
allocate outputs and workspaces with torch.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "Desc", "DSA3DError", "lib", "library_path", "make_desc",
    "dsa3d_version", "dsa3d_status_string", "dsa3d_validate", "dsa3d_workspace_size", "dsa3d_workspace_min",
    "dsa3d_offset_proj_forward", "dsa3d_forward", "dsa3d_backward", "dsa3d_offset_proj_backward",
    "dsa3d_debug_geometry", "forward", "backward", "offset_proj", "offset_proj_backward",
    "DSA3D_F32", "DSA3D_BF16", "WS_FORWARD", "WS_BACKWARD", "WS_PROJ_BACKWARD", "WS_DWCONV_BACKWARD",
    "WS_BACKWARD_FIXED",
    "dsa3d_dwconv_forward", "dsa3d_dwconv_backward", "dwconv", "dwconv_backward",
    "dsa3d_set_launch_log", "LaunchLog", "launch_timer", "KERNELS", "dsa3d_backward_noalloc",
    "NOALLOC_SCRATCH_BYTES", "dsa3d_layernorm_forward", "dsa3d_layernorm_workspace_size", "dsa3d_layernorm_backward",
    "dsa3d_linear_forward", "dsa3d_linear_workspace_size", "dsa3d_linear_backward", "layernorm", "linear",
    "dtype_code", "dsa3d_forward_hybrid", "dsa3d_backward_hybrid", "dsa3d_hybrid_workspace_size",
    "dsa3d_hybrid_workspace_min", "forward_hybrid", "backward_hybrid",
]

DSA3D_F32, DSA3D_BF16 = 0, 1
WS_FORWARD, WS_BACKWARD, WS_PROJ_BACKWARD, WS_DWCONV_BACKWARD, WS_BACKWARD_FIXED = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 64 << 20  # DSA3D_NOALLOC_SCRATCH_BYTES
EXPORTS = ("dsa3d_version", "dsa3d_status_string", "dsa3d_validate", "dsa3d_workspace_size",
           "dsa3d_workspace_min", "dsa3d_offset_proj_forward", "dsa3d_forward", "dsa3d_backward",
           "dsa3d_offset_proj_backward", "dsa3d_debug_geometry", "dsa3d_dwconv_forward", "dsa3d_dwconv_backward",
           "dsa3d_set_launch_log", "dsa3d_backward_noalloc", "dsa3d_layernorm_forward",
           "dsa3d_layernorm_workspace_size", "dsa3d_layernorm_backward", "dsa3d_linear_forward",
           "dsa3d_linear_workspace_size", "dsa3d_linear_backward", "dsa3d_forward_hybrid", "dsa3d_backward_hybrid",
           "dsa3d_hybrid_workspace_size", "dsa3d_hybrid_workspace_min")
# kernel ids of the launch log (dsa3d_kernel)
KERNELS = {1: "proj_forward", 2: "forward", 3: "bwd_query", 4: "bwd_key", 5: "fill", 6: "proj_bwd_dq",
           7: "proj_bwd_dw", 8: "split_sum", 9: "colsum", 10: "geometry", 11: "bwd_scan", 12: "bwd_count",
           13: "bwd_sort", 14: "transpose", 15: "dwconv", 16: "dwconv_wgrad", 17: "dwconv_dq", 18: "layernorm",
           19: "layernorm_bwd", 20: "linear_forward", 21: "linear_bwd_dx", 22: "linear_bwd_dw",
           23: "hybrid_forward", 24: "hybrid_bwd_query", 25: "hybrid_bwd_rows"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return os.environ.get("DSA3D_LIBRARY", os.path.join(_HERE, "libdsa3d.so"))


class DSA3DError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {message} (status {status})")
        self.status = status


class Desc(ctypes.Structure):
    """Mirror of `dsa3d_desc` (include/dsa3d.h)."""
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64), ("W", ctypes.c_int64),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kt", ctypes.c_int32), ("kh", ctypes.c_int32), ("kw", ctypes.c_int32),
                ("P", ctypes.c_int32),
                ("dil_t", ctypes.c_int32), ("dil_h", ctypes.c_int32), ("dil_w", ctypes.c_int32),
                ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float),
                ("deterministic", ctypes.c_int32)]


class LaunchLog(ctypes.Structure):
    """Mirror of `dsa3d_launch_log`."""
    _fields_ = [("capacity", ctypes.c_int32), ("count", ctypes.c_int32),
                ("kernel", ctypes.POINTER(ctypes.c_int32)),
                ("start", ctypes.POINTER(ctypes.c_void_p)), ("stop", ctypes.POINTER(ctypes.c_void_p))]


def lib() -> ctypes.CDLL:
    """Load libdsa3d.so once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise ImportError(f"libdsa3d.so not found at {path}: build it with "
                                  "`python -m deformable_local_attention_amd.build` (needs ROCm hipcc)")
            L = ctypes.CDLL(path)
            vp, sz, dp, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(Desc), ctypes.c_int64
            sig = {
                "dsa3d_version": ([], ctypes.c_int),
                "dsa3d_status_string": ([ctypes.c_int], ctypes.c_char_p),
                "dsa3d_validate": ([dp], ctypes.c_int),
                "dsa3d_workspace_size": ([dp, ctypes.c_int], sz),
                "dsa3d_workspace_min": ([dp, ctypes.c_int], sz),
                "dsa3d_offset_proj_forward": ([dp, vp, vp, vp, vp, vp], ctypes.c_int),
                "dsa3d_forward": ([dp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
                "dsa3d_backward": ([dp] + [vp] * 11 + [vp, sz, vp], ctypes.c_int),
                "dsa3d_offset_proj_backward": ([dp, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
                "dsa3d_debug_geometry": ([dp, vp, vp, vp, vp], ctypes.c_int),
                "dsa3d_dwconv_forward": ([dp, vp, vp, vp, vp, vp], ctypes.c_int),
                "dsa3d_dwconv_backward": ([dp, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
                "dsa3d_set_launch_log": ([ctypes.POINTER(LaunchLog)], ctypes.c_int),
                "dsa3d_backward_noalloc": ([dp] + [vp] * 12, ctypes.c_int),
                "dsa3d_layernorm_forward": ([ctypes.c_int, i64, i64, ctypes.c_float] + [vp] * 6, ctypes.c_int),
                "dsa3d_layernorm_workspace_size": ([i64, i64], sz),
                "dsa3d_layernorm_backward": ([ctypes.c_int, i64, i64] + [vp] * 9 + [sz, vp], ctypes.c_int),
                "dsa3d_linear_forward": ([ctypes.c_int, i64, i64, i64] + [vp] * 6, ctypes.c_int),
                "dsa3d_linear_workspace_size": ([ctypes.c_int, i64, i64, i64], sz),
                "dsa3d_linear_backward": ([ctypes.c_int, i64, i64, i64] + [vp] * 8 + [sz, vp], ctypes.c_int),
                "dsa3d_forward_hybrid": ([dp] + [vp] * 4 + [ctypes.c_int32] + [vp] * 5, ctypes.c_int),
                "dsa3d_backward_hybrid": ([dp] + [vp] * 7 + [ctypes.c_int32] + [vp] * 9 + [sz, vp], ctypes.c_int),
                "dsa3d_hybrid_workspace_size": ([dp, ctypes.c_int32, ctypes.c_int], sz),
                "dsa3d_hybrid_workspace_min": ([dp, ctypes.c_int32, ctypes.c_int], sz),
            }
            for name, (args, res) in sig.items():
                f = getattr(L, name)
                f.argtypes = args
                f.restype = res
            _lib = L
    return _lib


# ---------------------------------------------------------------------------
# descriptors and marshalling
# ---------------------------------------------------------------------------

def make_desc(B: int, T: int, H: int, W: int, heads: int, head_dim: int, window: Sequence[int],
              dilation: Sequence[int] = (1, 1, 1), dtype=torch.bfloat16, scale: float = 0.0,
              deterministic: bool = False) -> Desc:
    kt, kh, kw = window
    code = {torch.float32: DSA3D_F32, torch.bfloat16: DSA3D_BF16}.get(dtype, -1)
    return Desc(B, T, H, W, heads, head_dim, kt, kh, kw, kt * kh * kw, dilation[0], dilation[1], dilation[2],
                code, float(scale), 1 if deterministic else 0)


def desc_like(q: torch.Tensor, window, dilation=(1, 1, 1), scale: float = 0.0, deterministic: bool = False) -> Desc:
    B, T, H, W, nh, d = q.shape
    return make_desc(B, T, H, W, nh, d, window, dilation, q.dtype, scale, deterministic)


_TORCH_DTYPE = {DSA3D_F32: torch.float32, DSA3D_BF16: torch.bfloat16}


class _Args:
    """Checks the tensors of one call against its descriptor before any
    pointer reaches the library: each must be a contiguous tensor on the same
    GPU, of the expected element type and size (a tensor with the expected
    number of dimensions must have exactly the expected shape; another view of
    the same elements, such as [N, C] for [B,T,H,W,heads,d], is accepted).
    Raises ValueError (TypeError for a non-tensor)."""

    def __init__(self, fn: str, desc: Optional[Desc], dtype: Optional[int] = None):
        self.fn = fn
        self.tensors = []
        if desc is None:  # the block's calls: plain sizes, shapes given per tensor
            self.dt = _TORCH_DTYPE.get(dtype)
            return
        self.dt = _TORCH_DTYPE.get(desc.dtype)  # None: the library reports the unsupported dtype
        tok = (desc.B, desc.T, desc.H, desc.W)
        self.act = tok + (desc.heads, desc.head_dim)
        self.off = tok + (desc.heads, desc.P, 3)
        self.lse = tok + (desc.heads,)
        self.C = desc.heads * desc.head_dim
        self.F = desc.heads * desc.P * 3

    def __call__(self, name: str, t, shape, dtype="run", optional: bool = False):
        if t is None:
            if optional:
                return None
            raise ValueError(f"{self.fn}: {name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.fn}: {name} must be a torch.Tensor, not {type(t).__name__}")
        want = self.dt if dtype == "run" else dtype
        if want is not None and t.dtype != want:
            raise ValueError(f"{self.fn}: {name} has dtype {t.dtype}, expected {want}")
        if shape is not None:
            n = math.prod(shape)
            if t.numel() != n or (t.dim() == len(shape) and tuple(t.shape) != tuple(shape)):
                raise ValueError(f"{self.fn}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{self.fn}: {name} is not contiguous")
        self.tensors.append((name, t))
        return t

    def pointers(self, *ts):
        """Device pointers of the checked tensors, once every one of them is
        known to lie on one GPU (type and size errors are reported first)."""
        for name, t in self.tensors:
            if t.device.type != "cuda":
                raise ValueError(f"{self.fn}: {name} is on {t.device}; libdsa3d takes GPU tensors")
            if t.device != self.tensors[0][1].device:
                raise ValueError(f"{self.fn}: {name} is on {t.device}, the others on {self.tensors[0][1].device}")
        return [None if t is None else ctypes.c_void_p(t.data_ptr()) for t in ts]

    def workspace(self, t):
        """(the checked workspace, its size in bytes)."""
        if t is None:
            return None, 0
        return self("workspace", t, None, dtype=None), t.numel() * t.element_size()


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn: str, status: int):
    if status != 0:
        raise DSA3DError(fn, status, dsa3d_status_string(status))


# ---------------------------------------------------------------------------
# the C entry points, one to one
# ---------------------------------------------------------------------------

def dsa3d_version() -> int:
    return lib().dsa3d_version()


def dsa3d_status_string(status: int) -> str:
    return lib().dsa3d_status_string(status).decode()


def dsa3d_validate(desc: Desc) -> int:
    return lib().dsa3d_validate(ctypes.byref(desc))


def dsa3d_workspace_size(desc: Desc, kind: int) -> int:
    return lib().dsa3d_workspace_size(ctypes.byref(desc), kind)


def dsa3d_workspace_min(desc: Desc, kind: int) -> int:
    return lib().dsa3d_workspace_min(ctypes.byref(desc), kind)


def dsa3d_offset_proj_forward(desc: Desc, q, w, bias, offsets, stream=None):
    a = _Args("dsa3d_offset_proj_forward", desc)
    args = (a("q", q, a.act), a("w", w, (a.F, a.C)), a("bias", bias, (a.F,), optional=True),
            a("offsets", offsets, a.off))
    _check("dsa3d_offset_proj_forward",
           lib().dsa3d_offset_proj_forward(ctypes.byref(desc), *a.pointers(*args), _stream(stream)))


def dsa3d_forward(desc: Desc, q, k, v, offsets, out, lse, stream=None):
    a = _Args("dsa3d_forward", desc)
    args = (a("q", q, a.act), a("k", k, a.act), a("v", v, a.act), a("offsets", offsets, a.off, optional=True),
            a("out", out, a.act), a("lse", lse, a.lse, torch.float32))
    _check("dsa3d_forward", lib().dsa3d_forward(ctypes.byref(desc), *a.pointers(*args), _stream(stream)))


def dsa3d_backward(desc: Desc, q, k, v, offsets, out, lse, dout, dq, dk, dv, doffsets, workspace,
                   stream=None):
    a = _Args("dsa3d_backward", desc)
    args = (a("q", q, a.act), a("k", k, a.act), a("v", v, a.act), a("offsets", offsets, a.off, optional=True),
            a("out", out, a.act), a("lse", lse, a.lse, torch.float32), a("dout", dout, a.act),
            a("dq", dq, a.act), a("dk", dk, a.act), a("dv", dv, a.act),
            a("doffsets", doffsets, a.off, optional=True))
    ws, nbytes = a.workspace(workspace)
    _check("dsa3d_backward",
           lib().dsa3d_backward(ctypes.byref(desc), *a.pointers(*args, ws), nbytes, _stream(stream)))


def dsa3d_backward_noalloc(desc: Desc, q, k, v, offsets, out, lse, dout, dq, dk, dv, doffsets, stream=None):
    a = _Args("dsa3d_backward_noalloc", desc)
    args = (a("q", q, a.act), a("k", k, a.act), a("v", v, a.act), a("offsets", offsets, a.off, optional=True),
            a("out", out, a.act), a("lse", lse, a.lse, torch.float32), a("dout", dout, a.act),
            a("dq", dq, a.act), a("dk", dk, a.act), a("dv", dv, a.act),
            a("doffsets", doffsets, a.off, optional=True))
    _check("dsa3d_backward_noalloc",
           lib().dsa3d_backward_noalloc(ctypes.byref(desc), *a.pointers(*args), _stream(stream)))


def dsa3d_offset_proj_backward(desc: Desc, q, w, doffsets, dq_accum, dw, dbias, workspace, stream=None):
    a = _Args("dsa3d_offset_proj_backward", desc)
    args = (a("q", q, a.act), a("w", w, (a.F, a.C)), a("doffsets", doffsets, a.off),
            a("dq_accum", dq_accum, a.act), a("dw", dw, (a.F, a.C), torch.float32),
            a("dbias", dbias, (a.F,), torch.float32, optional=True))
    ws, nbytes = a.workspace(workspace)
    _check("dsa3d_offset_proj_backward",
           lib().dsa3d_offset_proj_backward(ctypes.byref(desc), *a.pointers(*args, ws), nbytes,
                                            _stream(stream)))


def dsa3d_dwconv_forward(desc: Desc, q, wt, bias, y, stream=None):
    a = _Args("dsa3d_dwconv_forward", desc)
    args = (a("q", q, a.act), a("wt", wt, (a.C, 3, 3, 3)), a("bias", bias, (a.C,), optional=True),
            a("y", y, a.act))
    _check("dsa3d_dwconv_forward",
           lib().dsa3d_dwconv_forward(ctypes.byref(desc), *a.pointers(*args), _stream(stream)))


def dsa3d_dwconv_backward(desc: Desc, q, wt, dy, dq_accum, dwt, dbias, workspace, stream=None):
    a = _Args("dsa3d_dwconv_backward", desc)
    args = (a("q", q, a.act), a("wt", wt, (a.C, 3, 3, 3)), a("dy", dy, a.act), a("dq_accum", dq_accum, a.act),
            a("dwt", dwt, (a.C, 3, 3, 3), torch.float32), a("dbias", dbias, (a.C,), torch.float32, optional=True))
    ws, nbytes = a.workspace(workspace)
    _check("dsa3d_dwconv_backward",
           lib().dsa3d_dwconv_backward(ctypes.byref(desc), *a.pointers(*args, ws), nbytes, _stream(stream)))


# ---------------------------------------------------------------------------
# hybrid attention: global tokens in each query's softmax
# ---------------------------------------------------------------------------

def dsa3d_forward_hybrid(desc: Desc, q, k, v, offsets, G: int, gk, gv, out, lse, stream=None):
    a = _Args("dsa3d_forward_hybrid", desc)
    grow = (desc.B, G, desc.heads, desc.head_dim)
    args = (a("q", q, a.act), a("k", k, a.act), a("v", v, a.act), a("offsets", offsets, a.off, optional=True))
    glob = (a("gk", gk, grow), a("gv", gv, grow))
    outs = (a("out", out, a.act), a("lse", lse, a.lse, torch.float32))
    p = a.pointers(*args, *glob, *outs)
    _check("dsa3d_forward_hybrid", lib().dsa3d_forward_hybrid(ctypes.byref(desc), *p[:4], G, *p[4:],
                                                              _stream(stream)))


def dsa3d_hybrid_workspace_size(desc: Desc, G: int, kind: int) -> int:
    return lib().dsa3d_hybrid_workspace_size(ctypes.byref(desc), G, kind)


def dsa3d_hybrid_workspace_min(desc: Desc, G: int, kind: int) -> int:
    return lib().dsa3d_hybrid_workspace_min(ctypes.byref(desc), G, kind)


def dsa3d_backward_hybrid(desc: Desc, q, k, v, offsets, out, lse, dout, G: int, gk, gv, dq, dk, dv, doffsets, dgk,
                          dgv, workspace, stream=None):
    a = _Args("dsa3d_backward_hybrid", desc)
    grow = (desc.B, G, desc.heads, desc.head_dim)
    first = (a("q", q, a.act), a("k", k, a.act), a("v", v, a.act), a("offsets", offsets, a.off, optional=True),
             a("out", out, a.act), a("lse", lse, a.lse, torch.float32), a("dout", dout, a.act))
    rest = (a("gk", gk, grow), a("gv", gv, grow), a("dq", dq, a.act), a("dk", dk, a.act), a("dv", dv, a.act),
            a("doffsets", doffsets, a.off, optional=True), a("dgk", dgk, grow), a("dgv", dgv, grow))
    ws, nbytes = a.workspace(workspace)
    p = a.pointers(*first, *rest, ws)
    _check("dsa3d_backward_hybrid", lib().dsa3d_backward_hybrid(ctypes.byref(desc), *p[:7], G, *p[7:], nbytes,
                                                                _stream(stream)))


def forward_hybrid(q, k, v, offsets, gk, gv, window, dilation=(1, 1, 1), scale: float = 0.0, stream=None):
    """Returns (out, lse) of the joint softmax over the local samples and the
    G global rows gk, gv [B, G, heads, d]."""
    desc = desc_like(q, window, dilation, scale)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:5], dtype=torch.float32, device=q.device)
    dsa3d_forward_hybrid(desc, q, k, v, offsets, gk.shape[1], gk, gv, out, lse, stream)
    return out, lse


def backward_hybrid(q, k, v, offsets, out, lse, dout, gk, gv, window, dilation=(1, 1, 1), scale: float = 0.0,
                    deterministic: bool = False, workspace: Optional[torch.Tensor] = None, stream=None):
    """Returns (dq, dk, dv, doffsets, dgk, dgv)."""
    desc = desc_like(q, window, dilation, scale, deterministic)
    G = gk.shape[1]
    if workspace is None:
        n = dsa3d_hybrid_workspace_size(desc, G, WS_BACKWARD if offsets is not None else WS_BACKWARD_FIXED)
        workspace = torch.empty((n + 15) // 16 * 16, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    doff = torch.empty_like(offsets) if offsets is not None else None
    dgk, dgv = torch.empty_like(gk), torch.empty_like(gv)
    dsa3d_backward_hybrid(desc, q, k, v, offsets, out, lse, dout, G, gk, gv, dq, dk, dv, doff, dgk, dgv, workspace,
                          stream)
    return dq, dk, dv, doff, dgk, dgv


# ---------------------------------------------------------------------------
# the transformer block around the operator: layer normalisation and linear layers
# ---------------------------------------------------------------------------

def dtype_code(dtype: torch.dtype) -> int:
    return {torch.float32: DSA3D_F32, torch.bfloat16: DSA3D_BF16}.get(dtype, -1)


def dsa3d_layernorm_forward(dtype: int, M: int, N: int, eps: float, x, gamma, beta, y, stats, stream=None):
    a = _Args("dsa3d_layernorm_forward", None, dtype)
    args = (a("x", x, (M, N)), a("gamma", gamma, (N,), optional=True), a("beta", beta, (N,), optional=True),
            a("y", y, (M, N)), a("stats", stats, (M, 2), torch.float32))
    _check("dsa3d_layernorm_forward",
           lib().dsa3d_layernorm_forward(dtype, M, N, float(eps), *a.pointers(*args), _stream(stream)))


def dsa3d_layernorm_workspace_size(M: int, N: int) -> int:
    return lib().dsa3d_layernorm_workspace_size(M, N)


def dsa3d_layernorm_backward(dtype: int, M: int, N: int, x, gamma, stats, dy, dres, dx, dgamma, dbeta, workspace,
                             stream=None):
    a = _Args("dsa3d_layernorm_backward", None, dtype)
    args = (a("x", x, (M, N)), a("gamma", gamma, (N,), optional=True), a("stats", stats, (M, 2), torch.float32),
            a("dy", dy, (M, N)), a("dres", dres, (M, N), optional=True), a("dx", dx, (M, N)),
            a("dgamma", dgamma, (N,), torch.float32, optional=True),
            a("dbeta", dbeta, (N,), torch.float32, optional=True))
    ws, nbytes = a.workspace(workspace)
    _check("dsa3d_layernorm_backward",
           lib().dsa3d_layernorm_backward(dtype, M, N, *a.pointers(*args, ws), nbytes, _stream(stream)))


def dsa3d_linear_forward(dtype: int, M: int, N: int, K: int, x, w, bias, residual, y, stream=None):
    a = _Args("dsa3d_linear_forward", None, dtype)
    args = (a("x", x, (M, K)), a("w", w, (N, K)), a("bias", bias, (N,), optional=True),
            a("residual", residual, (M, N), optional=True), a("y", y, (M, N)))
    _check("dsa3d_linear_forward", lib().dsa3d_linear_forward(dtype, M, N, K, *a.pointers(*args), _stream(stream)))


def dsa3d_linear_workspace_size(dtype: int, M: int, N: int, K: int) -> int:
    return lib().dsa3d_linear_workspace_size(dtype, M, N, K)


def dsa3d_linear_backward(dtype: int, M: int, N: int, K: int, x, w, dy, dres, dx, dw, dbias, workspace,
                          stream=None):
    a = _Args("dsa3d_linear_backward", None, dtype)
    args = (a("x", x, (M, K)), a("w", w, (N, K)), a("dy", dy, (M, N)), a("dres", dres, (M, K), optional=True),
            a("dx", dx, (M, K)), a("dw", dw, (N, K), torch.float32),
            a("dbias", dbias, (N,), torch.float32, optional=True))
    ws, nbytes = a.workspace(workspace)
    _check("dsa3d_linear_backward",
           lib().dsa3d_linear_backward(dtype, M, N, K, *a.pointers(*args, ws), nbytes, _stream(stream)))


def layernorm(x, gamma, beta, eps: float = 1e-6, stream=None):
    """Layer normalisation over the last axis; returns (y, stats [rows, 2] float32)."""
    N = x.shape[-1]
    M = x.numel() // N
    y = torch.empty_like(x)
    stats = torch.empty((M, 2), dtype=torch.float32, device=x.device)
    dsa3d_layernorm_forward(dtype_code(x.dtype), M, N, eps, x, gamma, beta, y, stats, stream)
    return y, stats


def linear(x, w, bias=None, residual=None, stream=None):
    """y = x . w^T + bias (+ residual) over the last axis of x."""
    K = x.shape[-1]
    M = x.numel() // K
    N = w.shape[0]
    y = torch.empty(tuple(x.shape[:-1]) + (N,), dtype=x.dtype, device=x.device)
    dsa3d_linear_forward(dtype_code(x.dtype), M, N, K, x, w, bias, residual, y, stream)
    return y


def dsa3d_set_launch_log(log: Optional[LaunchLog]):
    _check("dsa3d_set_launch_log", lib().dsa3d_set_launch_log(None if log is None else ctypes.byref(log)))


def dsa3d_debug_geometry(desc: Desc, offsets, base, frac, stream=None):
    a = _Args("dsa3d_debug_geometry", desc)
    args = (a("offsets", offsets, a.off), a("base", base, a.off, torch.int32), a("frac", frac, a.off, torch.float32))
    _check("dsa3d_debug_geometry",
           lib().dsa3d_debug_geometry(ctypes.byref(desc), *a.pointers(*args), _stream(stream)))


class launch_timer:
    """Context manager: log every libdsa3d kernel launched on this thread with
    HIP events (torch.cuda.Event handles) and report per-kernel durations.

        with launch_timer(capacity=256) as lt:
            ...libdsa3d calls...
        torch.cuda.synchronize(); lt.durations_ms() -> {"backward": [..], ...}
    """

    def __init__(self, capacity: int = 256):
        self.events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(capacity)]
        for a, b in self.events:  # torch creates the HIP event at its first record
            a.record(); b.record()
        self._kern = (ctypes.c_int32 * capacity)()
        self._start = (ctypes.c_void_p * capacity)(*[a.cuda_event for a, _ in self.events])
        self._stop = (ctypes.c_void_p * capacity)(*[b.cuda_event for _, b in self.events])
        self.log = LaunchLog(capacity, 0, self._kern, self._start, self._stop)

    def __enter__(self):
        torch.cuda.synchronize()
        _check("dsa3d_set_launch_log", lib().dsa3d_set_launch_log(ctypes.byref(self.log)))
        return self

    def __exit__(self, *exc):
        lib().dsa3d_set_launch_log(None)
        return False

    @property
    def count(self) -> int:
        return self.log.count

    def durations_ms(self):
        out = {}
        for i in range(self.log.count):
            a, b = self.events[i]
            out.setdefault(KERNELS.get(self._kern[i], str(self._kern[i])), []).append(a.elapsed_time(b))
        return out


# ---------------------------------------------------------------------------
# conveniences: descriptor + output/workspace allocation with torch
# ---------------------------------------------------------------------------

def _workspace(desc: Desc, kind: int, device, nbytes: Optional[int] = None) -> Optional[torch.Tensor]:
    n = dsa3d_workspace_size(desc, kind) if nbytes is None else nbytes
    if n == 0:
        return None
    return torch.empty((n + 15) // 16 * 16, dtype=torch.uint8, device=device)


def forward(q, k, v, offsets, window, dilation=(1, 1, 1), scale: float = 0.0, stream=None):
    """Returns (out, lse); offsets None is the fixed window (every offset zero)."""
    desc = desc_like(q, window, dilation, scale)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:5], dtype=torch.float32, device=q.device)
    dsa3d_forward(desc, q, k, v, offsets, out, lse, stream)
    return out, lse


def backward(q, k, v, offsets, out, lse, dout, window, dilation=(1, 1, 1), scale: float = 0.0,
             deterministic: bool = False, workspace: Optional[torch.Tensor] = None, stream=None):
    """Returns (dq, dk, dv, doffsets); offsets None is the fixed window (doffsets None)."""
    desc = desc_like(q, window, dilation, scale, deterministic)
    if workspace is None:
        workspace = _workspace(desc, WS_BACKWARD if offsets is not None else WS_BACKWARD_FIXED, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    doff = torch.empty_like(offsets) if offsets is not None else None
    dsa3d_backward(desc, q, k, v, offsets, out, lse, dout, dq, dk, dv, doff, workspace, stream)
    return dq, dk, dv, doff


def offset_proj(q, w, bias, window, stream=None):
    """offsets [B,T,H,W,heads,P,3] = Linear(q's C-wide row) with weight w [heads*P*3, C]."""
    B, T, H, W, nh, d = q.shape
    desc = desc_like(q, window)
    P = desc.P
    off = torch.empty((B, T, H, W, nh, P, 3), dtype=q.dtype, device=q.device)
    dsa3d_offset_proj_forward(desc, q, w, bias, off, stream)
    return off


def dwconv(q, wt, bias, stream=None):
    """Depthwise 3x3x3 convolution of q [B,T,H,W,heads,d] (channels = heads*d) with wt [C,3,3,3]."""
    desc = desc_like(q, (1, 1, 1))
    y = torch.empty_like(q)
    dsa3d_dwconv_forward(desc, q, wt, bias, y, stream)
    return y


def dwconv_backward(q, wt, dy, dq_accum, with_bias: bool = True, stream=None):
    """Adds the convolution's input gradient into dq_accum; returns (dwt, dbias) in float32."""
    desc = desc_like(q, (1, 1, 1))
    dwt = torch.empty(wt.shape, dtype=torch.float32, device=q.device)
    db = torch.empty(wt.shape[0], dtype=torch.float32, device=q.device) if with_bias else None
    ws = _workspace(desc, WS_DWCONV_BACKWARD, q.device)
    dsa3d_dwconv_backward(desc, q, wt, dy, dq_accum, dwt, db, ws, stream)
    return dwt, db


def offset_proj_backward(q, w, doffsets, dq_accum, window, with_bias: bool = True, stream=None):
    """Adds doff.W into dq_accum; returns (dW, db) in float32."""
    desc = desc_like(q, window)
    dw = torch.empty(w.shape, dtype=torch.float32, device=q.device)
    db = torch.empty(w.shape[0], dtype=torch.float32, device=q.device) if with_bias else None
    ws = _workspace(desc, WS_PROJ_BACKWARD, q.device)
    dsa3d_offset_proj_backward(desc, q, w, doffsets, dq_accum, dw, db, ws, stream)
    return dw, db
