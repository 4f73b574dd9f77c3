"""One pass of the 3D-DSA hot path over a workload's inputs, on one GPU.

The chain is: [depthwise convolution of q ->] offset projection (when the
workload computes its offsets) -> fused forward -> backward (when the workload
has one) -> projection backward [-> convolution backward].
Every output and workspace is allocated once, up front, so that `run()` only
enqueues kernels on the stream.
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import (WS_BACKWARD, WS_BACKWARD_FIXED, WS_DWCONV_BACKWARD, WS_PROJ_BACKWARD, desc_like, dsa3d_backward,
               dsa3d_backward_hybrid, dsa3d_dwconv_backward, dsa3d_dwconv_forward, dsa3d_forward,
               dsa3d_forward_hybrid, dsa3d_hybrid_workspace_size, dsa3d_offset_proj_backward,
               dsa3d_offset_proj_forward, dsa3d_workspace_size)
from .synth import Workload


class Chain:
    def __init__(self, wl: Workload, inputs: Dict[str, torch.Tensor], bwd_workspace_bytes: Optional[int] = None,
                 deterministic: Optional[bool] = None):
        self.wl = wl
        self.x = inputs
        q = inputs["q"]
        dev = q.device
        det = wl.deterministic if deterministic is None else deterministic
        self.desc = desc_like(q, wl.window, wl.dilation, 0.0, det)
        self.conv = wl.offsets == "conv"
        self.proj = wl.offsets in ("proj", "conv")
        # the projection's input: q itself, or its depthwise convolution
        self.pin = torch.empty_like(q) if self.conv else q
        self.fixed = wl.offsets == "none"  # fixed window: no offsets tensor
        if self.proj:
            self.offsets = torch.empty(q.shape[:5] + (wl.P, 3), dtype=q.dtype, device=dev)
        else:
            self.offsets = None if self.fixed else inputs["offsets"]
        self.out = torch.empty_like(q)
        self.lse = torch.empty(q.shape[:5], dtype=torch.float32, device=dev)
        self.backward = wl.backward
        if self.backward:
            self.dq = torch.empty_like(q)
            self.dk = torch.empty_like(q)
            self.dv = torch.empty_like(q)
            self.doff = None if self.fixed else torch.empty_like(self.offsets)
            kind = WS_BACKWARD_FIXED if self.fixed else WS_BACKWARD
            self.G = wl.global_tokens
            if self.G:
                self.dgk, self.dgv = torch.empty_like(inputs["gk"]), torch.empty_like(inputs["gv"])
            if bwd_workspace_bytes is not None:
                n = bwd_workspace_bytes
            elif self.G:
                n = dsa3d_hybrid_workspace_size(self.desc, self.G, kind)
            else:
                n = dsa3d_workspace_size(self.desc, kind)
            self.ws = torch.empty(max(16, (n + 15) // 16 * 16), dtype=torch.uint8, device=dev) if n else None
            if self.proj:
                self.dw = torch.empty(inputs["proj_w"].shape, dtype=torch.float32, device=dev)
                self.db = torch.empty(inputs["proj_w"].shape[0], dtype=torch.float32, device=dev)
                m = dsa3d_workspace_size(self.desc, WS_PROJ_BACKWARD)
                self.pws = torch.empty((m + 15) // 16 * 16, dtype=torch.uint8, device=dev)
            if self.conv:
                self.dpin = torch.empty_like(q)  # gradient at the convolution's output
                self.dcw = torch.empty(inputs["conv_w"].shape, dtype=torch.float32, device=dev)
                self.dcb = torch.empty(inputs["conv_w"].shape[0], dtype=torch.float32, device=dev)
                m = dsa3d_workspace_size(self.desc, WS_DWCONV_BACKWARD)
                self.cws = torch.empty((m + 15) // 16 * 16, dtype=torch.uint8, device=dev)

    def run(self, stream=None):
        x = self.x
        if self.conv:
            dsa3d_dwconv_forward(self.desc, x["q"], x["conv_w"], x["conv_b"], self.pin, stream)
        if self.proj:
            dsa3d_offset_proj_forward(self.desc, self.pin, x["proj_w"], x["proj_b"], self.offsets, stream)
        G = self.wl.global_tokens
        if G:
            dsa3d_forward_hybrid(self.desc, x["q"], x["k"], x["v"], self.offsets, G, x["gk"], x["gv"], self.out,
                                 self.lse, stream)
        else:
            dsa3d_forward(self.desc, x["q"], x["k"], x["v"], self.offsets, self.out, self.lse, stream)
        if not self.backward:
            return
        if G:
            dsa3d_backward_hybrid(self.desc, x["q"], x["k"], x["v"], self.offsets, self.out, self.lse, x["dout"], G,
                                  x["gk"], x["gv"], self.dq, self.dk, self.dv, self.doff, self.dgk, self.dgv,
                                  self.ws, stream)
        else:
            dsa3d_backward(self.desc, x["q"], x["k"], x["v"], self.offsets, self.out, self.lse, x["dout"],
                           self.dq, self.dk, self.dv, self.doff, self.ws, stream)
        if self.conv:
            # the projection's input gradient starts from zero (a device clear, no arithmetic)
            self.dpin.zero_()
            dsa3d_offset_proj_backward(self.desc, self.pin, x["proj_w"], self.doff, self.dpin, self.dw, self.db,
                                       self.pws, stream)
            dsa3d_dwconv_backward(self.desc, x["q"], x["conv_w"], self.dpin, self.dq, self.dcw, self.dcb,
                                  self.cws, stream)
        elif self.proj:
            dsa3d_offset_proj_backward(self.desc, x["q"], x["proj_w"], self.doff, self.dq, self.dw, self.db,
                                       self.pws, stream)


class BlockChain:
    """One pass of the transformer block around the operator, forward then
    backward, on one GPU (every buffer allocated up front):

        h = LayerNorm(x); q|k|v = h W_qkv^T + b_qkv; offsets = q W_off^T + b_off;
        o = 3D-DSA(q, k, v, offsets); y = x + o W_out^T + b_out

    and the gradients of x and every parameter for dL/dy = dout. Each step is
    one libdsa3d call; the residual add is the output projection's epilogue and
    the residual gradient enters the layer norm's backward as dres."""

    def __init__(self, wl: Workload, inputs: Dict[str, torch.Tensor], bwd_workspace_bytes: Optional[int] = None,
                 deterministic: Optional[bool] = None):
        from . import (dsa3d_layernorm_workspace_size, dsa3d_linear_workspace_size, dtype_code, make_desc)
        assert wl.block and wl.offsets == "proj"
        self.wl = wl
        self.x = inputs
        x = inputs["x"]
        dev = x.device
        det = wl.deterministic if deterministic is None else deterministic
        B, T, H, W, C = x.shape
        self.M, self.C, self.F = B * T * H * W, C, wl.F
        self.code = dtype_code(x.dtype)
        self.desc = make_desc(B, T, H, W, wl.heads, wl.head_dim, wl.window, wl.dilation, x.dtype, 0.0, det)
        act = (B, T, H, W, wl.heads, wl.head_dim)
        e = lambda shape=act, dt=x.dtype: torch.empty(shape, dtype=dt, device=dev)
        self.h = e(x.shape)
        self.stats = e((self.M, 2), torch.float32)
        self.q, self.k, self.v = e(), e(), e()
        self.offsets = e(act[:5] + (wl.P, 3))
        self.out = e()
        self.lse = e(act[:5], torch.float32)
        self.y = e(x.shape)
        self.backward = wl.backward
        if self.backward:
            self.do = e()
            self.dq, self.dk, self.dv = e(), e(), e()
            self.doff = e(self.offsets.shape)
            self.dh = e(x.shape)
            self.dx = e(x.shape)
            f32 = torch.float32
            self.dln_g, self.dln_b = e((C,), f32), e((C,), f32)
            self.dw_qkv, self.db_qkv = e((3 * C, C), f32), e((3 * C,), f32)
            self.dw_off, self.db_off = e((self.F, C), f32), e((self.F,), f32)
            self.dw_out, self.db_out = e((C, C), f32), e((C,), f32)
            n = dsa3d_workspace_size(self.desc, WS_BACKWARD) if bwd_workspace_bytes is None else bwd_workspace_bytes
            self.ws = torch.empty(max(16, (n + 15) // 16 * 16), dtype=torch.uint8, device=dev)
            m = max(dsa3d_workspace_size(self.desc, WS_PROJ_BACKWARD),
                    dsa3d_linear_workspace_size(self.code, self.M, C, C),
                    dsa3d_layernorm_workspace_size(self.M, C))
            self.lws = torch.empty((m + 15) // 16 * 16, dtype=torch.uint8, device=dev)

    def forward(self, stream=None):
        from . import dsa3d_layernorm_forward, dsa3d_linear_forward
        x, wl, M, C, code = self.x, self.wl, self.M, self.C, self.code
        dsa3d_layernorm_forward(code, M, C, wl.ln_eps, x["x"], x["ln_g"], x["ln_b"], self.h, self.stats, stream)
        for i, t in enumerate((self.q, self.k, self.v)):
            dsa3d_linear_forward(code, M, C, C, self.h, x["w_qkv"][i * C:(i + 1) * C], x["b_qkv"][i * C:(i + 1) * C],
                                 None, t, stream)
        dsa3d_offset_proj_forward(self.desc, self.q, x["proj_w"], x["proj_b"], self.offsets, stream)
        dsa3d_forward(self.desc, self.q, self.k, self.v, self.offsets, self.out, self.lse, stream)
        dsa3d_linear_forward(code, M, C, C, self.out, x["w_out"], x["b_out"], x["x"], self.y, stream)

    def backward_pass(self, stream=None):
        from . import dsa3d_layernorm_backward, dsa3d_linear_backward
        x, M, C, code = self.x, self.M, self.C, self.code
        dsa3d_linear_backward(code, M, C, C, self.out, x["w_out"], x["dout"], None, self.do, self.dw_out,
                              self.db_out, self.lws, stream)
        dsa3d_backward(self.desc, self.q, self.k, self.v, self.offsets, self.out, self.lse, self.do, self.dq,
                       self.dk, self.dv, self.doff, self.ws, stream)
        dsa3d_offset_proj_backward(self.desc, self.q, x["proj_w"], self.doff, self.dq, self.dw_off, self.db_off,
                                   self.lws, stream)
        for i, g in enumerate((self.dq, self.dk, self.dv)):
            dsa3d_linear_backward(code, M, C, C, self.h, x["w_qkv"][i * C:(i + 1) * C], g, None if i == 0 else self.dh,
                                  self.dh, self.dw_qkv[i * C:(i + 1) * C], self.db_qkv[i * C:(i + 1) * C], self.lws,
                                  stream)
        dsa3d_layernorm_backward(code, M, C, x["x"], x["ln_g"], self.stats, self.dh, x["dout"], self.dx, self.dln_g,
                                 self.dln_b, self.lws, stream)

    def run(self, stream=None):
        self.forward(stream)
        if self.backward:
            self.backward_pass(stream)


def make_chain(wl: Workload, inputs: Dict[str, torch.Tensor], **kw):
    """The chain of a workload: the transformer block or the operator's own chain."""
    return BlockChain(wl, inputs, **kw) if wl.block else Chain(wl, inputs, **kw)
