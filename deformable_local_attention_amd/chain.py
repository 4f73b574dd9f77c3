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
               dsa3d_dwconv_backward, dsa3d_dwconv_forward, dsa3d_forward, dsa3d_offset_proj_backward,
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
            n = dsa3d_workspace_size(self.desc, kind) if bwd_workspace_bytes is None else bwd_workspace_bytes
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
        dsa3d_forward(self.desc, x["q"], x["k"], x["v"], self.offsets, self.out, self.lse, stream)
        if self.backward:
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
