"""Seeded synthetic inputs for 3D Deformable Slide Attention (3D-DSA).

This module is shared by the tests, the benchmark and the oracle's callers. It
holds workload shapes, value distributions and a fixed draw order, and none of
the operator's arithmetic.

The pages measure on video latents (WebVid-2.5M) and VBench prompts
[MegaSlide-DiT, §6.1 Hardware and data]. Those do not change the operator's
cost, so i.i.d. Gaussian tensors at the pages' token-grid shapes stand in for
them: 1080p video at 16x16 patches gives a 67.5 x 120 patch grid per frame
[MegaSlide-DiT, §3.2 Activation memory and attention complexity], padded here
to 68 rows; 720p gives 45 x 80.

Draw order (one generator, seed 0 unless stated): q, k, v (float32 N(0,1),
then rounded to the run dtype), projection weight W (N(0, 0.02)), bias (zeros),
direct offsets (N(0, sigma)), upstream gradient dO (N(0,1)). Block workloads
draw the block's input and parameters instead (see make_inputs).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic 3D-DSA workload: token grid, heads, window and inputs."""

    name: str
    B: int
    T: int
    H: int
    W: int
    heads: int
    head_dim: int
    window: Tuple[int, int, int]          # (k_t, k_h, k_w)
    dilation: Tuple[int, int, int]        # (dil_t, dil_h, dil_w)
    dtype: str                            # "f32" or "bf16"
    offsets: str                          # "direct", "proj" (Linear of q), "conv" (Linear of dwconv(q))
                                          # or "none" (fixed window: every offset zero, none stored)
    offset_sigma: float = 0.0             # std of direct offsets (token units)
    weight_sigma: float = 0.02            # std of projection weights
    backward: bool = False                # chain includes the backward pass
    deterministic: bool = False           # K/V-gradient accumulation mode
    block: bool = False                   # the whole transformer block around the operator (layer norm,
                                          # q/k/v projections, offset projection, attention, output
                                          # projection with the residual add); offsets must be "proj"
    ln_eps: float = 1e-6                  # the block's layer-normalisation epsilon
    global_tokens: int = 0                # hybrid attention: G global key/value rows per (batch, head)
    description: str = ""

    @property
    def P(self) -> int:
        return self.window[0] * self.window[1] * self.window[2]

    @property
    def tokens(self) -> int:
        return self.B * self.T * self.H * self.W

    @property
    def C(self) -> int:
        return self.heads * self.head_dim

    @property
    def F(self) -> int:
        """Width of the offset projection's output: heads * P * 3."""
        return self.heads * self.P * 3

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_grid(self, B=None, T=None, H=None, W=None, heads=None, name=None) -> "Workload":
        """Same workload on another grid (used for bounded samples and crops)."""
        return dataclasses.replace(
            self, B=B or self.B, T=T or self.T, H=H or self.H, W=W or self.W,
            heads=heads or self.heads, name=name or self.name)


# The five workloads: a tiny fp32 correctness case, a small bf16 case with a
# projection, a 720p fwd+bwd case with spatial dilation 2, and two 1080p cases
# (2,088,960 tokens, 24 heads x 128).
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny-f32", 1, 4, 8, 8, 2, 32, (3, 3, 3), (1, 1, 1), "f32", "direct",
                 offset_sigma=0.5, backward=True,
                 description="fp32 fwd+bwd, 4x8x8 tokens, 2x32 heads, 3x3x3 window"),
        Workload("small-bf16-proj", 1, 16, 32, 32, 8, 64, (3, 3, 3), (1, 1, 1), "bf16", "proj",
                 description="bf16 projection + fwd, 16x32x32 tokens, 8x64 heads"),
        Workload("720p-bf16-proj-dil2", 1, 64, 45, 80, 16, 64, (3, 3, 3), (1, 2, 2), "bf16", "proj",
                 backward=True,
                 description="bf16 projection + fwd + bwd, 64x45x80 tokens, 16x64 heads, dilation (1,2,2)"),
        Workload("720p-bf16-conv-dil2", 1, 64, 45, 80, 16, 64, (3, 3, 3), (1, 2, 2), "bf16", "conv",
                 backward=True,
                 description="bf16 depthwise 3x3x3 conv + projection + fwd + bwd, 64x45x80 tokens, 16x64 heads, "
                             "dilation (1,2,2)"),
        Workload("1080p-bf16-proj", 1, 256, 68, 120, 24, 128, (3, 3, 3), (1, 1, 1), "bf16", "proj",
                 description="bf16 projection + fwd, 256x68x120 tokens, 24x128 heads"),
        Workload("1080p-bf16-fixed377", 1, 256, 68, 120, 24, 128, (3, 7, 7), (1, 1, 1), "bf16", "none",
                 backward=True,
                 description="bf16 fwd + bwd of the fixed 3x7x7 window (every offset zero), 256x68x120 tokens, "
                             "24x128 heads"),
        Workload("1080p-bf16-p75-det", 1, 256, 68, 120, 24, 128, (3, 5, 5), (1, 1, 1), "bf16", "direct",
                 offset_sigma=2.0, backward=True, deterministic=True,
                 description="bf16 fwd + bwd, 256x68x120 tokens, 24x128 heads, 3x5x5 window, "
                             "offsets N(0,2), deterministic K/V gradients"),
        Workload("1080p-bf16-p75-hybrid64", 1, 256, 68, 120, 24, 128, (3, 5, 5), (1, 1, 1), "bf16", "direct",
                 offset_sigma=2.0, backward=True, deterministic=True, global_tokens=64,
                 description="bf16 hybrid attention fwd + bwd: the 3x5x5 deformable samples plus 64 global tokens per "
                             "head in one softmax, 256x68x120 tokens, 24x128 heads, deterministic"),
        Workload("720p-bf16-block", 1, 64, 45, 80, 16, 64, (3, 3, 3), (1, 2, 2), "bf16", "proj",
                 backward=True, block=True,
                 description="bf16 transformer block fwd + bwd: layer norm, q/k/v projections, offset projection, "
                             "3D-DSA, output projection + residual; 64x45x80 tokens, 16x64 heads, dilation (1,2,2)"),
        Workload("1080p-bf16-block", 1, 256, 68, 120, 24, 128, (3, 3, 3), (1, 1, 1), "bf16", "proj",
                 backward=True, block=True,
                 description="bf16 transformer block fwd + bwd around 3D-DSA, 256x68x120 tokens, 24x128 heads"),
    ]
}

# Depthwise-convolution weights of the "conv" offset network: N(0, 0.2^2), so
# that the 27-tap sums keep the scale of q (0.2 * sqrt(27) ~ 1).
CONV_SIGMA = 0.2

# The headline workload: fwd+bwd on the 256x68x120 grid.
HEADLINE = "1080p-bf16-p75-det"

_CHUNK = 1 << 26  # elements drawn per generator call for large tensors


def _randn(shape, std: float, dtype: torch.dtype, gen: torch.Generator, device) -> torch.Tensor:
    """N(0, std^2) drawn in float32 in fixed-size chunks, then rounded to dtype."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x = torch.randn(e - s, generator=gen, dtype=torch.float32, device=device)
        if std != 1.0:
            x.mul_(std)
        flat[s:e].copy_(x)
    return out


def make_inputs(wl: Workload, device="cpu", seed: int = 0,
                with_grad: Optional[bool] = None) -> Dict[str, torch.Tensor]:
    """Draw the inputs of workload `wl` on `device` in the fixed order.

    Returns q, k, v [B,T,H,W,heads,d]; for direct offsets `offsets`
    [B,T,H,W,heads,P,3]; for projected offsets `proj_w` [heads*P*3, C] and
    `proj_b` [heads*P*3]; and `dout` when the chain has a backward pass. A
    block workload instead returns the block's input x [B,T,H,W,C], its
    parameters (ln_g, ln_b, w_qkv, b_qkv, proj_w, proj_b, w_out, b_out) and
    `dout` [B,T,H,W,C], the gradient of the block's output.
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    dt = wl.torch_dtype
    shp = (wl.B, wl.T, wl.H, wl.W, wl.heads, wl.head_dim)
    out = {}
    if wl.block:
        # the block's input and parameters: x ~ N(0,1); layer-norm gain 1 + N(0, 0.1^2), shift N(0, 0.1^2);
        # q/k/v and output projections N(0, 1/C) (so q, k, v and the output keep unit scale), their
        # biases N(0, 0.1^2); the offset projection N(0, weight_sigma^2) with zero bias; dO of y ~ N(0,1)
        C, F = wl.C, wl.F
        xs = (wl.B, wl.T, wl.H, wl.W, C)
        out["x"] = _randn(xs, 1.0, dt, gen, dev)
        out["ln_g"] = _randn((C,), 0.1, torch.float32, gen, dev).add_(1.0).to(dt)
        out["ln_b"] = _randn((C,), 0.1, dt, gen, dev)
        out["w_qkv"] = _randn((3 * C, C), C ** -0.5, dt, gen, dev)
        out["b_qkv"] = _randn((3 * C,), 0.1, dt, gen, dev)
        out["proj_w"] = _randn((F, C), wl.weight_sigma, dt, gen, dev)
        out["proj_b"] = torch.zeros(F, dtype=dt, device=dev)
        out["w_out"] = _randn((C, C), C ** -0.5, dt, gen, dev)
        out["b_out"] = _randn((C,), 0.1, dt, gen, dev)
        if with_grad if with_grad is not None else wl.backward:
            out["dout"] = _randn(xs, 1.0, dt, gen, dev)
        return out
    out["q"] = _randn(shp, 1.0, dt, gen, dev)
    out["k"] = _randn(shp, 1.0, dt, gen, dev)
    out["v"] = _randn(shp, 1.0, dt, gen, dev)
    if wl.offsets == "conv":
        out["conv_w"] = _randn((wl.C, 3, 3, 3), CONV_SIGMA, dt, gen, dev)
        out["conv_b"] = torch.zeros(wl.C, dtype=dt, device=dev)
    if wl.offsets in ("proj", "conv"):
        out["proj_w"] = _randn((wl.F, wl.C), wl.weight_sigma, dt, gen, dev)
        out["proj_b"] = torch.zeros(wl.F, dtype=dt, device=dev)
    elif wl.offsets == "direct":
        out["offsets"] = _randn(shp[:5] + (wl.P, 3), wl.offset_sigma, dt, gen, dev)
    if with_grad if with_grad is not None else wl.backward:
        out["dout"] = _randn(shp, 1.0, dt, gen, dev)
    if wl.global_tokens:
        # hybrid attention's global key and value rows, N(0,1), [B, G, heads, d]
        gs = (wl.B, wl.global_tokens, wl.heads, wl.head_dim)
        out["gk"] = _randn(gs, 1.0, dt, gen, dev)
        out["gv"] = _randn(gs, 1.0, dt, gen, dev)
    return out


def checksum(t: torch.Tensor) -> str:
    """A short fingerprint of a tensor's bytes (records which inputs were drawn).

    Hashes at most 2^20 evenly strided elements so that it stays cheap on
    multi-gigabyte tensors.
    """
    x = t.detach().reshape(-1)
    n = x.numel()
    step = max(1, n // (1 << 20))
    x = x[::step]
    if x.dtype == torch.bfloat16:
        x = x.view(torch.int16).to(torch.int64) & 0xFFFF
    elif x.dtype == torch.float32:
        x = x.view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    idx = torch.arange(x.numel(), device=x.device, dtype=torch.int64)
    h = int(((x * ((idx % 65521) + 1)) % 1000000007).sum().item())
    return f"{n}:{h:x}"


def describe(wl: Workload) -> str:
    return (f"{wl.name}: B={wl.B} T={wl.T} H={wl.H} W={wl.W} heads={wl.heads} d={wl.head_dim} "
            f"window={wl.window} dil={wl.dilation} P={wl.P} {wl.dtype} offsets={wl.offsets}"
            + (f" sigma={wl.offset_sigma}" if wl.offsets == "direct" else "")
            + (" +bwd" if wl.backward else "") + (" det" if wl.deterministic else "") + (" block" if wl.block else "")
            + (f" G={wl.global_tokens}" if wl.global_tokens else ""))

