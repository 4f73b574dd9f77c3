"""Helpers for the GPU parity tests: exact widening to float64 and oracle
evaluation at sampled queries / key tokens of grids too large to run whole.

Everything the oracle consumes here is an input drawn by the seeded generator
(or, for the attention behind a bf16 projection, the offsets tensor the GPU
fed to its own attention -- the projection itself is checked separately).
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np
import torch

import oracle


def to_np(t: torch.Tensor) -> np.ndarray:
    """bf16/f32 tensor -> float64 array (exact widening)."""
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def to_np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy()


def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((x - ref).ravel()))
    return num / den if den > 0 else num


def window_points(window, dilation) -> np.ndarray:
    kt, kh, kw = window
    it, ih, iw = np.meshgrid(np.arange(kt), np.arange(kh), np.arange(kw), indexing="ij")
    return np.stack([dilation[0] * (it.ravel() - (kt - 1) // 2), dilation[1] * (ih.ravel() - (kh - 1) // 2),
                     dilation[2] * (iw.ravel() - (kw - 1) // 2)], 1).astype(np.int64)


def sample_floor(x: Sequence[int], off32: np.ndarray, window, dilation) -> Tuple[np.ndarray, np.ndarray]:
    """floor of the float32 sample positions of one query [P,3] and a mask of
    samples that can touch the grid (finite, |pos| < 2^30)."""
    ref = np.asarray(x, dtype=np.int64)[None, :] + window_points(window, dilation)
    with np.errstate(invalid="ignore", over="ignore"):
        pos = ref.astype(np.float32) + off32.astype(np.float32)
        ok = np.all(np.isfinite(pos) & (np.abs(pos) < 2.0 ** 30), axis=1)
        fl = np.where(ok[:, None], np.floor(np.where(np.isfinite(pos), pos, 0)), 0).astype(np.int64)
    return fl, ok


def corner_box(fls: List[np.ndarray], oks: List[np.ndarray], grid, extra: Sequence[Sequence[int]] = ()):
    """Smallest box (origin, shape) inside the grid holding every in-grid corner."""
    lo = np.array([10 ** 12] * 3)
    hi = np.array([-1] * 3)
    for fl, ok in zip(fls, oks):
        if not ok.any():
            continue
        f = fl[ok]
        lo = np.minimum(lo, f.min(0))
        hi = np.maximum(hi, f.max(0) + 1)
    for e in extra:
        lo = np.minimum(lo, e)
        hi = np.maximum(hi, e)
    size = np.array(grid)
    lo = np.clip(lo, 0, size - 1)
    hi = np.clip(hi, 0, size - 1)
    hi = np.maximum(hi, lo)
    return tuple(int(v) for v in lo), tuple(int(v) for v in (hi - lo + 1))


def oracle_queries(wl, x: Dict[str, torch.Tensor], offsets: torch.Tensor, queries, dout=None, scale=None):
    """Oracle forward (and backward if dout is given) of listed queries
    (b, t, h, w, head) of a grid held on the GPU. Returns dict of arrays
    o [n,d], lse [n] (and dq [n,d], doff [n,P,3])."""
    grid = (wl.T, wl.H, wl.W)
    d = wl.head_dim
    scale = oracle.default_scale(d) if scale is None else scale
    res = {"o": [], "lse": [], "dq": [], "doff": []}
    for (b, t, h, w, e) in queries:
        off32 = to_np32(offsets[b, t, h, w, e])
        fl, ok = sample_floor((t, h, w), off32, wl.window, wl.dilation)
        org, shp = corner_box([fl], [ok], grid, extra=[(t, h, w)])
        sl = (b, slice(org[0], org[0] + shp[0]), slice(org[1], org[1] + shp[1]), slice(org[2], org[2] + shp[2]), e)
        K = to_np(x["k"][sl])
        V = to_np(x["v"][sl])
        qrow = to_np(x["q"][b, t, h, w, e])[None]
        qpos = np.array([[t, h, w]])
        o, lse = oracle.forward_queries(grid, wl.window, wl.dilation, scale, qpos, qrow, off32[None], org, K, V)
        res["o"].append(o[0]); res["lse"].append(lse[0])
        if dout is not None:
            g = to_np(dout[b, t, h, w, e])[None]
            dq, doff, _, _ = oracle.backward_queries(grid, wl.window, wl.dilation, scale, qpos, qrow, off32[None],
                                                     org, K, V, g)
            res["dq"].append(dq[0]); res["doff"].append(doff[0])
    return {k: np.array(v) for k, v in res.items() if v}


def max_finite_abs(t: torch.Tensor) -> float:
    a = t.detach().abs().to(torch.float32)
    a = torch.where(torch.isfinite(a) & (a < 2.0 ** 30), a, torch.zeros_like(a))
    return float(a.max().item())


def oracle_dkdv_at_keys(wl, x: Dict[str, torch.Tensor], offsets: torch.Tensor, dout: torch.Tensor, keys,
                        scale=None):
    """Oracle dK and dV rows at listed key tokens (b, t, h, w, head): every
    query whose samples can reach the key is found, its backward is run by the
    oracle, and the key's rows of the accumulated dK/dV are returned."""
    grid = (wl.T, wl.H, wl.W)
    d = wl.head_dim
    scale = oracle.default_scale(d) if scale is None else scale
    rad = np.array([(wl.window[a] - 1) // 2 * wl.dilation[a] for a in range(3)])
    out_k, out_v = [], []
    for (b, tj, hj, wj, e) in keys:
        m = [max_finite_abs(offsets[b, ..., e, :, a]) for a in range(3)]
        R = rad + np.ceil(np.array(m)).astype(np.int64) + 2
        lo = np.maximum(0, np.array([tj, hj, wj]) - R)
        hi = np.minimum(np.array(grid) - 1, np.array([tj, hj, wj]) + R)
        sl = (b, slice(lo[0], hi[0] + 1), slice(lo[1], hi[1] + 1), slice(lo[2], hi[2] + 1), e)
        off_c = to_np32(offsets[sl])                     # [bt,bh,bw,P,3]
        cand = oracle.grid_positions(*(hi - lo + 1)) + lo
        chosen, fls, oks = [], [], []
        for i, (t, h, w) in enumerate(cand):
            fl, ok = sample_floor((t, h, w), off_c[t - lo[0], h - lo[1], w - lo[2]], wl.window, wl.dilation)
            hit = ok & np.all((fl == [tj, hj, wj]) | (fl + 1 == [tj, hj, wj]), axis=1)
            if hit.any():
                chosen.append(i); fls.append(fl); oks.append(ok)
        qpos = cand[chosen]
        org, shp = corner_box(fls, oks, grid, extra=[(tj, hj, wj)])
        bsl = (b, slice(org[0], org[0] + shp[0]), slice(org[1], org[1] + shp[1]), slice(org[2], org[2] + shp[2]), e)
        K, V = to_np(x["k"][bsl]), to_np(x["v"][bsl])
        loc = qpos - lo
        qsub = to_np(x["q"][sl])[loc[:, 0], loc[:, 1], loc[:, 2]]
        gsub = to_np(dout[sl])[loc[:, 0], loc[:, 1], loc[:, 2]]
        osub = off_c[loc[:, 0], loc[:, 1], loc[:, 2]]
        if len(qpos):
            _, _, dK, dV = oracle.backward_queries(grid, wl.window, wl.dilation, scale, qpos, qsub, osub, org, K, V,
                                                   gsub)
            jj = (tj - org[0], hj - org[1], wj - org[2])
            out_k.append(dK[jj]); out_v.append(dV[jj])
        else:
            out_k.append(np.zeros(d)); out_v.append(np.zeros(d))
    return np.array(out_k), np.array(out_v)


def sample_queries(wl, heads, n_random, seed=0, faces=16):
    """Random queries plus the 8 grid corners and random points on the six faces."""
    rng = np.random.default_rng(seed)
    T, H, W = wl.T, wl.H, wl.W
    qs = []
    for e in heads:
        for b in range(wl.B):
            for t in (0, T - 1):
                for h in (0, H - 1):
                    for w in (0, W - 1):
                        qs.append((b, t, h, w, e))
            for _ in range(faces):
                ax = rng.integers(0, 3)
                p = [int(rng.integers(0, T)), int(rng.integers(0, H)), int(rng.integers(0, W))]
                p[ax] = 0 if rng.integers(0, 2) == 0 else (T, H, W)[ax] - 1
                qs.append((b, p[0], p[1], p[2], e))
        for _ in range(n_random):
            qs.append((int(rng.integers(0, wl.B)), int(rng.integers(0, T)), int(rng.integers(0, H)),
                       int(rng.integers(0, W)), e))
    return qs


def gather(t: torch.Tensor, idx) -> np.ndarray:
    """Rows t[b,t,h,w,head] of the listed indices, widened to float64."""
    ii = torch.tensor(idx, dtype=torch.long)
    return to_np(t[ii[:, 0], ii[:, 1], ii[:, 2], ii[:, 3], ii[:, 4]])
