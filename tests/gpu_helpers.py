"""Helpers for the GPU parity tests: exact widening to float64 and oracle
evaluation at sampled queries / key tokens of grids too large to run whole.

Everything the oracle consumes here is an input drawn by the seeded generator
(or, for the attention behind a bf16 projection, the offsets tensor the GPU
fed to its own attention -- the projection itself is checked separately).
"""
from __future__ import annotations

import math
import os
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


# ---------------------------------------------------------------------------
# Full-size parity: one (batch item, head) of the device tensors at a time
# ---------------------------------------------------------------------------

def head_slab(t: torch.Tensor, b: int, e: int, dtype=np.float32) -> np.ndarray:
    """t[b, :, :, :, e] (a [B,T,H,W,heads,...] tensor) as a host array,
    widened exactly (bf16 and f32 values are exact in float32)."""
    return t[b, :, :, :, e].to(torch.float32).cpu().numpy().astype(dtype, copy=False)


def face_tokens(T: int, H: int, W: int) -> np.ndarray:
    """Every token on the six faces of a T x H x W grid, [n,3] (t,h,w)."""
    pos = oracle.grid_positions(T, H, W)
    on = ((pos[:, 0] == 0) | (pos[:, 0] == T - 1) | (pos[:, 1] == 0) | (pos[:, 1] == H - 1) |
          (pos[:, 2] == 0) | (pos[:, 2] == W - 1))
    return pos[on]


def random_tokens(T: int, H: int, W: int, n: int, rng) -> np.ndarray:
    """n distinct random tokens of the grid, [n,3]."""
    flat = rng.choice(T * H * W, size=min(n, T * H * W), replace=False)
    return np.stack([flat // (H * W), (flat // W) % H, flat % W], 1).astype(np.int32)


def interior_tokens(T: int, H: int, W: int, n: int, rng, margin: int = 1) -> np.ndarray:
    """n random tokens at least `margin` tokens away from every face (fewer
    if the grid has no interior)."""
    lo = np.array([min(margin, (X - 1) // 2) for X in (T, H, W)])
    hi = np.array([T, H, W]) - lo
    out = np.stack([rng.integers(lo[a], hi[a], size=n) for a in range(3)], 1).astype(np.int32)
    return np.unique(out, axis=0)


def grid_corner_tokens(T: int, H: int, W: int) -> np.ndarray:
    return np.unique(np.array([(t, h, w) for t in (0, T - 1) for h in (0, H - 1) for w in (0, W - 1)],
                              dtype=np.int32), axis=0)


class HeadOracle:
    """The oracle on one (batch item, head) of a full-size problem held on the
    device: the head's key and value rows are copied to the host once (the
    oracle's box is then the whole grid), and queries are evaluated in bulk.

    offsets: a [B,T,H,W,heads,P,3] device tensor, or None for the fixed window
    (every offset zero)."""

    def __init__(self, wl, x: Dict[str, torch.Tensor], b: int, e: int, offsets=None, dout=None, threads=None,
                 global_rows=None):
        """global_rows: (gk, gv) device tensors [B, G, heads, d] of hybrid
        attention (their rows join each query's softmax), or None."""
        self.wl, self.b, self.e = wl, b, e
        self.GK = self.GV = None
        if global_rows is not None:
            self.GK = global_rows[0][b, :, e].to(torch.float32).cpu().numpy().astype(np.float64)
            self.GV = global_rows[1][b, :, e].to(torch.float32).cpu().numpy().astype(np.float64)
        self.grid = (wl.T, wl.H, wl.W)
        self.scale = oracle.default_scale(wl.head_dim)
        self.threads = threads or min(16, os.cpu_count() or 1)
        self.K = head_slab(x["k"], b, e, np.float64)
        self.V = head_slab(x["v"], b, e, np.float64)
        self.q = head_slab(x["q"], b, e)
        self.g = None if dout is None else head_slab(dout, b, e)
        self.off = None if offsets is None else head_slab(offsets, b, e)

    def _rows(self, a, pos):
        return a[pos[:, 0], pos[:, 1], pos[:, 2]]

    def offsets_at(self, pos) -> np.ndarray:
        if self.off is None:
            return np.zeros((len(pos), self.wl.P, 3), dtype=np.float32)
        return self._rows(self.off, pos)

    def forward(self, pos):
        wl = self.wl
        if self.GK is not None:
            return oracle.forward_hybrid_queries(self.grid, wl.window, wl.dilation, self.scale, pos,
                                                 self._rows(self.q, pos), self.offsets_at(pos), (0, 0, 0), self.K,
                                                 self.V, self.GK, self.GV, threads=self.threads)
        return oracle.forward_queries(self.grid, wl.window, wl.dilation, self.scale, pos, self._rows(self.q, pos),
                                      self.offsets_at(pos), (0, 0, 0), self.K, self.V, threads=self.threads)

    def global_grads(self):
        """dGK, dGV [G,d] of the hybrid attention: every query of the head."""
        wl = self.wl
        pos = oracle.grid_positions(*self.grid)
        _, _, dgk, dgv, _, _ = oracle.backward_hybrid_queries(
            self.grid, wl.window, wl.dilation, self.scale, pos, self.q.reshape(-1, wl.head_dim),
            self.offsets_at(pos), (0, 0, 0), self.K, self.V, self.GK, self.GV, self.g.reshape(-1, wl.head_dim),
            threads=self.threads)
        return dgk, dgv

    def backward_queries(self, pos):
        """dq [n,d] and doffsets [n,P,3] of the listed queries."""
        wl = self.wl
        if self.GK is not None:
            dq, doff, _, _, _, _ = oracle.backward_hybrid_queries(
                self.grid, wl.window, wl.dilation, self.scale, pos, self._rows(self.q, pos), self.offsets_at(pos),
                (0, 0, 0), self.K, self.V, self.GK, self.GV, self._rows(self.g, pos), threads=self.threads)
            return dq, doff
        dq, doff, _, _ = oracle.backward_queries(self.grid, wl.window, wl.dilation, self.scale, pos,
                                                 self._rows(self.q, pos), self.offsets_at(pos), (0, 0, 0), self.K,
                                                 self.V, self._rows(self.g, pos), want_kv=False,
                                                 threads=self.threads)
        return dq, doff

    def queries_reaching(self, keys) -> np.ndarray:
        """Every query with a sample whose trilinear cell has one of `keys`
        ([n,3]) as a corner (the float32 position arithmetic of the operator,
        vectorised over the candidates around each key)."""
        wl = self.wl
        T, H, W = self.grid
        rad = np.array([(wl.window[a] - 1) // 2 * wl.dilation[a] for a in range(3)])
        if self.off is None:
            m = np.zeros(3)
        else:
            a = np.abs(self.off.reshape(-1, 3))
            a = np.where(np.isfinite(a) & (a < 2.0 ** 30), a, 0.0)
            m = a.max(0)
        R = rad + np.ceil(m).astype(np.int64) + 2
        wp = window_points(wl.window, wl.dilation)
        chosen = np.zeros((T, H, W), dtype=bool)
        for key in np.asarray(keys):
            lo = np.maximum(0, key - R)
            hi = np.minimum(np.array(self.grid) - 1, key + R)
            cand = oracle.grid_positions(*(hi - lo + 1)) + lo
            off = self.offsets_at(cand)
            with np.errstate(invalid="ignore", over="ignore"):
                pos = (cand[:, None, :] + wp[None]).astype(np.float32) + off.astype(np.float32)
                ok = np.all(np.isfinite(pos) & (np.abs(pos) < 2.0 ** 30), axis=2)
                fl = np.floor(np.where(ok[..., None], pos, 0)).astype(np.int64)
            hit = ok & np.all((fl == key) | (fl + 1 == key), axis=2)
            sel = cand[hit.any(1)]
            chosen[sel[:, 0], sel[:, 1], sel[:, 2]] = True
        return np.argwhere(chosen).astype(np.int32)

    def dkdv_at(self, keys):
        """dK and dV rows [n,d] at `keys`: the backward of every query that
        reaches one of them, accumulated over the whole grid."""
        wl = self.wl
        keys = np.asarray(keys)
        qpos = self.queries_reaching(keys)
        if len(qpos) == 0:
            z = np.zeros((len(keys), wl.head_dim))
            return z, z.copy()
        if self.GK is not None:
            _, _, _, _, dK, dV = oracle.backward_hybrid_queries(
                self.grid, wl.window, wl.dilation, self.scale, qpos, self._rows(self.q, qpos), self.offsets_at(qpos),
                (0, 0, 0), self.K, self.V, self.GK, self.GV, self._rows(self.g, qpos), want_kv=True)
        else:
            _, _, dK, dV = oracle.backward_queries(self.grid, wl.window, wl.dilation, self.scale, qpos,
                                                   self._rows(self.q, qpos), self.offsets_at(qpos), (0, 0, 0),
                                                   self.K, self.V, self._rows(self.g, qpos))
        return self._rows(dK, keys), self._rows(dV, keys)


def rows_at(t: torch.Tensor, b: int, e: int, pos) -> np.ndarray:
    """Rows t[b, t, h, w, e] of a device tensor at positions pos [n,3], widened to float64."""
    ii = torch.as_tensor(np.asarray(pos, dtype=np.int64), device=t.device)
    return to_np(t[b][ii[:, 0], ii[:, 1], ii[:, 2], e])


def errors(gpu: np.ndarray, ref: np.ndarray) -> Dict[str, float]:
    """Per-tensor error figures: relative L2, max abs, and the reference's max abs."""
    return {"rel_l2": rel_l2(gpu, ref), "max_abs": float(np.abs(gpu - ref).max()) if gpu.size else 0.0,
            "ref_max_abs": float(np.abs(ref).max()) if ref.size else 0.0, "n": int(gpu.shape[0]) if gpu.ndim else 1}


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
