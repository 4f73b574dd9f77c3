"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties one part of the oracle to something it does not share code
with: fixed-window local attention written with array slicing (zero offsets,
[MegaSlide-DiT, §9.1 Effect of local offsets]); exact gathers for integer
offsets; torch's grid_sample (bilinear on 5-D input, zero padding, the route of
[MegaSlide-DiT, §5.3 Implementation considerations]) with autograd; central
finite differences; affine reproduction by trilinear interpolation; dense
brute-force attention with multiplicities; hand-worked fixtures; and the
softmax's own invariants.
"""
import glob
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(12345)


def _rand(*shape, rng=None, scale=1.0):
    rng = rng or RNG
    return rng.standard_normal(shape) * scale


def _inputs(B, T, H, W, nh, d, window, off_sigma, rng, dtype_off=np.float32):
    P = window[0] * window[1] * window[2]
    q = _rand(B, T, H, W, nh, d, rng=rng)
    k = _rand(B, T, H, W, nh, d, rng=rng)
    v = _rand(B, T, H, W, nh, d, rng=rng)
    off = (_rand(B, T, H, W, nh, P, 3, rng=rng) * off_sigma).astype(dtype_off)
    return q, k, v, off


def _window_points(window, dilation):
    """Integer displacement of every window point, row-major over (t, h, w)."""
    kt, kh, kw = window
    pts = []
    for it in range(kt):
        for ih in range(kh):
            for iw in range(kw):
                pts.append((dilation[0] * (it - (kt - 1) // 2),
                            dilation[1] * (ih - (kh - 1) // 2),
                            dilation[2] * (iw - (kw - 1) // 2)))
    return pts


# ---------------------------------------------------------------------------
# 1. Zero offsets: fixed-window slide attention, written with slicing.
# ---------------------------------------------------------------------------

def _window_attention(q, k, v, window, dilation, scale):
    """Local attention over a fixed dilated window; K/V padded with zeros."""
    B, T, H, W, nh, d = q.shape
    pts = _window_points(window, dilation)
    R = [max(abs(p[a]) for p in pts) for a in range(3)]
    kp = np.pad(k, [(0, 0), (R[0], R[0]), (R[1], R[1]), (R[2], R[2]), (0, 0), (0, 0)])
    vp = np.pad(v, [(0, 0), (R[0], R[0]), (R[1], R[1]), (R[2], R[2]), (0, 0), (0, 0)])
    logits, vals = [], []
    for (dt, dh, dw) in pts:
        ks = kp[:, R[0] + dt:R[0] + dt + T, R[1] + dh:R[1] + dh + H, R[2] + dw:R[2] + dw + W]
        vs = vp[:, R[0] + dt:R[0] + dt + T, R[1] + dh:R[1] + dh + H, R[2] + dw:R[2] + dw + W]
        logits.append(scale * (q * ks).sum(-1))
        vals.append(vs)
    s = np.stack(logits, -1)
    m = s.max(-1, keepdims=True)
    e = np.exp(s - m)
    a = e / e.sum(-1, keepdims=True)
    o = np.einsum("bthwnp,pbthwnd->bthwnd", a, np.stack(vals, 0))
    lse = (m[..., 0] + np.log(e.sum(-1)))
    return o, lse


@pytest.mark.parametrize("window,dilation", [((3, 3, 3), (1, 1, 1)), ((3, 5, 5), (1, 1, 1)),
                                             ((3, 3, 3), (1, 2, 2)), ((1, 3, 5), (2, 1, 3))])
def test_zero_offsets_equal_fixed_window_attention(window, dilation):
    rng = np.random.default_rng(1)
    q, k, v, off = _inputs(2, 4, 6, 7, 2, 8, window, 0.0, rng)
    o, lse = oracle.forward(q, k, v, off, window, dilation)
    o_ref, lse_ref = _window_attention(q, k, v, window, dilation, 1 / math.sqrt(8))
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12


# ---------------------------------------------------------------------------
# 2. Integer offsets: every sample is an exact gather.
# ---------------------------------------------------------------------------

def test_integer_offsets_are_exact_gathers():
    rng = np.random.default_rng(2)
    window, dil = (3, 3, 3), (1, 1, 1)
    B, T, H, W, nh, d = 1, 3, 5, 6, 2, 4
    q, k, v, _ = _inputs(B, T, H, W, nh, d, window, 0.0, rng)
    P = 27
    off = rng.integers(-3, 4, size=(B, T, H, W, nh, P, 3)).astype(np.float32)
    o, lse, attn = oracle.forward(q, k, v, off, window, dil, want_attn=True)
    base, frac = oracle.geometry(off, window, dil)
    assert np.all(frac == 0)
    pts = np.array(_window_points(window, dil))
    scale = 1 / math.sqrt(d)
    for t in range(T):
        for h in range(H):
            for w in range(W):
                for n in range(nh):
                    pos = np.array([t, h, w]) + pts + off[0, t, h, w, n].astype(int)
                    assert np.array_equal(base[0, t, h, w, n], pos)
                    ks, vs = [], []
                    for (a, b_, c) in pos:
                        inside = 0 <= a < T and 0 <= b_ < H and 0 <= c < W
                        ks.append(k[0, a, b_, c, n] if inside else np.zeros(d))
                        vs.append(v[0, a, b_, c, n] if inside else np.zeros(d))
                    s = scale * np.array(ks) @ q[0, t, h, w, n]
                    e = np.exp(s - s.max())
                    ref = (e / e.sum()) @ np.array(vs)
                    assert np.abs(o[0, t, h, w, n] - ref).max() < 1e-12
                    assert abs(lse[0, t, h, w, n] - (s.max() + np.log(e.sum()))) < 1e-12


# ---------------------------------------------------------------------------
# 3. The pages' own route: grid_sample (trilinear, zeros) + softmax + sum,
#    with autograd for every gradient, in float64.
# ---------------------------------------------------------------------------

def _torch_route(q, k, v, off, window, dilation, scale, dout, gk=None, gv=None):
    """The route with autograd; with gk, gv [B,G,heads,d] the G global rows of
    each (batch, head) join the softmax (returns their gradients too)."""
    B, T, H, W, nh, d = q.shape
    P = off.shape[-2]
    pts = torch.tensor(_window_points(window, dilation), dtype=torch.int64)            # [P,3]
    tt, hh, ww = torch.meshgrid(torch.arange(T), torch.arange(H), torch.arange(W), indexing="ij")
    xyz = torch.stack([tt, hh, ww], -1).reshape(1, T, H, W, 1, 1, 3)
    ref = (xyz + pts.reshape(1, 1, 1, 1, 1, P, 3)).expand(B, T, H, W, nh, P, 3)
    # positions rounded as single-precision adds, then used in float64
    pos32 = ref.to(torch.float32) + torch.from_numpy(off)
    # the fraction is a single-precision subtraction (rounded for -0.5 < pos < 0);
    # hand grid_sample the position that this fraction stands for
    fl32 = torch.floor(pos32)
    pos32 = fl32.to(torch.float64) + (pos32 - fl32).to(torch.float64)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    ot = torch.tensor(off.astype(np.float64), requires_grad=True)
    pos = pos32 + (ot - ot.detach())                    # value: pos32; d pos / d off = 1
    size = torch.tensor([T, H, W], dtype=torch.float64)
    norm = 2.0 * pos / (size - 1) - 1.0                 # align_corners=True
    grid = norm[..., [2, 1, 0]]                          # grid_sample wants (x=w, y=h, z=t)
    grid = grid.permute(0, 4, 1, 2, 3, 5, 6).reshape(B * nh, T * H * W, P, 1, 3)

    def vol(x):  # [B,T,H,W,nh,d] -> [B*nh, d, T, H, W]
        return x.permute(0, 4, 5, 1, 2, 3).reshape(B * nh, d, T, H, W)

    ks = torch.nn.functional.grid_sample(vol(kt), grid, mode="bilinear", padding_mode="zeros",
                                         align_corners=True)[..., 0]          # [B*nh, d, N, P]
    vs = torch.nn.functional.grid_sample(vol(vt), grid, mode="bilinear", padding_mode="zeros",
                                         align_corners=True)[..., 0]
    qf = qt.permute(0, 4, 5, 1, 2, 3).reshape(B * nh, d, T * H * W, 1)
    s = scale * (qf * ks).sum(1)                         # [B*nh, N, P]
    if gk is not None:
        gkt = torch.tensor(gk, requires_grad=True)
        gvt = torch.tensor(gv, requires_grad=True)
        G = gk.shape[1]
        gkf = gkt.permute(0, 2, 3, 1).reshape(B * nh, d, 1, G)     # [B*nh, d, 1, G]
        gvf = gvt.permute(0, 2, 3, 1).reshape(B * nh, d, 1, G)
        s = torch.cat([s, scale * (qf * gkf).sum(1)], -1)          # [B*nh, N, P+G]
        vs = torch.cat([vs, gvf.expand(B * nh, d, T * H * W, G)], -1)
    a = torch.softmax(s, -1)
    o = (a.unsqueeze(1) * vs).sum(-1)                    # [B*nh, d, N]
    lse = torch.logsumexp(s, -1)
    o = o.reshape(B, nh, d, T, H, W).permute(0, 3, 4, 5, 1, 2)
    lse = lse.reshape(B, nh, T, H, W).permute(0, 2, 3, 4, 1)
    (o * torch.tensor(dout)).sum().backward()
    out = (o.detach().numpy(), lse.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(),
           ot.grad.numpy())
    return out + ((gkt.grad.numpy(), gvt.grad.numpy()) if gk is not None else ())


@pytest.mark.parametrize("window,dilation,sigma", [((3, 3, 3), (1, 1, 1), 0.7), ((3, 5, 5), (1, 1, 1), 2.0),
                                                   ((3, 3, 3), (1, 2, 2), 1.3), ((1, 1, 3), (1, 1, 2), 3.0)])
def test_matches_grid_sample_route_with_autograd(window, dilation, sigma):
    rng = np.random.default_rng(3)
    q, k, v, off = _inputs(2, 4, 5, 6, 2, 8, window, sigma, rng)
    dout = _rand(*q.shape, rng=rng)
    scale = 1 / math.sqrt(8)
    o, lse = oracle.forward(q, k, v, off, window, dilation)
    dq, dk, dv, doff = oracle.backward(q, k, v, off, dout, window, dilation)
    r = _torch_route(q, k, v, off, window, dilation, scale, dout)
    for name, mine, ref in zip(["o", "lse", "dq", "dk", "dv", "doff"], [o, lse, dq, dk, dv, doff], r):
        err = np.abs(mine - ref).max()
        assert err < 1e-10 * max(1.0, np.abs(ref).max()), (name, err)


# ---------------------------------------------------------------------------
# 4. Central finite differences of L = sum(o * G).
# ---------------------------------------------------------------------------

def test_backward_matches_finite_differences():
    rng = np.random.default_rng(4)
    window, dil = (3, 3, 3), (1, 1, 1)
    B, T, H, W, nh, d = 1, 3, 4, 4, 1, 4
    q, k, v, _ = _inputs(B, T, H, W, nh, d, window, 0.0, rng)
    P = 27
    # offsets on a 2^-12 lattice with fractions in [0.1, 0.9): every perturbed
    # position is exactly representable in single precision and stays in its cell
    whole = rng.integers(-2, 3, size=(B, T, H, W, nh, P, 3))
    frac = rng.integers(410, 3686, size=whole.shape) / 4096.0
    off = (whole + frac).astype(np.float32)
    G = _rand(*q.shape, rng=rng)
    dq, dk, dv, doff = oracle.backward(q, k, v, off, G, window, dil)

    def loss(q_, k_, v_, off_):
        return float((oracle.forward(q_, k_, v_, off_, window, dil)[0] * G).sum())

    eps = 1e-6
    for name, x, g in [("q", q, dq), ("k", k, dk), ("v", v, dv)]:
        for _ in range(12):
            i = tuple(rng.integers(0, s) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p, off) - loss(*args_m, off)) / (2 * eps)
            assert abs(fd - g[i]) <= 1e-6 * max(1.0, abs(fd)), (name, i, fd, g[i])
    h = 2.0 ** -12
    for _ in range(24):
        i = tuple(rng.integers(0, s) for s in off.shape)
        op, om = off.copy(), off.copy()
        op[i] += np.float32(h)
        om[i] -= np.float32(h)
        fd = (loss(q, k, v, op) - loss(q, k, v, om)) / (2 * h)
        # the loss is a smooth function of the offset inside a cell: O(h^2) error
        assert abs(fd - doff[i]) <= 2e-5 * max(1.0, abs(fd)), (i, fd, doff[i])


# ---------------------------------------------------------------------------
# 5. Affine reproduction: trilinear interpolation of an affine field is exact.
# ---------------------------------------------------------------------------

def test_affine_field_is_reproduced_at_the_sample_position():
    rng = np.random.default_rng(5)
    B, T, H, W, nh, d = 1, 5, 6, 7, 2, 3
    window, dil = (1, 1, 1), (1, 1, 1)
    tt, hh, ww = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    alpha = np.array([0.5, -1.0, 2.0])
    beta = np.array([[1.0, 0.3, -2.0], [-0.7, 2.5, 0.25], [0.125, -1.5, 3.0]])  # rows: t, h, w slopes
    field = alpha + tt[..., None] * beta[0] + hh[..., None] * beta[1] + ww[..., None] * beta[2]
    v = np.broadcast_to(field[None, :, :, :, None, :], (B, T, H, W, nh, d)).copy()
    q, k, _, _ = _inputs(B, T, H, W, nh, d, window, 0.0, rng)
    # keep every corner inside the grid: position in [0, size-1)
    target = np.stack([rng.uniform(0, T - 1, (B, T, H, W, nh)), rng.uniform(0, H - 1, (B, T, H, W, nh)),
                       rng.uniform(0, W - 1, (B, T, H, W, nh))], -1)
    off = (target - np.stack([tt, hh, ww], -1)[None, :, :, :, None, :]).astype(np.float32)[..., None, :]
    o, _ = oracle.forward(q, k, v, off, window, dil)
    pos = (np.stack([tt, hh, ww], -1)[None, :, :, :, None, :].astype(np.float32) + off[..., 0, :]).astype(np.float64)
    expect = alpha + pos[..., 0:1] * beta[0] + pos[..., 1:2] * beta[1] + pos[..., 2:3] * beta[2]
    assert np.abs(o - expect).max() < 1e-12


def test_single_point_window_zero_offset_is_identity():
    rng = np.random.default_rng(6)
    q, k, v, off = _inputs(2, 3, 4, 5, 3, 4, (1, 1, 1), 0.0, rng)
    o, lse = oracle.forward(q, k, v, off, (1, 1, 1))
    assert np.array_equal(o, v)
    assert np.abs(lse - (q * k).sum(-1) / 2.0).max() < 1e-14


# ---------------------------------------------------------------------------
# 6. Softmax invariants and the all-outside case.
# ---------------------------------------------------------------------------

def test_attention_weights_are_a_distribution_and_uniform_for_zero_keys():
    rng = np.random.default_rng(7)
    window = (3, 5, 5)
    q, k, v, off = _inputs(1, 4, 6, 6, 2, 8, window, 2.0, rng)
    _, _, a = oracle.forward(q, k, v, off, window, want_attn=True)
    assert np.all(a >= 0) and np.all(a <= 1)
    assert np.abs(a.sum(-1) - 1).max() < 1e-13
    o0, lse0, a0 = oracle.forward(q, np.zeros_like(k), v, off, window, want_attn=True)
    assert np.abs(a0 - 1 / 75).max() < 1e-15
    assert np.abs(lse0 - math.log(75)).max() < 1e-13


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan, 3.0e9, -1.5e9])
def test_samples_far_outside_or_not_finite_read_zero(bad):
    rng = np.random.default_rng(8)
    window = (3, 3, 3)
    q, k, v, off = _inputs(1, 3, 4, 4, 1, 4, window, 0.0, rng)
    off[...] = np.float32(bad)
    o, lse = oracle.forward(q, k, v, off, window)
    assert np.array_equal(o, np.zeros_like(o))
    assert np.abs(lse - math.log(27)).max() < 1e-13
    base, frac = oracle.geometry(off, window)
    assert np.all(base == oracle.OUTSIDE) and np.all(frac == 0)
    dq, dk, dv, doff = oracle.backward(q, k, v, off, _rand(*q.shape, rng=rng), window)
    for g in (dq, dk, dv, doff):
        assert np.array_equal(g, np.zeros_like(g))


# ---------------------------------------------------------------------------
# 7. Dense brute force with multiplicities (integer offsets).
# ---------------------------------------------------------------------------

def test_dense_bruteforce_attention_with_multiplicity():
    rng = np.random.default_rng(9)
    window, dil = (3, 3, 3), (1, 1, 1)
    B, T, H, W, nh, d = 1, 3, 3, 3, 2, 4
    q, k, v, _ = _inputs(B, T, H, W, nh, d, window, 0.0, rng)
    off = rng.integers(-2, 3, size=(B, T, H, W, nh, 27, 3)).astype(np.float32)
    o, lse = oracle.forward(q, k, v, off, window, dil)
    pts = np.array(_window_points(window, dil))
    N = T * H * W
    scale = 0.5
    for n in range(nh):
        Kf = k[0, :, :, :, n].reshape(N, d)
        Vf = v[0, :, :, :, n].reshape(N, d)
        for x in range(N):
            t, h, w = np.unravel_index(x, (T, H, W))
            pos = np.array([t, h, w]) + pts + off[0, t, h, w, n].astype(int)
            count = np.zeros(N)
            n_out = 0
            for (a, b_, c) in pos:
                if 0 <= a < T and 0 <= b_ < H and 0 <= c < W:
                    count[np.ravel_multi_index((a, b_, c), (T, H, W))] += 1
                else:
                    n_out += 1
            s = scale * Kf @ q[0, t, h, w, n]                     # dense logits over all N keys
            z = (count * np.exp(s)).sum() + n_out                # outside samples: logit 0, value 0
            ref = (count * np.exp(s)) @ Vf / z
            assert np.abs(o[0, t, h, w, n] - ref).max() < 1e-12
            assert abs(lse[0, t, h, w, n] - math.log(z)) < 1e-12


# ---------------------------------------------------------------------------
# 8. Backward invariants.
# ---------------------------------------------------------------------------

def test_dv_mass_equals_dout_mass_for_in_grid_samples():
    rng = np.random.default_rng(10)
    window = (3, 3, 3)
    T, H, W, d = 9, 9, 9, 4
    K = _rand(T, H, W, d, rng=rng)
    V = _rand(T, H, W, d, rng=rng)
    qpos = oracle.grid_positions(T, H, W)
    interior = np.all((qpos >= 3) & (qpos <= 5), axis=1)
    qpos = qpos[interior]
    n = len(qpos)
    q = _rand(n, d, rng=rng)
    off = rng.uniform(-0.99, 0.99, size=(n, 27, 3)).astype(np.float32)
    dO = _rand(n, d, rng=rng)
    dq, doff, dK, dV = oracle.backward_queries((T, H, W), window, (1, 1, 1), 0.5, qpos, q, off, (0, 0, 0),
                                               K, V, dO)
    assert np.abs(dV.sum((0, 1, 2)) - dO.sum(0)).max() < 1e-12
    # all keys equal -> all logits equal -> dq = 0 and dK sums to zero
    Kc = np.broadcast_to(_rand(d, rng=rng), K.shape).copy()
    dq2, _, dK2, _ = oracle.backward_queries((T, H, W), window, (1, 1, 1), 0.5, qpos, q, off, (0, 0, 0),
                                             Kc, V, dO)
    assert np.abs(dq2).max() < 1e-12
    assert np.abs(dK2.sum((0, 1, 2))).max() < 1e-12


def test_heads_are_independent_and_permute():
    rng = np.random.default_rng(11)
    window = (3, 3, 3)
    q, k, v, off = _inputs(1, 3, 4, 5, 3, 4, window, 1.0, rng)
    dO = _rand(*q.shape, rng=rng)
    perm = [2, 0, 1]
    o, lse = oracle.forward(q, k, v, off, window)
    o2, lse2 = oracle.forward(q[..., perm, :], k[..., perm, :], v[..., perm, :], off[..., perm, :, :], window)
    assert np.array_equal(o[..., perm, :], o2) and np.array_equal(lse[..., perm], lse2)
    g = oracle.backward(q, k, v, off, dO, window)
    g2 = oracle.backward(q[..., perm, :], k[..., perm, :], v[..., perm, :], off[..., perm, :, :],
                         dO[..., perm, :], window)
    for a, b in zip(g, g2):
        assert np.array_equal(a[..., perm, :] if a.ndim == 6 else a[..., perm, :, :], b)


def test_sub_box_matches_whole_grid():
    rng = np.random.default_rng(12)
    window = (3, 3, 3)
    T, H, W, d = 6, 7, 8, 4
    q, k, v, off = _inputs(1, T, H, W, 1, d, window, 0.4, rng)
    dO = _rand(*q.shape, rng=rng)
    o, lse = oracle.forward(q, k, v, off, window)
    dq, dk, dv, doff = oracle.backward(q, k, v, off, dO, window)
    # queries in the middle of the grid; their samples stay within +-3 tokens
    qpos = oracle.grid_positions(T, H, W)
    sel = np.all((qpos >= 2) & (qpos <= [3, 4, 5]), axis=1)
    qp = qpos[sel]
    assert np.abs(off[0][qp[:, 0], qp[:, 1], qp[:, 2]]).max() < 1.9
    box0, box1 = (0, 0, 0), (T, H, W)
    sl = (slice(box0[0], box1[0]), slice(box0[1], box1[1]), slice(box0[2], box1[2]))
    o2, lse2 = oracle.forward_queries((T, H, W), window, (1, 1, 1), 0.5, qp, q[0][qp[:, 0], qp[:, 1], qp[:, 2], 0],
                                      off[0][qp[:, 0], qp[:, 1], qp[:, 2], 0], box0, k[0][sl][..., 0, :],
                                      v[0][sl][..., 0, :])
    assert np.array_equal(o2, o[0][qp[:, 0], qp[:, 1], qp[:, 2], 0])
    # a box too small to hold every touched corner is an error, not a zero
    with pytest.raises(RuntimeError):
        oracle.forward_queries((T, H, W), window, (1, 1, 1), 0.5, qp, q[0][qp[:, 0], qp[:, 1], qp[:, 2], 0],
                               off[0][qp[:, 0], qp[:, 1], qp[:, 2], 0], (2, 2, 2), k[0][2:4, 2:4, 2:4, 0],
                               v[0][2:4, 2:4, 2:4, 0])


# ---------------------------------------------------------------------------
# 9. Geometry: single-precision positions, written independently in numpy.
# ---------------------------------------------------------------------------

def test_geometry_is_single_precision_floor_and_fraction():
    rng = np.random.default_rng(13)
    window, dil = (3, 5, 5), (1, 2, 2)
    T, H, W = 6, 9, 11
    off = (rng.standard_normal((1, T, H, W, 1, 75, 3)) * 3).astype(np.float32)
    off[0, 0, 0, 0, 0, :5] = np.float32([0.5, -0.5, 1e-8, -1e-8, 2.0])[:, None]
    base, frac = oracle.geometry(off, window, dil)
    pts = np.array(_window_points(window, dil), dtype=np.int64)
    tt, hh, ww = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    ref = np.stack([tt, hh, ww], -1)[:, :, :, None, :] + pts[None, None, None]
    pos = ref.astype(np.float32) + off[0, :, :, :, 0]            # float32 + float32: RNE single add
    fl = np.floor(pos)
    assert np.array_equal(base[0, :, :, :, 0], fl.astype(np.int32))
    assert np.array_equal(frac[0, :, :, :, 0].view(np.int32), (pos - fl).view(np.int32))
    assert np.all((frac >= 0) & (frac <= 1))
    # a tiny negative position: the single-precision fraction rounds up to 1
    b1, f1 = oracle.geometry(np.full((1, 1, 1, 1, 1, 1, 3), -1e-9, np.float32), (1, 1, 1))
    assert np.array_equal(b1.ravel(), [-1, -1, -1]) and np.array_equal(f1.ravel(), [1.0, 1.0, 1.0])


# ---------------------------------------------------------------------------
# 10. Hand-worked fixtures.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(HERE, "golden", "*.json"))))
def test_hand_worked_fixture(path):
    g = json.load(open(path))
    T, H, W = g["grid"]
    d = g["d"]
    qpos = oracle.grid_positions(T, H, W)
    N = T * H * W
    q = np.array(g["q"]).reshape(N, d)
    K = np.array(g["k"]).reshape(T, H, W, d)
    V = np.array(g["v"]).reshape(T, H, W, d)
    P = g["window"][0] * g["window"][1] * g["window"][2]
    off = np.array(g["offsets"], dtype=np.float32).reshape(N, P, 3)
    o, lse = oracle.forward_queries((T, H, W), g["window"], g["dilation"], g["scale"], qpos, q, off, (0, 0, 0), K, V)
    ex = g["expect"]
    assert np.abs(o - np.array(ex["o"]).reshape(N, d)).max() < 1e-14
    assert np.abs(lse - np.array(ex["lse"])).max() < 1e-14
    if "dout" in g:
        dO = np.array(g["dout"]).reshape(N, d)
        dq, doff, dK, dV = oracle.backward_queries((T, H, W), g["window"], g["dilation"], g["scale"], qpos, q,
                                                   off, (0, 0, 0), K, V, dO)
        assert np.abs(dq - np.array(ex["dq"]).reshape(N, d)).max() < 1e-14
        assert np.abs(dK.reshape(N, d) - np.array(ex["dk"])).max() < 1e-14
        assert np.abs(dV.reshape(N, d) - np.array(ex["dv"])).max() < 1e-14
        assert np.abs(doff - np.array(ex["doff"]).reshape(N, P, 3)).max() < 1e-14


# ---------------------------------------------------------------------------
# 11. Offset projection: a textbook GEMM, checked by explicit loops.
# ---------------------------------------------------------------------------

def test_projection_matches_explicit_loops():
    rng = np.random.default_rng(14)
    N, C, F = 5, 7, 6
    q = rng.standard_normal((N, C)); w = rng.standard_normal((F, C)); b = rng.standard_normal(F)
    out = oracle.offset_proj(q, w, b)
    g = rng.standard_normal((N, F))
    dq, dw, db = oracle.offset_proj_backward(q, w, g)
    for n in range(N):
        for f in range(F):
            assert abs(out[n, f] - (sum(q[n, c] * w[f, c] for c in range(C)) + b[f])) < 1e-12
        for c in range(C):
            assert abs(dq[n, c] - sum(g[n, f] * w[f, c] for f in range(F))) < 1e-12
    for f in range(F):
        for c in range(C):
            assert abs(dw[f, c] - sum(g[n, f] * q[n, c] for n in range(N))) < 1e-12
        assert abs(db[f] - sum(g[n, f] for n in range(N))) < 1e-12
    # a basis-vector weight picks single query columns (catches a transposed operand)
    w1 = np.zeros((F, C)); w1[np.arange(F), np.arange(F)] = 1
    assert np.array_equal(oracle.offset_proj(q, w1), q[:, :F])


# ---------------------------------------------------------------------------
# 12. Depthwise 3-D convolution of the offset network: explicit loops, a
# library correlation, shifted deltas, the adjoint identity and finite
# differences pin the forward and all three gradients.
# ---------------------------------------------------------------------------

def _dwconv_loops(q, w, b):
    B, T, H, W, C = q.shape
    y = np.zeros_like(q)
    for bb in range(B):
        for t in range(T):
            for h in range(H):
                for x in range(W):
                    for c in range(C):
                        s = b[c]
                        for i in range(3):
                            for j in range(3):
                                for k in range(3):
                                    tt, hh, xx = t + i - 1, h + j - 1, x + k - 1
                                    if 0 <= tt < T and 0 <= hh < H and 0 <= xx < W:
                                        s += w[c, i, j, k] * q[bb, tt, hh, xx, c]
                        y[bb, t, h, x, c] = s
    return y


def test_dwconv_matches_explicit_loops():
    rng = np.random.default_rng(21)
    q = rng.standard_normal((2, 3, 4, 5, 3)); w = rng.standard_normal((3, 3, 3, 3)); b = rng.standard_normal(3)
    assert np.abs(oracle.dwconv3d(q, w, b) - _dwconv_loops(q, w, b)).max() < 1e-12


def test_dwconv_matches_library_correlation():
    from scipy.ndimage import correlate
    rng = np.random.default_rng(22)
    q = rng.standard_normal((1, 5, 6, 7, 4)); w = rng.standard_normal((4, 3, 3, 3))
    y = oracle.dwconv3d(q, w)
    for c in range(4):
        ref = correlate(q[0, ..., c], w[c], mode="constant", cval=0.0)
        assert np.abs(y[0, ..., c] - ref).max() < 1e-12


def test_dwconv_deltas_identity_and_shift():
    rng = np.random.default_rng(23)
    q = rng.standard_normal((1, 4, 5, 6, 2))
    w = np.zeros((2, 3, 3, 3)); w[:, 1, 1, 1] = 1.0
    assert np.array_equal(oracle.dwconv3d(q, w), q)
    # tap (2, 1, 0) reads the input one frame later and one token to the left
    w = np.zeros((2, 3, 3, 3)); w[:, 2, 1, 0] = 1.0
    y = oracle.dwconv3d(q, w)
    assert np.array_equal(y[0, :-1, :, 1:], q[0, 1:, :, :-1])
    assert np.all(y[0, -1] == 0) and np.all(y[0, :, :, 0] == 0)


def test_dwconv_backward_adjoint_and_finite_differences():
    rng = np.random.default_rng(24)
    q = rng.standard_normal((1, 3, 3, 4, 2)); w = rng.standard_normal((2, 3, 3, 3)); b = rng.standard_normal(2)
    g = rng.standard_normal(q.shape)
    dq, dw, db = oracle.dwconv3d_backward(q, w, g)
    # <conv(q), g> = <q, conv^T(g)> for the linear part
    assert abs(np.sum(oracle.dwconv3d(q, w) * g) - np.sum(q * dq)) < 1e-10
    L = lambda q_, w_, b_: float(np.sum(oracle.dwconv3d(q_, w_, b_) * g))
    eps = 1e-6
    for idx in [(0, 0, 0, 0, 0), (0, 1, 2, 3, 1), (0, 2, 1, 0, 0)]:
        e = np.zeros_like(q); e[idx] = eps
        assert abs((L(q + e, w, b) - L(q - e, w, b)) / (2 * eps) - dq[idx]) < 1e-6
    for idx in [(0, 0, 0, 0), (1, 2, 1, 0), (0, 1, 1, 1), (1, 0, 2, 2)]:
        e = np.zeros_like(w); e[idx] = eps
        assert abs((L(q, w + e, b) - L(q, w - e, b)) / (2 * eps) - dw[idx]) < 1e-6
    for c in range(2):
        e = np.zeros_like(b); e[c] = eps
        assert abs((L(q, w, b + e) - L(q, w, b - e)) / (2 * eps) - db[c]) < 1e-6


# ---------------------------------------------------------------------------
# The transformer block around the operator (layer normalisation, linear
# layers, residual; [MegaSlide-DiT, §5.3 Implementation considerations]).
# ---------------------------------------------------------------------------

def test_layernorm_matches_torch_with_autograd():
    """Forward and all three gradients against torch's layer_norm in float64
    (an independent library routine) with autograd."""
    rng = np.random.default_rng(71)
    x = rng.standard_normal((37, 48)) * 3.0 + 1.5
    g = 1.0 + 0.3 * rng.standard_normal(48)
    b = 0.2 * rng.standard_normal(48)
    dy = rng.standard_normal((37, 48))
    eps = 1e-6
    y, mean, rstd = oracle.layernorm(x, g, b, eps)
    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    yt = torch.nn.functional.layer_norm(xt, (48,), gt, bt, eps)
    yt.backward(torch.tensor(dy))
    assert np.abs(y - yt.detach().numpy()).max() < 1e-12
    dx, dg, db = oracle.layernorm_backward(x, g, dy, eps)
    assert np.abs(dx - xt.grad.numpy()).max() < 1e-11
    assert np.abs(dg - gt.grad.numpy()).max() < 1e-11
    assert np.abs(db - bt.grad.numpy()).max() < 1e-11
    assert np.allclose(mean, x.mean(1)) and np.allclose(rstd, 1.0 / np.sqrt(x.var(1) + eps))


def test_layernorm_invariants():
    """Without affine parameters every row has mean 0 and (population) variance
    var/(var+eps); the result is invariant under x -> a*x + c for a > 0 (up to
    eps); gamma and beta act per channel (a channel permutation commutes)."""
    rng = np.random.default_rng(72)
    x = rng.standard_normal((20, 64))
    y, _, _ = oracle.layernorm(x, None, None, 1e-12)
    assert np.abs(y.mean(1)).max() < 1e-12
    assert np.abs(y.var(1) - 1.0).max() < 1e-9
    y2, _, _ = oracle.layernorm(2.5 * x - 7.0, None, None, 1e-12)
    assert np.abs(y2 - y).max() < 1e-9
    g, b = rng.standard_normal(64), rng.standard_normal(64)
    perm = rng.permutation(64)
    ya, _, _ = oracle.layernorm(x, g, b)
    yp, _, _ = oracle.layernorm(x[:, perm], g[perm], b[perm])
    assert np.abs(ya[:, perm] - yp).max() < 1e-12


def test_layernorm_backward_finite_differences():
    rng = np.random.default_rng(73)
    x = rng.standard_normal((5, 16))
    g = 1.0 + 0.5 * rng.standard_normal(16)
    b = rng.standard_normal(16)
    G = rng.standard_normal((5, 16))
    loss = lambda xx, gg, bb: float((oracle.layernorm(xx, gg, bb)[0] * G).sum())
    dx, dg, db = oracle.layernorm_backward(x, g, G)
    eps = 1e-6
    for _ in range(12):
        i, j = rng.integers(5), rng.integers(16)
        xp, xm = x.copy(), x.copy()
        xp[i, j] += eps
        xm[i, j] -= eps
        fd = (loss(xp, g, b) - loss(xm, g, b)) / (2 * eps)
        assert abs(fd - dx[i, j]) <= 1e-6 * max(1.0, abs(fd))
    for arr, grad in ((g, dg), (b, db)):
        j = rng.integers(16)
        ap, am = arr.copy(), arr.copy()
        ap[j] += eps
        am[j] -= eps
        args_p = (x, ap, b) if arr is g else (x, g, ap)
        args_m = (x, am, b) if arr is g else (x, g, am)
        fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert abs(fd - grad[j]) <= 1e-6 * max(1.0, abs(fd))


def _block_params(C, heads, P, rng, off_scale=0.2):
    return {"ln_g": 1.0 + 0.2 * rng.standard_normal(C), "ln_b": 0.1 * rng.standard_normal(C),
            "w_qkv": rng.standard_normal((3 * C, C)) / np.sqrt(C), "b_qkv": 0.1 * rng.standard_normal(3 * C),
            "w_off": off_scale * rng.standard_normal((heads * P * 3, C)),
            "b_off": 0.3 * rng.standard_normal(heads * P * 3),
            "w_out": rng.standard_normal((C, C)) / np.sqrt(C), "b_out": 0.1 * rng.standard_normal(C)}


def test_block_residual_and_projections():
    """With a zero output projection the block is the identity (the residual
    path); the block's q/k/v are the linear maps of the normalised input, and
    its attention output is the attention oracle's on them."""
    rng = np.random.default_rng(74)
    heads, d, window = 2, 4, (3, 3, 3)
    C, P = heads * d, 27
    x = rng.standard_normal((1, 3, 3, 4, C))
    p = _block_params(C, heads, P, rng)
    p0 = dict(p, w_out=np.zeros((C, C)), b_out=np.zeros(C))
    assert np.array_equal(oracle.block_forward(x, p0, heads, window)["y"], x)
    f = oracle.block_forward(x, p, heads, window)
    h = (x - x.mean(-1, keepdims=True)) / np.sqrt(x.var(-1, keepdims=True) + 1e-6) * p["ln_g"] + p["ln_b"]
    assert np.abs(f["h"] - h).max() < 1e-12
    q = h @ p["w_qkv"][:C].T + p["b_qkv"][:C]
    assert np.abs(f["q"].reshape(q.shape) - q).max() < 1e-12
    o, _ = oracle.forward(f["q"], f["k"], f["v"], f["offsets"], window)
    assert np.abs(f["o"] - o).max() < 1e-12
    assert np.abs(f["y"] - (x + o.reshape(x.shape) @ p["w_out"].T + p["b_out"])).max() < 1e-12


@pytest.mark.parametrize("off_scale,eps,tol", [(0.0, 1e-4, 1e-7), (0.2, 1e-3, 1e-2)])
def test_block_backward_finite_differences(off_scale, eps, tol):
    """The block's gradients (through the output projection, the attention with
    offsets that depend on q, the q/k/v projections, the layer normalisation
    and the residual path) against central finite differences of the whole
    block's forward. With a zero offset projection the loss is smooth and the
    check is tight; with offsets that follow q, the single-precision rounding
    of the offsets (part of the operator) makes the loss a staircase at the
    1e-7 scale and its kinks at integer positions are crossed by some of the
    many samples a parameter moves, so the step is larger and the bound looser:
    the offsets' path carries about twice the direct share of dq here, so a
    dropped or mis-signed term is an O(1) error."""
    rng = np.random.default_rng(75)
    heads, d, window = 2, 4, (3, 3, 3)
    C, P = heads * d, 27
    x = rng.standard_normal((1, 3, 3, 4, C))
    p = _block_params(C, heads, P, rng, off_scale=off_scale)
    G = rng.standard_normal(x.shape)
    loss = lambda xx, pp: float((oracle.block_forward(xx, pp, heads, window)["y"] * G).sum())
    g = oracle.block_backward(x, p, G, heads, window)

    def fd(name, idx):
        if name == "x":
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            return (loss(xp, p) - loss(xm, p)) / (2 * eps)
        pp, pm = dict(p), dict(p)
        pp[name] = p[name].copy()
        pm[name] = p[name].copy()
        pp[name][idx] += eps
        pm[name][idx] -= eps
        return (loss(x, pp) - loss(x, pm)) / (2 * eps)

    # with the tight bound, the offset projection's own parameters are left out:
    # perturbing them moves the (single-precision) offsets directly
    names = [n for n in oracle.BLOCK_PARAMS if off_scale > 0 or n not in ("w_off", "b_off")]
    checks = [("x", "dx")] * 6 + [(n, "d" + n) for n in names for _ in range(2)]
    for name, gname in checks:
        arr = x if name == "x" else p[name]
        idx = tuple(int(rng.integers(s)) for s in arr.shape)
        ref = fd(name, idx)
        err = abs(ref - g[gname][idx]) / max(1.0, abs(ref))
        assert err <= tol, (name, idx, ref, g[gname][idx])


# ---------------------------------------------------------------------------
# Hybrid attention: G global tokens join each query's softmax ([MegaSlide-DiT,
# §11 Limitations and Discussion, future work (i)]).
# ---------------------------------------------------------------------------

def test_hybrid_without_global_tokens_is_the_operator():
    rng = np.random.default_rng(81)
    window = (3, 3, 3)
    q, k, v, off = _inputs(1, 3, 4, 5, 2, 8, window, 1.0, rng)
    dout = _rand(*q.shape, rng=rng)
    empty = np.zeros((1, 0, 2, 8))
    o, lse = oracle.forward(q, k, v, off, window)
    oh, lh = oracle.forward_hybrid(q, k, v, off, empty, empty, window)
    assert np.array_equal(o, oh) and np.array_equal(lse, lh)
    ref = oracle.backward(q, k, v, off, dout, window)
    got = oracle.backward_hybrid(q, k, v, off, empty, empty, dout, window)
    for a, b in zip(ref, got[:4]):
        assert np.array_equal(a, b)
    assert got[4].shape == (1, 0, 2, 8)


@pytest.mark.parametrize("window,dilation,sigma,G", [((3, 3, 3), (1, 1, 1), 0.8, 5), ((3, 5, 5), (1, 1, 1), 2.0, 16),
                                                     ((1, 3, 3), (1, 2, 2), 1.3, 1)])
def test_hybrid_matches_grid_sample_route_with_global_keys(window, dilation, sigma, G):
    """The hybrid forward and every gradient (q, k, v, offsets and the global
    rows) against torch: grid_sample for the local samples, the global rows
    appended to each query's logits, one softmax, autograd."""
    rng = np.random.default_rng(82)
    q, k, v, off = _inputs(2, 3, 4, 5, 2, 8, window, sigma, rng)
    gk, gv = _rand(2, G, 2, 8, rng=rng), _rand(2, G, 2, 8, rng=rng)
    dout = _rand(*q.shape, rng=rng)
    scale = 1 / math.sqrt(8)
    o, lse = oracle.forward_hybrid(q, k, v, off, gk, gv, window, dilation)
    got = oracle.backward_hybrid(q, k, v, off, gk, gv, dout, window, dilation)
    r = _torch_route(q, k, v, off, window, dilation, scale, dout, gk, gv)
    for name, mine, ref in zip(["o", "lse", "dq", "dk", "dv", "doff", "dgk", "dgv"], [o, lse] + list(got), r):
        err = np.abs(mine - ref).max()
        assert err < 1e-10 * max(1.0, np.abs(ref).max()), (name, err)


def test_hybrid_global_tokens_as_grid_tokens_equal_dense_attention():
    """With a single-point window at zero offset and global tokens that are
    copies of grid tokens, each query attends to itself plus those tokens:
    plain dense attention over that list (written here directly)."""
    rng = np.random.default_rng(83)
    B, T, H, W, nh, d = 1, 2, 3, 4, 2, 6
    q, k, v = (_rand(B, T, H, W, nh, d, rng=rng) for _ in range(3))
    off = np.zeros((B, T, H, W, nh, 1, 3), dtype=np.float32)
    picks = [(0, 0, 0), (1, 2, 3), (0, 1, 2)]
    gk = np.stack([k[0, t, h, w] for (t, h, w) in picks])[None]   # [1, G, nh, d]
    gv = np.stack([v[0, t, h, w] for (t, h, w) in picks])[None]
    o, lse = oracle.forward_hybrid(q, k, v, off, gk, gv, (1, 1, 1))
    scale = 1 / math.sqrt(d)
    for t in range(T):
        for h in range(H):
            for w in range(W):
                for n in range(nh):
                    keys = [k[0, t, h, w, n]] + [gk[0, g, n] for g in range(len(picks))]
                    vals = [v[0, t, h, w, n]] + [gv[0, g, n] for g in range(len(picks))]
                    s = scale * np.array(keys) @ q[0, t, h, w, n]
                    e = np.exp(s - s.max())
                    assert np.abs(o[0, t, h, w, n] - (e / e.sum()) @ np.array(vals)).max() < 1e-12
                    assert abs(lse[0, t, h, w, n] - (s.max() + np.log(e.sum()))) < 1e-12


def test_hybrid_backward_finite_differences_of_global_rows():
    rng = np.random.default_rng(84)
    window = (3, 3, 3)
    q, k, v, off = _inputs(1, 2, 3, 4, 1, 4, window, 0.9, rng)
    gk, gv = _rand(1, 3, 1, 4, rng=rng), _rand(1, 3, 1, 4, rng=rng)
    G_ = _rand(*q.shape, rng=rng)
    loss = lambda a, b: float((oracle.forward_hybrid(q, k, v, off, a, b, window)[0] * G_).sum())
    _, _, _, _, dgk, dgv = oracle.backward_hybrid(q, k, v, off, gk, gv, G_, window)
    eps = 1e-6
    for arr, grad, first in ((gk, dgk, True), (gv, dgv, False)):
        for _ in range(4):
            idx = tuple(int(rng.integers(s)) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[idx] += eps
            am[idx] -= eps
            fd = (loss(ap, gv) - loss(am, gv)) / (2 * eps) if first else (loss(gk, ap) - loss(gk, am)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd))
