"""The sampled-oracle helpers used by the full-size GPU parity tests agree
with the whole-grid oracle (CPU tensors stand in for device tensors)."""
import numpy as np

import oracle
from deformable_local_attention_amd import synth
from gpu_helpers import (HeadOracle, face_tokens, gather, grid_corner_tokens, interior_tokens, oracle_dkdv_at_keys,
                         oracle_queries, random_tokens, rows_at, sample_queries, to_np)


def test_sampled_queries_and_keys_match_whole_grid():
    wl = synth.WORKLOADS["1080p-bf16-p75-det"].with_grid(T=5, H=7, W=9, heads=2, name="crop")
    x = synth.make_inputs(wl, "cpu", seed=3)
    off = x["offsets"]
    o, lse = oracle.forward(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), to_np(off), wl.window, wl.dilation)
    dq, dk, dv, doff = oracle.backward(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), to_np(off), to_np(x["dout"]),
                                       wl.window, wl.dilation)
    qs = sample_queries(wl, heads=[0, 1], n_random=6, seed=1, faces=4)
    r = oracle_queries(wl, x, off, qs, dout=x["dout"])
    idx = np.array(qs)
    sel = (idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3], idx[:, 4])
    assert np.abs(r["o"] - o[sel]).max() < 1e-12
    assert np.abs(r["lse"] - lse[sel]).max() < 1e-12
    assert np.abs(r["dq"] - dq[sel]).max() < 1e-12
    assert np.abs(r["doff"] - doff[sel]).max() < 1e-12
    keys = [(0, 2, 3, 4, 0), (0, 0, 0, 0, 1), (0, 4, 6, 8, 1), (0, 1, 6, 0, 0)]
    kk, vv = oracle_dkdv_at_keys(wl, x, off, x["dout"], keys)
    ki = np.array(keys)
    ksel = (ki[:, 0], ki[:, 1], ki[:, 2], ki[:, 3], ki[:, 4])
    assert np.abs(kk - dk[ksel]).max() < 1e-12
    assert np.abs(vv - dv[ksel]).max() < 1e-12
    assert np.array_equal(gather(x["q"], qs), to_np(x["q"])[sel])


def test_head_oracle_matches_whole_grid():
    """The full-size parity driver's per-head oracle (whole-grid box, bulk and
    threaded query calls, vectorised search for the queries reaching a key)
    against the whole-grid oracle."""
    wl = synth.WORKLOADS["1080p-bf16-p75-det"].with_grid(T=6, H=8, W=11, heads=3, name="crop")
    x = synth.make_inputs(wl, "cpu", seed=4)
    off = x["offsets"]
    o, lse = oracle.forward(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), to_np(off), wl.window, wl.dilation)
    dq, dk, dv, doff = oracle.backward(to_np(x["q"]), to_np(x["k"]), to_np(x["v"]), to_np(off), to_np(x["dout"]),
                                       wl.window, wl.dilation)
    rng = np.random.default_rng(0)
    for e in range(wl.heads):
        ho = HeadOracle(wl, x, 0, e, off, x["dout"], threads=3)
        pos = np.unique(np.concatenate([face_tokens(wl.T, wl.H, wl.W), random_tokens(wl.T, wl.H, wl.W, 20, rng)]),
                        axis=0)
        sel = (0, pos[:, 0], pos[:, 1], pos[:, 2], e)
        oo, ll = ho.forward(pos)
        assert np.abs(oo - o[sel]).max() < 1e-12 and np.abs(ll - lse[sel]).max() < 1e-12
        qq, ff = ho.backward_queries(pos)
        assert np.abs(qq - dq[sel]).max() < 1e-12 and np.abs(ff - doff[sel]).max() < 1e-12
        keys = np.unique(np.concatenate([grid_corner_tokens(wl.T, wl.H, wl.W),
                                         interior_tokens(wl.T, wl.H, wl.W, 6, rng)]), axis=0)
        kk, vv = ho.dkdv_at(keys)
        ksel = (0, keys[:, 0], keys[:, 1], keys[:, 2], e)
        assert np.abs(kk - dk[ksel]).max() < 1e-12 and np.abs(vv - dv[ksel]).max() < 1e-12
        assert np.array_equal(rows_at(x["q"], 0, e, pos), to_np(x["q"])[sel])
    # the fixed window (no offsets tensor): the queries reaching a key are its window's
    wlf = synth.Workload("fixed-crop", 1, 5, 7, 9, 2, 32, (3, 7, 7), (1, 1, 1), "f32", "none", backward=True)
    xf = synth.make_inputs(wlf, "cpu", seed=6)
    zeros = np.zeros((1, 5, 7, 9, 2, wlf.P, 3))
    _, dkf, dvf, _ = oracle.backward(to_np(xf["q"]), to_np(xf["k"]), to_np(xf["v"]), zeros, to_np(xf["dout"]),
                                     wlf.window, wlf.dilation)
    ho = HeadOracle(wlf, xf, 0, 1, None, xf["dout"])
    keys = grid_corner_tokens(5, 7, 9)
    kk, vv = ho.dkdv_at(keys)
    ksel = (0, keys[:, 0], keys[:, 1], keys[:, 2], 1)
    assert np.abs(kk - dkf[ksel]).max() < 1e-12 and np.abs(vv - dvf[ksel]).max() < 1e-12
