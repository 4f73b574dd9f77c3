"""The sampled-oracle helpers used by the full-size GPU parity tests agree
with the whole-grid oracle (CPU tensors stand in for device tensors)."""
import numpy as np

import oracle
from deformable_local_attention_amd import synth
from gpu_helpers import gather, oracle_dkdv_at_keys, oracle_queries, sample_queries, to_np


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
