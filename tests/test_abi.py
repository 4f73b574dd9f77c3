"""The C ABI of libdsa3d on the host: exports, validation and workspace sizing.

No kernel is launched here; these run without a GPU.
"""
import os
import re
import subprocess

import pytest
import torch

import deformable_local_attention_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa3d.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(dsa3d_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert len(declared) == 24, declared
    out = subprocess.run(["nm", "-D", "--defined-only", dsa.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (dsa3d_\w+)", out))
    assert set(declared) <= exported, set(declared) - exported
    assert set(dsa.EXPORTS) == set(declared)
    L = dsa.lib()
    for name in declared:
        assert getattr(L, name) is not None


def test_descriptor_layout_matches_header():
    # int64 x4, int32 x10, float, int32 -> 80 bytes with 8-byte alignment
    import ctypes
    assert ctypes.sizeof(dsa.Desc) == 80
    fields = [f[0] for f in dsa.Desc._fields_]
    text = open(HEADER).read()
    body = text[text.index("typedef struct dsa3d_desc"):text.index("} dsa3d_desc;")]
    in_header = re.findall(r"\b(\w+)\s*[,;]", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
    assert fields == in_header


def _desc(**kw):
    base = dict(B=1, T=4, H=8, W=8, heads=2, head_dim=32, window=(3, 3, 3), dilation=(1, 1, 1),
                dtype=torch.float32)
    base.update(kw)
    return dsa.make_desc(base["B"], base["T"], base["H"], base["W"], base["heads"], base["head_dim"],
                         base["window"], base["dilation"], base["dtype"])


OK, INVALID, UNSUPPORTED = 0, -1, -2


@pytest.mark.parametrize("kw,expect", [
    ({}, OK),
    ({"window": (3, 5, 5)}, OK),
    ({"window": (1, 1, 1)}, OK),
    ({"dtype": torch.bfloat16, "head_dim": 128, "heads": 24}, OK),
    ({"head_dim": 8}, OK), ({"head_dim": 256}, OK),
    ({"window": (2, 3, 3)}, INVALID),        # even window
    ({"window": (3, 3, 0)}, INVALID),
    ({"dilation": (0, 1, 1)}, INVALID),
    ({"B": 0}, INVALID), ({"T": -1}, INVALID),
    ({"heads": 0}, INVALID),
    ({"head_dim": 48}, UNSUPPORTED),         # not a power of two
    ({"head_dim": 512}, UNSUPPORTED),
    ({"head_dim": 4}, UNSUPPORTED),
    ({"dtype": torch.float16}, UNSUPPORTED),
    ({"window": (11, 11, 11)}, UNSUPPORTED), # P = 1331 > 1024
    ({"B": 1, "T": 2048, "H": 2048, "W": 1024}, INVALID),  # 2^32 tokens
])
def test_validate(kw, expect):
    assert dsa.dsa3d_validate(_desc(**kw)) == expect


def test_validate_rejects_p_mismatch_and_bad_flags():
    d = _desc()
    d.P = 26
    assert dsa.dsa3d_validate(d) == INVALID
    d = _desc()
    d.deterministic = 2
    assert dsa.dsa3d_validate(d) == INVALID
    d = _desc()
    d.scale = -1.0
    assert dsa.dsa3d_validate(d) == INVALID
    d = _desc()
    d.scale = float("nan")
    assert dsa.dsa3d_validate(d) == INVALID


def _bwd_bounds(B, T, H, W, P, nh):
    """Bounds on the backward workspace of a pass over nh heads: a 32-byte
    record per sample, two 4-byte words per base cell (count and start) of the
    grid extended by one cell per axis, plus small scan and queue buffers and
    256-byte alignment."""
    nsamp = nh * B * T * H * W * P
    ncell = nh * B * (T + 1) * (H + 1) * (W + 1)
    lo = nsamp * 32 + ncell * 8
    return lo, lo + nsamp // 513 * 4 + ncell // 4096 * 4 + 8 * 256 + 64


def test_workspace_sizes():
    d = _desc()  # B=1, 4x8x8, 2 heads x 32, 3x3x3
    assert dsa.dsa3d_workspace_size(d, dsa.WS_FORWARD) == 0
    one = dsa.dsa3d_workspace_min(d, dsa.WS_BACKWARD)
    lo, hi = _bwd_bounds(1, 4, 8, 8, 27, 1)
    assert lo <= one <= hi
    lo2, hi2 = _bwd_bounds(1, 4, 8, 8, 27, 2)
    assert lo2 <= dsa.dsa3d_workspace_size(d, dsa.WS_BACKWARD) <= hi2
    # the accumulation mode does not change the workspace
    d.deterministic = 1
    assert dsa.dsa3d_workspace_min(d, dsa.WS_BACKWARD) == one
    # 1080p, 24 x 128, 3x5x5: one head needs ~5.0 GB; the recommended size
    # takes as many heads as fit in 16 GiB
    big = dsa.make_desc(1, 256, 68, 120, 24, 128, (3, 5, 5), dtype=torch.bfloat16, deterministic=True)
    ph = dsa.dsa3d_workspace_min(big, dsa.WS_BACKWARD)
    lo, hi = _bwd_bounds(1, 256, 68, 120, 75, 1)
    assert lo <= ph <= hi
    rec = dsa.dsa3d_workspace_size(big, dsa.WS_BACKWARD)
    assert rec <= (16 << 30) < rec + ph
    assert dsa.dsa3d_workspace_size(dsa.make_desc(1, 1, 1, 1, 1, 8, (1, 1, 1), dtype=torch.bfloat16),
                                    dsa.WS_PROJ_BACKWARD) > 0
    # depthwise convolution backward: float32 partials of 27 taps plus the bias per channel and row group
    conv = dsa.make_desc(1, 256, 68, 120, 24, 128, (3, 3, 3), dtype=torch.bfloat16)
    cw = dsa.dsa3d_workspace_size(conv, dsa.WS_DWCONV_BACKWARD)
    assert 28 * 3072 * 4 <= cw <= 28 * 3072 * 4 * (256 * 68) + 1024
    assert dsa.dsa3d_workspace_size(conv, 7) == 0
    # sized for either split of the weight-gradient sums (the path depends on the input's alignment):
    # 720p, 1024 channels: 480 groups of six rows against 6 x 5 tiles x 4 runs of 16 frames = 120
    c720 = dsa.make_desc(1, 64, 45, 80, 16, 64, (3, 3, 3), dtype=torch.bfloat16)
    assert dsa.dsa3d_workspace_size(c720, dsa.WS_DWCONV_BACKWARD) == 480 * 1024 * 27 * 4 + 480 * 1024 * 4 + 512
    # one 512 x 512 frame of 64 channels: 64 x 32 tiles of 8 x 16 tokens outnumber the 512 row groups
    wide = dsa.make_desc(1, 1, 512, 512, 1, 64, (3, 3, 3), dtype=torch.bfloat16)
    assert dsa.dsa3d_workspace_size(wide, dsa.WS_DWCONV_BACKWARD) == 2048 * 64 * 27 * 4 + 2048 * 64 * 4 + 512
    # the fixed-window backward keeps one float per (token, head)
    assert dsa.dsa3d_workspace_size(conv, dsa.WS_BACKWARD_FIXED) == 256 * 68 * 120 * 24 * 8 + 256
    bad = _desc(window=(2, 2, 2))
    assert dsa.dsa3d_workspace_size(bad, dsa.WS_BACKWARD) == 0
    # one head with 2^30 tokens x 27 samples cannot be numbered in 32 bits
    huge = dsa.make_desc(1, 1024, 1024, 1024, 1, 8, (3, 3, 3), dtype=torch.bfloat16)
    assert dsa.dsa3d_validate(huge) == 0
    assert dsa.dsa3d_workspace_min(huge, dsa.WS_BACKWARD) == 0
    assert dsa.dsa3d_workspace_size(huge, dsa.WS_BACKWARD) == 0


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert dsa.dsa3d_status_string(s)
    assert dsa.dsa3d_status_string(-99) == "unknown status"
    assert dsa.dsa3d_version() >= 100


def test_binding_has_no_cpu_fallback(monkeypatch, tmp_path):
    # a missing library is an error, never a silent substitute
    import importlib
    monkeypatch.setenv("DSA3D_LIBRARY", str(tmp_path / "missing.so"))
    mod = importlib.reload(dsa)
    try:
        with pytest.raises(ImportError):
            mod.lib()
    finally:
        monkeypatch.delenv("DSA3D_LIBRARY")
        importlib.reload(dsa)


def test_product_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "deformable_local_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower() or f == "synth.py" and "import oracle" not in text, f


def _cpu_tensors(dtype=torch.bfloat16, B=1, T=2, H=3, W=4, heads=2, d=16, window=(3, 3, 3)):
    P = window[0] * window[1] * window[2]
    act = lambda: torch.zeros((B, T, H, W, heads, d), dtype=dtype)
    return dict(desc=dsa.make_desc(B, T, H, W, heads, d, window, dtype=dtype), q=act(), k=act(), v=act(),
                off=torch.zeros((B, T, H, W, heads, P, 3), dtype=dtype), out=act(),
                lse=torch.zeros((B, T, H, W, heads), dtype=torch.float32))


@pytest.mark.parametrize("bad,match", [
    ("k_dtype", "dtype"),          # f32 keys in a bf16 run
    ("off_dtype", "dtype"),        # f32 offsets in a bf16 run
    ("lse_dtype", "dtype"),        # bf16 lse (always float32)
    ("k_heads", "shape"),          # keys with fewer heads
    ("off_points", "shape"),       # offsets built for another P
    ("out_small", "shape"),        # an output with fewer elements
    ("not_contiguous", "contiguous"),
    ("cpu", "GPU"),                # host tensors of the right type and shape
])
def test_binding_rejects_mismatched_tensors_before_the_library(bad, match):
    """The binding checks every tensor against the descriptor (type, size,
    contiguity, device) and raises before any pointer reaches libdsa3d: a
    wrong tensor is an error, never an out-of-bounds device access."""
    t = _cpu_tensors()
    if bad == "k_dtype":
        t["k"] = t["k"].float()
    elif bad == "off_dtype":
        t["off"] = t["off"].float()
    elif bad == "lse_dtype":
        t["lse"] = t["lse"].bfloat16()
    elif bad == "k_heads":
        t["k"] = t["k"][:, :, :, :, :1].contiguous()
    elif bad == "off_points":
        t["off"] = torch.zeros(t["off"].shape[:5] + (26, 3), dtype=torch.bfloat16)
    elif bad == "out_small":
        t["out"] = t["out"].reshape(-1)[:-8].clone()
    elif bad == "not_contiguous":
        t["q"] = t["q"].transpose(4, 5).contiguous().transpose(4, 5)
    with pytest.raises(ValueError, match=match):
        dsa.dsa3d_forward(t["desc"], t["q"], t["k"], t["v"], t["off"], t["out"], t["lse"])


def test_binding_checks_backward_and_projection_tensors():
    t = _cpu_tensors()
    d = t["desc"]
    act = lambda: torch.zeros_like(t["q"])
    with pytest.raises(ValueError, match="dk"):
        dsa.dsa3d_backward(d, t["q"], t["k"], t["v"], t["off"], t["out"], t["lse"], act(), act(),
                           torch.zeros(5, dtype=torch.bfloat16), act(), torch.zeros_like(t["off"]), None)
    with pytest.raises(ValueError, match="dw"):
        F, C = 2 * 27 * 3, 2 * 16
        dsa.dsa3d_offset_proj_backward(d, t["q"], torch.zeros((F, C), dtype=torch.bfloat16), t["off"], act(),
                                       torch.zeros((F, C), dtype=torch.bfloat16), None, None)
    with pytest.raises(ValueError, match="wt"):
        dsa.dsa3d_dwconv_forward(d, t["q"], torch.zeros((32, 3, 3), dtype=torch.bfloat16), None, act())
    with pytest.raises(TypeError):
        dsa.dsa3d_forward(d, t["q"], t["k"], t["v"], t["off"], t["out"], [0.0])


def test_noalloc_backward_rejects_problems_beyond_its_scratch_on_the_host():
    """dsa3d_backward_noalloc checks the problem against its fixed 64 MiB
    scratch array before it touches the GPU: the 1080p 3x5x5 problem (about
    5 GB per head) is refused with DSA3D_ERR_WORKSPACE, an invalid
    descriptor with its own error."""
    import ctypes
    big = dsa.make_desc(1, 256, 68, 120, 24, 128, (3, 5, 5), dtype=torch.bfloat16, deterministic=True)
    assert dsa.dsa3d_workspace_min(big, dsa.WS_BACKWARD) > dsa.NOALLOC_SCRATCH_BYTES
    L = dsa.lib()
    nul = [None] * 12
    assert L.dsa3d_backward_noalloc(ctypes.byref(big), *nul) == -4  # DSA3D_ERR_WORKSPACE
    assert L.dsa3d_backward_noalloc(ctypes.byref(_desc(window=(2, 3, 3))), *nul) == INVALID
    fixed = dsa.make_desc(1, 256, 68, 120, 24, 128, (3, 7, 7), dtype=torch.bfloat16)
    assert dsa.dsa3d_workspace_min(fixed, dsa.WS_BACKWARD_FIXED) > dsa.NOALLOC_SCRATCH_BYTES
    assert L.dsa3d_backward_noalloc(ctypes.byref(fixed), *nul) == -4
    assert dsa.NOALLOC_SCRATCH_BYTES == 64 << 20
    text = open(HEADER).read()
    assert "#define DSA3D_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
