#!/usr/bin/env python
"""3D-DSA fwd+bwd throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--cpu-baseline on|off]

One step is one pass of the whole hot path over one batch of synthetic input
(the 256x68x120-token grid, 24 heads x 128, 3x5x5 window, offsets N(0,2),
deterministic K/V gradients by default): forward then backward, every kernel
included. Inputs are drawn on the GPU (seed 0) and are resident in HBM before
the timed region starts. Prints one JSON line on stdout; progress goes to
stderr.

`roofline` is taken for the attention kernel with the largest share of the
timed region, timed per launch with HIP events that libdsa3d records around
each of its launches (dsa3d_set_launch_log) on the launch stream. That kernel
is bound by vector-ALU work, so `roofline` is its algorithmic flops of one
launch over its mean launch duration against the vector fp32 peak;
`roofline_hbm` is the same launch's algorithmic bytes (each tensor read or
written once; sampled K/V rows are never counted) against the HBM peak, and
`roofline_step` the whole step's flops against the vector peak.
`roofline_gather` gives each attention kernel's gathered corner-row bytes
against the vector-L1 load rate, the limit those kernels actually meet.

`--copy-calibration` instead runs a plain device copy of a known size, whose
rocprofv3 FETCH_SIZE / WRITE_SIZE readings scale the counters of the kernels.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
VALU_F32_PEAK_TFLOPS = 157.3   # MI355X vector fp32: 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (packed) x 2.4 GHz
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published
L1_LOAD_PEAK_TBS = 39.3        # vector L1 loads, measured: 64 B/clock/CU x 256 CUs x 2.4 GHz
METRIC = "3D-DSA fwd+bwd tokens/sec at 256×68×120 tokens; achieved HBM GB/s vs peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(wl):
    """Algorithmic bytes and flops per (token, head), each tensor read or
    written once (sampled key/value rows are never counted: they are the
    gathers the fused kernels exist to avoid materialising).

    forward:   reads q, k, v (3d elements) and the offsets (3P), writes o (d)
               and lse (4 B); flops 32*d*P (per sample: 8 corner dot products
               of length d weighted into the logit, 8 weighted row updates).
    bwd_query: reads q, k, v, o, dO (5d), offsets (3P) and lse (4 B), writes
               dq (d) and doffsets (3P).
    bwd_key:   reads q and dO (2d), writes dk and dv (2d).
    The whole backward is then 8d + 6P elements + 4 B, flops 80*d*P: per
    sample 48*d in the query kernel (logit, <dO, V[c]> and the dq update over
    8 corners) and 32*d in the key kernel (the dK and dV updates of 8 corners).
    Keys "<kernel>_flops" give the flops per (token, head) of each kernel.
    """
    s = 4 if wl.dtype == "f32" else 2
    d, P = wl.head_dim, wl.P
    if wl.offsets == "none":
        # fixed window (no offsets): forward reads q, k, v, writes o and lse;
        # flops 4*d*P (one dot product and one row update per sample). Backward
        # per query reads q, k, v, o, dO and lse, writes dq and <dO,o> (4 B);
        # per key reads k, v, lse and <dO,o> of its queries (8 B), writes dk, dv;
        # flops 10*d*P (logit, dL/da, dq, dk and dv per sample).
        return {
            "forward": 4 * d * s + 4,
            "bwd_query": 6 * d * s + 8,
            "bwd_key": 4 * d * s + 8,
            "fwd_bytes": 4 * d * s + 4,
            "bwd_bytes": 8 * d * s + 8,
            "fwd_flops": 4 * d * P,
            "bwd_flops": 10 * d * P,
            "forward_flops": 4 * d * P,
            "bwd_query_flops": 6 * d * P,
            "bwd_key_flops": 4 * d * P,
        }
    return {
        "forward": 4 * d * s + 3 * P * s + 4,
        "bwd_query": 6 * d * s + 6 * P * s + 4,
        "bwd_key": 4 * d * s,
        "fwd_bytes": 4 * d * s + 3 * P * s + 4,
        "bwd_bytes": 8 * d * s + 6 * P * s + 4,
        "fwd_flops": 32 * d * P,
        "bwd_flops": 80 * d * P,
        "forward_flops": 32 * d * P,
        "bwd_query_flops": 48 * d * P,
        "bwd_key_flops": 32 * d * P,
    }


def fixed_on_mfma(wl):
    """Rows per wave of the fixed window's matrix-core kernels, per kernel, or
    None where libdsa3d runs the fixed window on the vector units: bf16 rows of
    32-256 channels (32-128 for the backward), no dilation along w, k_w <= 17,
    a grid row of all heads below 2 GiB; two rows per wave when h is not
    dilated and rows have at most 128 channels (64 for the key kernel)."""
    d = wl.head_dim
    if wl.offsets != "none" or wl.dtype != "bf16" or d not in (32, 64, 128, 256) or wl.dilation[2] != 1 \
            or wl.window[2] > 17 or wl.W * wl.heads * d * 2 > 2**31 - 1:
        return None
    und = wl.dilation[1] == 1
    rows = {"forward": 2 if und and d <= 128 else 1}
    if d <= 128:
        rows["bwd_query"] = 2 if und else 1
        rows["bwd_key"] = 2 if und and d <= 64 else 1
    return rows


def host_cpu():
    """(usable cores, cores the OS reports, CPU model) of this host."""
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return usable, os.cpu_count() or 1, model


def cpu_baseline_block(wl, budget_s: float = 20.0):
    """The oracle's transformer block (float64 numpy and the attention oracle,
    one head per thread) forward and backward on a bounded crop of the block
    workload: 4 frames of 12 x 12 tokens with the workload's channels, heads
    and window. Returns whole tokens per second."""
    import numpy as np

    import oracle
    from deformable_local_attention_amd import synth

    usable, nproc, model = host_cpu()
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    cores = max(1, min(usable, share) if share > 0 else usable)
    crop = wl.with_grid(B=1, T=min(wl.T, 4), H=min(wl.H, 12), W=min(wl.W, 12), name=wl.name + "-crop")
    x = synth.make_inputs(crop, "cpu", seed=0)
    f64 = lambda t: t.double().numpy()
    p = {"ln_g": f64(x["ln_g"]), "ln_b": f64(x["ln_b"]), "w_qkv": f64(x["w_qkv"]), "b_qkv": f64(x["b_qkv"]),
         "w_off": f64(x["proj_w"]), "b_off": f64(x["proj_b"]), "w_out": f64(x["w_out"]), "b_out": f64(x["b_out"])}
    xx, dy = f64(x["x"]), f64(x["dout"])

    def one_pass():
        t0 = time.perf_counter()
        oracle.block_backward(xx, p, dy, crop.heads, crop.window, crop.dilation, crop.ln_eps)
        return time.perf_counter() - t0

    dt1 = one_pass()
    reps = max(1, int(math.ceil((budget_s - dt1) / dt1)))
    dt = sum(one_pass() for _ in range(reps))
    return {"value": crop.tokens * reps / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "host": {"usable_cores": usable, "nproc": nproc, "omp_num_threads": share or None, "cpu_model": model},
            "sample": (f"float64 oracle block (layer norm, projections, attention forward and backward) on a "
                       f"{crop.T}x{crop.H}x{crop.W}-token crop with {crop.heads} heads x {crop.head_dim}; {reps} "
                       f"passes in {dt:.1f} s (the backward recomputes the forward); the attention runs one head per "
                       f"thread, numpy's products on its own threads")}


def cpu_baseline(wl, budget_s: float = 20.0):
    """The oracle, as it is, on a bounded sample of the same workload: the
    interior queries of a 16x24x24-token crop drawn with the workload's
    distributions, one head per usable host core (heads are independent and
    run in parallel, one thread each). Returns tokens/s for whole tokens (all
    heads), scaled from the heads sampled."""
    import numpy as np

    import oracle
    from deformable_local_attention_amd import synth

    usable, nproc, model = host_cpu()
    # the CPU share granted to this process: OMP_NUM_THREADS where the host
    # sets it (a GPU job's share of a shared host), else every usable core
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    cores = max(1, min(usable, share) if share > 0 else usable)
    crop = wl.with_grid(B=1, T=min(wl.T, 16), H=min(wl.H, 24), W=min(wl.W, 24), heads=cores, name=wl.name + "-crop")
    x = synth.make_inputs(crop, "cpu", seed=0, with_grad=True)
    if crop.offsets in ("proj", "conv"):
        q2 = x["q"].double().numpy().reshape(crop.tokens, crop.C)
        if crop.offsets == "conv":
            q5 = q2.reshape(crop.B, crop.T, crop.H, crop.W, crop.C)
            q2 = oracle.dwconv3d(q5, x["conv_w"].double().numpy(), None).reshape(crop.tokens, crop.C)
        off = oracle.offset_proj(q2, x["proj_w"].double().numpy(), None).astype(np.float32)
        off = off.reshape(crop.B, crop.T, crop.H, crop.W, crop.heads, crop.P, 3)
    else:
        off = (x["offsets"].float().numpy() if crop.offsets == "direct"
               else np.zeros((crop.B, crop.T, crop.H, crop.W, crop.heads, crop.P, 3), dtype=np.float32))
    np64 = lambda t: t.double().numpy()
    q, k, v, g = np64(x["q"]), np64(x["k"]), np64(x["v"]), np64(x["dout"])
    T, H, W = crop.T, crop.H, crop.W
    m = [min(4, T // 4), min(8, H // 4), min(8, W // 4)]
    pos = oracle.grid_positions(T, H, W)
    interior = np.all((pos >= m) & (pos < np.array([T, H, W]) - m), axis=1)
    pos = pos[interior]
    scale = 1.0 / np.sqrt(crop.head_dim)

    def one_pass():
        from concurrent.futures import ThreadPoolExecutor

        def one(h):
            qq = q[0][pos[:, 0], pos[:, 1], pos[:, 2], h]
            oo = off[0][pos[:, 0], pos[:, 1], pos[:, 2], h]
            oracle.forward_queries((T, H, W), crop.window, crop.dilation, scale, pos, qq, oo, (0, 0, 0),
                                   k[0, :, :, :, h], v[0, :, :, :, h])
            if crop.backward:
                gg = g[0][pos[:, 0], pos[:, 1], pos[:, 2], h]
                oracle.backward_queries((T, H, W), crop.window, crop.dilation, scale, pos, qq, oo, (0, 0, 0),
                                        k[0, :, :, :, h], v[0, :, :, :, h], gg)

        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=cores) as ex:
            list(ex.map(one, range(cores)))
        return time.perf_counter() - t0

    dt1 = one_pass()
    reps = max(1, int(math.ceil((budget_s - dt1) / dt1)))
    dt = sum(one_pass() for _ in range(reps))
    n = len(pos) * reps
    token_heads_per_s = n * cores / dt
    return {"value": token_heads_per_s / wl.heads, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "host": {"usable_cores": usable, "nproc": nproc, "omp_num_threads": share or None, "cpu_model": model},
            "sample": (f"fp64 oracle, {'fwd+bwd' if crop.backward else 'fwd'}: the {len(pos)} interior queries of a "
                       f"{T}x{H}x{W}-token crop (the workload's window, dilation and input distributions), "
                       f"{cores} heads in parallel, {reps} passes, {dt:.1f} s on {cores} threads; tokens/s counts "
                       f"whole tokens ({wl.heads} heads)")}


# the sources the attention kernels (forward, backward per query and per key)
# are compiled from
ATTN_SOURCES = ("dsa3d_attn.hip", "dsa3d_bwd.hip", "dsa3d_attn_common.h", "dsa3d_device.h", "dsa3d_internal.h")


def code_text(src: str) -> str:
    """A source's code without its comments and with whitespace collapsed."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash(read=None) -> str:
    """sha256 over the attention kernels' code (comments and layout do not
    count): counter readings taken on other code no longer describe the
    kernels."""
    import hashlib
    pkg = os.path.join(ROOT, "deformable_local_attention_amd", "csrc")
    if read is None:
        read = lambda name: open(os.path.join(pkg, name)).read()
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        h.update(f.encode())
        h.update(code_text(read(f)).encode())
    return h.hexdigest()[:16]


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# What `traffic` counts: the bytes a launch moves beyond the L2 caches (rocprofv3 FETCH_SIZE + WRITE_SIZE, each
# scaled by its reading for a plain device copy of known size), which includes hits in the memory-side cache,
# so it is an upper bound on the HBM bytes.
TRAFFIC_SCOPE = "beyond-L2 bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated; includes memory-side cache hits)"


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none for this kernel and workload or the kernel sources
    changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k["hbm_bytes_per_launch"]


def _short_kernel(name: str) -> str:
    import re
    n = re.sub(r"\(.*", "", name).replace("void ", "")
    n = n.replace("dsa3d::dsa3d_", "")
    return n


def pmc_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, workload, out_json=None):
    """Per-kernel HBM traffic from rocprofv3 counter CSVs (FETCH_SIZE and
    WRITE_SIZE, KiB per dispatch). Each counter is scaled by what it reads for
    a plain device copy of known size (copy_calibration: 4 GiB read and 4 GiB
    written per launch)."""
    import csv
    import collections

    def per_kernel(path, counter):
        acc = collections.defaultdict(list)
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == counter:
                    acc[_short_kernel(row["Kernel_Name"])].append(float(row["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    copy_bytes = 4 * (1 << 30)
    cf = per_kernel(copy_fetch_csv, "FETCH_SIZE")
    cw = per_kernel(copy_write_csv, "WRITE_SIZE")
    ck = [k for k in cf if "copyBuffer" in k][0]
    f_fac = copy_bytes / (cf[ck] * 1024.0)
    w_fac = copy_bytes / (cw[ck] * 1024.0)
    fk = per_kernel(fetch_csv, "FETCH_SIZE")
    wk = per_kernel(write_csv, "WRITE_SIZE")
    kernels = {}
    for k in sorted(fk):
        if k not in wk:
            continue
        rd = fk[k] * 1024.0 * f_fac
        wr = wk[k] * 1024.0 * w_fac
        kernels[k] = {"fetch_kib_per_dispatch": round(fk[k], 1), "write_kib_per_dispatch": round(wk[k], 1),
                      "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
                      "hbm_bytes_per_launch": rd + wr}
    rec = {"workload": workload, "source_hash": kernel_source_hash(), "fetch_factor": round(f_fac, 4),
           "write_factor": round(w_fac, 4), "copy_kernel": ck, "kernels": kernels}
    for k, v in kernels.items():
        if k.startswith(("fwd_kernel", "bwd_", "sort_", "gemm")):
            print(f"{k:40s} read {v['hbm_read_bytes_per_launch'] / 1e9:9.3f} GB  "
                  f"write {v['hbm_write_bytes_per_launch'] / 1e9:9.3f} GB per launch")
    print(f"scale factors from the copy: FETCH_SIZE x{f_fac:.3f}, WRITE_SIZE x{w_fac:.3f}")
    if out_json:
        with open(out_json, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    return rec


def copy_calibration(gib: float = 4.0, reps: int = 5):
    import torch
    n = int(gib * (1 << 30)) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "ms": dt * 1e3,
                      "gbs": 2 * n * 4 / dt / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--fast", action="store_true", help="float32 (non-deterministic) K/V-gradient accumulation")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--alt-steps", type=int, default=2,
                    help="steps timed again with deterministic=0 after a deterministic run (0: none)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="summarise rocprofv3 FETCH_SIZE/WRITE_SIZE counter CSVs into HBM bytes per launch")
    ap.add_argument("--pmc-json", default=None, help="with --pmc-summary: write the summary to this JSON file")
    args = ap.parse_args()

    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, workload=args.workload or "1080p-bf16-p75-det", out_json=args.pmc_json)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the 3D-DSA path here runs on a single MI355X "
              "(multi-GPU sharding is not built). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import deformable_local_attention_amd as dsa
    from deformable_local_attention_amd import synth
    from deformable_local_attention_amd.chain import make_chain

    if args.copy_calibration:
        copy_calibration()
        return

    wl = synth.WORKLOADS[args.workload or synth.HEADLINE]
    if args.fast:
        import dataclasses
        wl = dataclasses.replace(wl, deterministic=False)
    log(f"[bench] {synth.describe(wl)}; steps={args.steps} warmup={args.warmup}")
    t0 = time.perf_counter()
    x = synth.make_inputs(wl, "cuda:0", seed=0)
    ch = make_chain(wl, x)
    torch.cuda.synchronize()
    log(f"[bench] inputs drawn and buffers allocated in {time.perf_counter() - t0:.1f} s; "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB on the device")

    for i in range(args.warmup):
        ch.run()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")

    stream = torch.cuda.current_stream()
    timer = dsa.launch_timer(capacity=max(256, 160 * args.steps))
    torch.cuda.synchronize()
    with timer:
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t_wall = time.perf_counter()
        ev0.record(stream)
        for i in range(args.steps):
            ch.run()
        ev1.record(stream)
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    tokens_per_s = wl.tokens * args.steps / (ms_total / 1e3)
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.2f} ms/step (wall {t_wall:.2f} s), "
        f"{tokens_per_s / 1e6:.3f} M tokens/s")

    durs = timer.durations_ms()
    if timer.count >= timer.log.capacity:
        log("[bench] warning: launch log full; per-kernel figures cover the first launches only")
    per_kernel = {k: {"launches": len(v), "mean_ms": sum(v) / len(v), "total_ms": sum(v)} for k, v in durs.items()}
    for k, v in sorted(per_kernel.items(), key=lambda kv: -kv[1]["total_ms"]):
        log(f"[bench]   {k:14s} {v['launches']:4d} launches, mean {v['mean_ms']:.3f} ms, total {v['total_ms']:.1f} ms")

    alg = algorithmic(wl)
    attn = [k for k in per_kernel if k in ("forward", "bwd_query", "bwd_key")]
    dom = max(attn, key=lambda k: per_kernel[k]["total_ms"])
    # the backward runs in passes over ranges of heads: a launch covers, on
    # average, (all (token, head) units of the timed steps) / (its launches)
    units = wl.tokens * wl.heads * args.steps / per_kernel[dom]["launches"]
    mean_s = per_kernel[dom]["mean_ms"] / 1e3
    unit_bytes = alg[dom]
    achieved_gbs = unit_bytes * units / mean_s / 1e9
    kname = {"forward": "fwd_kernel<unsigned short, %d>", "bwd_query": "bwd_query_kernel<unsigned short, %d>",
             "bwd_key": "bwd_key_kernel<unsigned short, %d>"}[dom] % wl.head_dim
    if wl.dtype == "f32":
        kname = kname.replace("unsigned short", "float")
    traffic = recorded_traffic(kname, wl.name)
    unit_flops = alg[dom + "_flops"]
    achieved_tf = unit_flops * units / mean_s / 1e12
    mf_rows = fixed_on_mfma(wl)
    on_mfma = mf_rows is not None and dom in mf_rows  # the fixed window's matrix-core kernels
    peak = MFMA_BF16_PEAK_TFLOPS if on_mfma else VALU_F32_PEAK_TFLOPS
    roofline = {"bound": "mfma" if on_mfma else "alu", "kernel": dom, "achieved": round(achieved_tf, 3),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved_tf / peak, 5),
                "traffic": None if traffic is None else round(traffic), "traffic_scope": TRAFFIC_SCOPE,
                "launch_ms": round(per_kernel[dom]["mean_ms"], 3), "units_per_launch": units,
                "flops_per_unit": unit_flops}
    roofline_hbm = {"bound": "hbm", "kernel": dom, "achieved": round(achieved_gbs, 2), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 5),
                    "traffic": None if traffic is None else round(traffic), "traffic_scope": TRAFFIC_SCOPE,
                    "launch_ms": round(per_kernel[dom]["mean_ms"], 3), "units_per_launch": units,
                    "bytes_per_unit": unit_bytes}
    step_flops = wl.tokens * wl.heads * (alg["fwd_flops"] + (alg["bwd_flops"] if wl.backward else 0))
    roofline_step = {"bound": "alu", "scope": "whole step",
                     "achieved": round(step_flops / (ms_per_step / 1e3) / 1e12, 3), "peak": VALU_F32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(step_flops / (ms_per_step / 1e3) / 1e12 / VALU_F32_PEAK_TFLOPS, 5),
                     "flops_per_token": step_flops // wl.tokens}

    # The whole step's algorithmic bytes (each attention tensor read or written once: forward and backward
    # per (token, head) as above) over the step time, against the HBM peak: the metric's "achieved HBM GB/s".
    step_bytes = wl.tokens * wl.heads * (alg["fwd_bytes"] + (alg["bwd_bytes"] if wl.backward else 0))
    step_gbs = step_bytes / (ms_per_step / 1e3) / 1e9
    roofline_hbm_step = {"bound": "hbm", "scope": "whole step, attention tensors", "achieved": round(step_gbs, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(step_gbs / HBM_PEAK_GBS, 5),
                         "bytes_per_step": step_bytes}

    # The gathers: in the forward and the query kernel every sample reads the head's rows of its 8 corner
    # tokens in two tensors (keys and values), 16*d*s*P bytes per (token, head). The key kernel reads the
    # query and output-gradient rows of each record once per 2x2 group of keys it reaches, 4.5 groups per
    # sample on average (18 buckets per group of 4 keys instead of 8 per key): 9*d*s*P. The fixed window
    # reads 2 rows per window column, shared by the 4 tokens of a task along w when w is not dilated:
    # 2 * (4 + k_w - 1) / (4 * k_w) rows per sample; its matrix-core kernels load, per wave of R rows of
    # 16 tokens, two tensors' rows of 32 tokens for each of the k_t * (k_h + R - 1) segments of the union
    # of their windows. These bytes pass through each CU's vector L1 and its
    # texture-data path, which rocprofv3 shows 98-99% busy in all three kernels; the ceiling is the L1
    # load rate measured with a probe kernel streaming 16-byte loads from an L1-resident buffer,
    # 64 B per clock per CU (256 CUs at 2.4 GHz).
    s_el = 4 if wl.dtype == "f32" else 2
    rows_per_sample = {"forward": 16, "bwd_query": 16, "bwd_key": 9}
    roofline_gather = {}
    for k in attn:
        if mf_rows is not None and k in mf_rows:
            r = mf_rows[k]
            gather_unit = wl.window[0] * (wl.window[1] + r - 1) * 2 * 32 * wl.head_dim * s_el / (16 * r)
        else:
            if wl.offsets == "none":
                kw = wl.window[2]
                rows = 2.0 * (4 + kw - 1) / (4 * kw) if wl.dilation[2] == 1 else 2.0
            else:
                rows = rows_per_sample[k]
            gather_unit = rows * wl.head_dim * s_el * wl.P
        u = wl.tokens * wl.heads * args.steps / per_kernel[k]["launches"]
        tbs = gather_unit * u / (per_kernel[k]["mean_ms"] / 1e3) / 1e12
        roofline_gather[k] = {"bound": "l1", "achieved": round(tbs, 2), "peak": L1_LOAD_PEAK_TBS, "unit": "TB/s",
                              "frac": round(tbs / L1_LOAD_PEAK_TBS, 4), "bytes_per_unit": gather_unit}

    # the projection GEMMs (workloads whose offsets come from the Linear): MFMA-bound
    roofline_proj = None
    if wl.offsets in ("proj", "conv"):
        gemm_flops = 2.0 * wl.tokens * wl.C * wl.F  # one product of the projection
        roofline_proj = {}
        for k in ("proj_forward", "proj_bwd_dq", "proj_bwd_dw"):
            if k in per_kernel:
                tf = gemm_flops / (per_kernel[k]["mean_ms"] / 1e3) / 1e12
                roofline_proj[k] = {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                                    "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                    "launch_ms": round(per_kernel[k]["mean_ms"], 3),
                                    "flops_per_launch": gemm_flops}

    # the depthwise convolution of the "conv" offset network: HBM-bound, algorithmic bytes per token
    # forward 2Cs (q read, y written), dq 3Cs (dy read, dq read and written), weight sums 2Cs (q, dy read)
    # the transformer block's own kernels: the layer norm is HBM-bound (forward reads x and writes h, 2Cs per
    # token, plus 8 B of statistics; backward reads x, dy and the residual gradient and writes dx, 4Cs + 8 B),
    # the q/k/v and output projections are bf16 contractions of 2*C*C flops per token each (MFMA)
    roofline_block = None
    if wl.block:
        s_el = 4 if wl.dtype == "f32" else 2
        roofline_block = {}
        ln_bytes = {"layernorm": 2 * wl.C * s_el + 8, "layernorm_bwd": 4 * wl.C * s_el + 8}
        for k, per_tok in ln_bytes.items():
            if k in per_kernel:
                gbs = per_tok * wl.tokens / (per_kernel[k]["mean_ms"] / 1e3) / 1e9
                roofline_block[k] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                                     "launch_ms": round(per_kernel[k]["mean_ms"], 3)}
        lin_flops = 2.0 * wl.tokens * wl.C * wl.C  # one C x C projection
        for k in ("linear_forward", "linear_bwd_dx", "linear_bwd_dw"):
            if k in per_kernel:
                tf = lin_flops / (per_kernel[k]["mean_ms"] / 1e3) / 1e12
                roofline_block[k] = {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                     "launch_ms": round(per_kernel[k]["mean_ms"], 3), "flops_per_launch": lin_flops}

    # hybrid attention's global rows. bf16 rows of 32-128 channels run on the matrix cores, where the kernels
    # are HBM-bound: algorithmic bytes per (token, head) are, forward, q read, the local o read and the merged
    # o written, lse read and written (3*d*s + 8); query kernel, q, dO and o read, dq read and written, lse read
    # and <dO, o> written (5*d*s + 8); rows kernel, q and dO read, lse and <dO, o> read (2*d*s + 8) (the G
    # global rows themselves are negligible). Beside it, the bf16 products issued: forward S and the split-weight
    # O product (6*d*G flops per (token, head)), query kernel S, dP and the split dq product (8*d*G), rows kernel
    # S, dP and the split dGK, dGV products (12*d*G), against the bf16 matrix-core peak. Other rows run on the
    # vector units: 4*d*G, 6*d*G and 8*d*G flops against the vector ALU peak.
    roofline_hybrid = None
    if wl.global_tokens:
        G = wl.global_tokens
        roofline_hybrid = {}
        on_mfma = wl.dtype == "bf16" and wl.head_dim in (32, 64, 128)
        s_el = 4 if wl.dtype == "f32" else 2
        for k, per, nbytes, issued in (("hybrid_forward", 4, 3, 6), ("hybrid_bwd_query", 6, 5, 8),
                                       ("hybrid_bwd_rows", 8, 2, 12)):
            if k not in per_kernel:
                continue
            sec = per_kernel[k]["mean_ms"] / 1e3
            units = wl.tokens * wl.heads
            if on_mfma:
                per_unit = nbytes * wl.head_dim * s_el + 8
                gbs = per_unit * units / sec / 1e9
                tf = issued * wl.head_dim * G * units / sec / 1e12
                roofline_hybrid[k] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(gbs / HBM_PEAK_GBS, 4), "launch_ms": round(per_kernel[k]["mean_ms"], 3),
                                      "bytes_per_unit": per_unit,
                                      "mfma_issued": {"achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                                                      "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}}
            else:
                tf = per * wl.head_dim * G * units / sec / 1e12
                roofline_hybrid[k] = {"bound": "alu", "achieved": round(tf, 2), "peak": VALU_F32_PEAK_TFLOPS,
                                      "unit": "TFLOP/s", "frac": round(tf / VALU_F32_PEAK_TFLOPS, 4),
                                      "launch_ms": round(per_kernel[k]["mean_ms"], 3)}

    roofline_conv = None
    if wl.offsets == "conv":
        s_el = 4 if wl.dtype == "f32" else 2
        conv_bytes = {"dwconv": 2, "dwconv_dq": 3, "dwconv_wgrad": 2}
        roofline_conv = {}
        for k, m in conv_bytes.items():
            if k in per_kernel:
                gbs = m * wl.C * s_el * wl.tokens / (per_kernel[k]["mean_ms"] / 1e3) / 1e9
                roofline_conv[k] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": round(gbs / HBM_PEAK_GBS, 4), "launch_ms": round(per_kernel[k]["mean_ms"], 3),
                                    "bytes_per_launch": m * wl.C * s_el * wl.tokens}

    result = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": ("synthetic (seeded N(0,1) block input x and dO; random-init layer-norm, q/k/v and output "
                 "projection weights; offsets from a Linear with N(0,0.02) weights of q)") if wl.block else
        "synthetic (seeded N(0,1) q/k/v/dO; offsets "
        + (f"N(0,{wl.offset_sigma})" if wl.offsets == "direct" else "none: fixed window, every offset zero"
           if wl.offsets == "none" else "from a Linear with N(0,0.02) weights"
           + (" of a depthwise 3x3x3 conv with N(0,0.2) weights" if wl.offsets == "conv" else "")) + ")",
        "config": {"workload": wl.name, "grid": [wl.B, wl.T, wl.H, wl.W], "heads": wl.heads, "head_dim": wl.head_dim,
                   "window": list(wl.window), "P": wl.P, "dilation": list(wl.dilation), "offsets": wl.offsets,
                   **({"global_tokens": wl.global_tokens} if wl.global_tokens else {}),
                   "chain": ("layernorm+qkv+" if wl.block else "") + {"proj": "proj+", "conv": "dwconv+proj+"}.get(
                       wl.offsets, "") + ("fwd" if not wl.block else "fwd+out_proj+residual")
                       + ("+bwd" if wl.backward else ""),
                   "deterministic": wl.deterministic},
        "roofline": roofline, "roofline_hbm": roofline_hbm, "roofline_step": roofline_step,
        "roofline_hbm_step": roofline_hbm_step,
        "roofline_gather": roofline_gather,
        **({"roofline_proj": roofline_proj} if roofline_proj else {}),
        **({"roofline_conv": roofline_conv} if roofline_conv else {}),
        **({"roofline_block": roofline_block} if roofline_block else {}),
        **({"roofline_hybrid": roofline_hybrid} if roofline_hybrid else {}),
        "kernels": {k: {"launches": v["launches"], "mean_ms": round(v["mean_ms"], 3)} for k, v in per_kernel.items()},
    }
    if wl.backward and wl.deterministic and args.alt_steps > 0:
        # the same step with the fast (order-free) K/V-gradient accumulation, on the same buffers
        ch.desc.deterministic = 0
        ch.run()
        ev2, ev3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev2.record(stream)
        for _ in range(args.alt_steps):
            ch.run()
        ev3.record(stream)
        torch.cuda.synchronize()
        ch.desc.deterministic = 1
        ms_fast = ev2.elapsed_time(ev3) / args.alt_steps
        result["deterministic_0"] = {"ms_per_step": round(ms_fast, 3),
                                     "value": round(wl.tokens / (ms_fast / 1e3), 1), "steps": args.alt_steps}
        log(f"[bench] deterministic=0: {ms_fast:.2f} ms/step, {wl.tokens / ms_fast / 1e3:.3f} M tokens/s")
    if args.cpu_baseline == "on":
        log("[bench] timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline_block(wl) if wl.block else cpu_baseline(wl)
        log(f"[bench] cpu baseline: {result['cpu_baseline']['value']:.1f} tokens/s")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
