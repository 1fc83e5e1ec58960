"""Benchmark: im2win convolution TFLOPS and workspace bytes on one MI355X.

A step is one forward convolution call over one batch of seeded synthetic
input already resident in HBM: the im2win transform, the filter staging, the
windowed dot products and the fp32 output store, all inside the library's HIP
kernels. The headline workload is the cv1 layer of Table I ("Enabling
Memory-efficient Im2win Convolution with Multi-precision Support on GPU CUDA
and Tensor Cores"): N=32, 3x227x227 input, 96 11x11 filters, stride 4, fp32
inputs, products and accumulation (on the fp32 matrix instructions by
default; mode fused_valu forces the vector-ALU kernel). The other Table I
layers (cv5 fp32 N=1; cv5, cv3, cv4 fp16 on the matrix cores; cv2 fp32) are
timed the same way and reported under "layers", each with the roofline of
its kernel, the im2win transform timed on its own, and the CPU oracle timed
on a bounded sample of it.

Prints ONE JSON line on stdout (rank 0); progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

# Published MI355X peaks (dense) used for the roofline fractions.
PEAK_FP32_VECTOR_TFLOPS = 157.3   # 256 CU x 2.4 GHz x 256 flop/clk (packed FMA)
PEAK_FP32_MFMA_TFLOPS = 157.3     # dense fp32 matrix (v_mfma_f32_32x32x2_f32)
PEAK_FP16_MFMA_TFLOPS = 2516.6    # dense fp16 matrix
PEAK_HBM_GBS = 8000.0

HEADLINE = "cv1_f32_n32"
LAYER_KEYS = ["cv5_f32_n1", "cv1_f32_n32", "cv5_f16_n128", "cv3_f16_n64", "cv4_f16_n64",
              "cv2_f32_n32"]
# The source file of each convolution kernel: its counter measurements in
# profiles/traffic.json stay valid while that file and common.hpp do not
# change.
KERNEL_FILE = {"conv_f32_mfma_kernel": "conv_f32_mfma.hip",
               "conv_f32_small_kernel": "conv_f32_small.hip", "conv_f32_kernel": "conv_f32.hip",
               "conv_f16_fused_kernel": "conv_f16_fused.hip",
               "conv_f16_rows_kernel": "conv_f16_rows.hip",
               "conv_f16_reuse_kernel": "conv_f16_reuse.hip",
               "conv_f16_thin_kernel": "conv_f16_thin.hip",
               "conv_f16_wide_kernel": "conv_f16_wide.hip", "conv_f16_ws_kernel": "conv_f16_ws.hip",
               "conv_f16_res_kernel": "conv_f16_res.hip",
               "conv_f16_kernel": "conv_f16.hip"}
# Modes: fused (no workspace), fused_valu (fp32 on the vector-ALU kernel),
# prepacked (fp16 fused with the filter prepacked per call into a small
# workspace, conv2d_fused), materialized (the im2win tensor of the whole batch
# in HBM: a workspace of exactly workspace_bytes(N)).
MODES = ["fused", "fused_valu", "prepacked", "materialized"]
# Timed calls per layer (median and min reported): 50, and 20 for cv4.
LAYER_STEPS = {"cv4_f16_n64": 20}


CONV_KERNELS = ("conv_f32_mfma_kernel", "conv_f32_small_kernel", "conv_f32_kernel",
                "conv_f16_fused_kernel", "conv_f16_rows_kernel", "conv_f16_reuse_kernel",
                "conv_f16_thin_kernel", "conv_f16_wide_kernel", "conv_f16_res_kernel",
                "conv_f16_ws_kernel", "conv_f16_kernel")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def flops(sh, Ho, Wo) -> int:
    return 2 * sh.N * sh.Co * Ho * Wo * sh.Ci * sh.Hf * sh.Wf


def kernel_source_hash(kernel: str) -> str:
    """Hash of the sources of one convolution kernel (its file and
    common.hpp); of every library source for a name not in KERNEL_FILE."""
    csrc = os.path.join(ROOT, "memory_efficient_im2win_amd", "csrc")
    if kernel in KERNEL_FILE:
        files = [KERNEL_FILE[kernel], "common.hpp"]
    else:
        files = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".hpp")))
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _knobs_of(mode):
    return {"f32_valu": 1} if mode == "fused_valu" else {}


def time_layer(sh, mode, steps, warmup):
    """Times `steps` calls of one mode on layer sh (inputs resident in HBM,
    warm caches) with HIP events around each call on the stream the library
    launches on. Returns per-call mean, median and min, and the step rate."""
    import torch
    import memory_efficient_im2win_amd as m
    with m.knobs(**_knobs_of(mode)):
        return _time_layer(sh, mode, steps, warmup)


def _time_layer(sh, mode, steps, warmup):
    import torch
    call, info, hold = _layer_call(sh, mode)
    res = _time_calls(call, steps, warmup)
    f = info["flops"]
    res.update({
        "tflops": f / (res["ms_per_step"]) / 1e9,
        "tflops_median": f / res["ms_per_launch_median"] / 1e9,
        **info,
    })
    del call, hold
    torch.cuda.empty_cache()
    return res


def time_variants(sh, mode, variants, steps, rounds=4):
    """Times knob variants of one mode on layer sh over the same resident
    inputs, interleaved: `rounds` rounds, each timing steps // rounds calls
    of every variant in turn, so slow drifts of the clock (the chip's power
    management) fall on every variant alike. Per variant: the median call."""
    import torch
    import memory_efficient_im2win_amd as m
    with m.knobs(**_knobs_of(mode)):
        call, info, hold = _layer_call(sh, mode)
        per = {label: [] for label, _ in variants}
        for _ in range(rounds):
            for label, kn in variants:
                with m.knobs(**kn):
                    per[label] += _time_calls(call, max(1, steps // rounds), 2, raw=True)["per"]
    del call, hold
    torch.cuda.empty_cache()
    out = {}
    for label, _ in variants:
        med = float(np.median(per[label]))
        out[label] = {"ms_per_launch_median": med, "tflops_median": info["flops"] / med / 1e9,
                      "calls": len(per[label]), **info}
    return out


def _layer_call(sh, mode):
    """One mode on layer sh with seeded inputs, output and workspace resident
    on the GPU: the call, its flops and workspace bytes, and the tensors it
    holds."""
    import torch
    import memory_efficient_im2win_amd as m
    dev = torch.device("cuda:0")
    x, w = workloads.make_inputs(sh, seed=0)
    if mode in ("nhwc_materialized", "nhwc_fused"):
        x = np.ascontiguousarray(x.transpose(0, 2, 3, 1))
    xt = torch.from_numpy(x).to(dev)
    wt = torch.from_numpy(w).to(dev)
    Ho, Wo = m.output_dims(sh.Hi, sh.Wi, sh.Hf, sh.Wf, sh.s)
    y = torch.empty((sh.N, sh.Co, Ho, Wo), dtype=torch.float32, device=dev)
    ws = None
    wsb = 0
    if mode == "nhwc_materialized":
        y = torch.empty((sh.N, Ho, Wo, sh.Co), dtype=torch.float32, device=dev)
        wsb = m.nhwc_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s,
                                     sh.elem_bytes)
    elif mode == "nhwc_fused":
        y = torch.empty((sh.N, Ho, Wo, sh.Co), dtype=torch.float32, device=dev)
        wsb = m.nhwc_fused_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s)
    elif mode == "im2col":
        wsb = m.im2col_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s,
                                       sh.elem_bytes)
    elif mode == "materialized":
        wsb = m.workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Hf, sh.Wf, sh.s, sh.elem_bytes)
    elif mode == "prepacked" and sh.dtype == "f16":
        wsb = m.fused_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s)
    if wsb:
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def call():
        if mode == "nhwc_materialized":
            m.conv2d_nhwc(xt, wt, sh.s, ws=ws, out=y)
        elif mode == "nhwc_fused":
            m.conv2d_nhwc_fused(xt, wt, sh.s, fws=ws, out=y)
        elif mode == "im2col":
            m.conv2d_im2col(xt, wt, sh.s, ws=ws, out=y)
        elif mode == "direct":
            m.conv2d_direct(xt, wt, sh.s, out=y)
        elif mode == "prepacked" and sh.dtype == "f16":
            m.conv2d_fused(xt, wt, sh.s, fws=ws, out=y)
        else:
            m.conv2d(xt, wt, sh.s, ws=ws, out=y)
    info = {"flops": flops(sh, Ho, Wo), "workspace_bytes": wsb, "Ho": Ho, "Wo": Wo}
    return call, info, (xt, wt, y, ws)


def _time_calls(call, steps, warmup, raw=False):
    """Times `steps` calls on torch's current stream (the stream the binding
    passes to the library). The timed region holds the calls only, bracketed
    by two HIP events after a synchronisation: ms_per_step is its time per
    call. A second pass of the same calls with an event pair around each
    gives the per-call distribution (median, min, mean; per-call events add
    their own few microseconds of gaps, so they stay out of the first pass)."""
    import torch
    for _ in range(warmup):
        call()
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record()
    for _ in range(steps):
        call()
    t_all1.record()
    torch.cuda.synchronize()
    total_ms = t_all0.elapsed_time(t_all1)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        starts[i].record()
        call()
        ends[i].record()
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    res = {
        "ms_per_step": total_ms / steps,
        "ms_per_launch_avg": float(np.mean(per)),
        "ms_per_launch_median": float(np.median(per)),
        "ms_per_launch_min": float(np.min(per)),
    }
    if raw:
        res["per"] = per
    return res


def time_pack(sh, steps, warmup):
    """The im2win transform alone (im2win_pack of the whole batch): per-call
    median and min, and the rate of its algorithmic bytes (x read + the
    im2win tensor written) against the HBM peak."""
    import torch
    import memory_efficient_im2win_amd as m
    dev = torch.device("cuda:0")
    x, _ = workloads.make_inputs(sh, seed=0)
    xt = torch.from_numpy(x).to(dev)
    Ho, _ = m.output_dims(sh.Hi, sh.Wi, sh.Hf, sh.Wf, sh.s)
    out = torch.empty((sh.N, sh.Ci, Ho, sh.Wi * sh.Hf), dtype=xt.dtype, device=dev)
    r = _time_calls(lambda: m.pack(xt, sh.Hf, sh.Wf, sh.s, out=out), steps, warmup)
    nbytes = (xt.numel() + out.numel()) * xt.element_size()
    del xt, out
    torch.cuda.empty_cache()
    gbs = nbytes / (r["ms_per_launch_median"] * 1e-3) / 1e9
    return {"kernel": "pack_kernel", "us_median": round(r["ms_per_launch_median"] * 1e3, 2),
            "us_min": round(r["ms_per_launch_min"] * 1e3, 2), "bytes": nbytes,
            "GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(sh, budget_s=12.0):
    """The oracle (plain C loops, fp64 accumulation) on the host cores, on a
    bounded sample of the workload: as many images as fit the time budget,
    and when the whole batch takes less than that, the whole batch repeated
    until the budget is used. Scaled to TFLOPS. The oracle's im2win transform
    of the same sample is timed beside it."""
    import oracle
    O = oracle.default()
    x, w = workloads.make_inputs(sh, seed=0)
    Ho, Wo = O.out_hw(sh.Hi, sh.Wi, sh.Hf, sh.Wf, sh.s)
    t0 = time.perf_counter()
    O.conv_direct(x[:1], w, sh.s)
    t1 = time.perf_counter() - t0
    n = int(max(1, min(sh.N, budget_s / max(t1, 1e-6))))
    reps, dt = 0, 0.0
    while reps == 0 or (dt < 0.8 * budget_s and dt / reps * (reps + 1) < 1.5 * budget_s):
        t0 = time.perf_counter()
        O.conv_direct(x[:n], w, sh.s)
        dt += time.perf_counter() - t0
        reps += 1
    t0 = time.perf_counter()
    pk = O.im2win_pack(x[:n], sh.Hf, sh.Wf, sh.s)
    tp = time.perf_counter() - t0
    pbytes = (x[:n].nbytes + pk.nbytes)
    f = 2 * n * reps * sh.Co * Ho * Wo * sh.Ci * sh.Hf * sh.Wf
    what = f"{n} of {sh.N} images" + (f", {reps} times" if reps > 1 else "")
    return {
        "value": f / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": O.num_threads(),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"{what}, of {sh.name} ({sh.dtype} inputs, fp64 accumulation), {dt:.2f} s",
        "pack_s": round(tp, 4),
        "pack_GBps": round(pbytes / tp / 1e9, 3),
    }


def load_traffic(key, mode, kernel):
    """HBM bytes per launch of `kernel` measured with rocprofv3 counters for
    its current sources, or None (no measurement, another kernel, or its
    sources changed since)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    ent = d.get(f"{key}:{mode}")
    if not ent or ent.get("conv_kernel") != kernel or \
            ent.get("source_hash") != kernel_source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def calibrate_copy(nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size, for scaling the HBM
    counters (FETCH_SIZE / WRITE_SIZE) of a profiled run."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy: {reps} x {nbytes} bytes")


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def baselines(sh, entry):
    """Times the im2col + GEMM and direct-convolution baselines and the NHWC
    materialised im2win mode on a layer (and, for fp16 layers the fused NHWC
    kernel takes, the fused NHWC call) and adds them, and the im2win/im2col
    ratios, to its entry. Memory is the bytes a call touches in HBM:
    x + w + y + workspace."""
    import memory_efficient_im2win_amd as m
    peak = PEAK_FP32_MFMA_TFLOPS if sh.dtype == "f32" else PEAK_FP16_MFMA_TFLOPS
    modes = ["im2col", "direct", "nhwc_materialized"]
    if sh.dtype == "f16":
        k = m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, 2,
                               "nhwc_prepacked")
        if k == "conv_f16_res_kernel":
            modes.append("nhwc_fused")
        else:
            entry["nhwc_fused"] = {"kernel": k, "skipped": "outside the fused NHWC kernel's envelope"}
    for mode in modes:
        r = time_layer(sh, mode, 3, 1)
        entry[mode] = {"tflops": round(r["tflops_median"], 3),
                       "us_per_call": round(r["ms_per_launch_median"] * 1e3, 2),
                       "frac_of_peak": round(r["tflops"] / peak, 4),
                       "workspace_bytes": r["workspace_bytes"]}
        if mode == "nhwc_fused":
            entry[mode]["kernel"] = "conv_f16_res_kernel"
        log(f"[bench] {sh.name} {mode}: {r['tflops']:.2f} TFLOP/s "
            f"({r['ms_per_step']*1e3:.1f} us/call, ws {r['workspace_bytes']} B)")
    Ho = (sh.Hi - sh.Hf) // workloads_stride(sh)[0] + 1
    Wo = (sh.Wi - sh.Wf) // workloads_stride(sh)[1] + 1
    base = (sh.N * sh.Ci * sh.Hi * sh.Wi + sh.Co * sh.Ci * sh.Hf * sh.Wf) * sh.elem_bytes + \
        sh.N * sh.Co * Ho * Wo * 4
    im2win_modes = [k for k in ("fused", "prepacked", "materialized") if k in entry]
    best = max(im2win_modes, key=lambda k: entry[k]["tflops"])
    col = base + entry["im2col"]["workspace_bytes"]
    # Whatever the GEMM, an im2col convolution writes and then reads its
    # matrix: at the HBM peak that alone bounds its time from below.
    col_bound_us = (base + 2 * entry["im2col"]["workspace_bytes"]) / (PEAK_HBM_GBS * 1e9) * 1e6
    entry["vs_baselines"] = {
        "best_im2win_mode": best,
        "tflops_vs_im2col": round(entry[best]["tflops"] / entry["im2col"]["tflops"], 3),
        "im2col_hbm_bound_us": round(col_bound_us, 2),
        "speed_vs_im2col_hbm_bound": round(col_bound_us / entry[best]["us_per_call"], 3),
        "tflops_vs_direct": round(entry[best]["tflops"] / entry["direct"]["tflops"], 3),
        "memory_vs_im2col_best_mode": round((base + entry[best]["workspace_bytes"]) / col, 4),
        "memory_vs_im2col_materialized": round((base + entry["materialized"]["workspace_bytes"]) / col, 4),
    }
    log(f"[bench] {sh.name} im2win {best} vs im2col: {entry['vs_baselines']['tflops_vs_im2col']}x TFLOP/s "
        f"({entry['vs_baselines']['speed_vs_im2col_hbm_bound']}x its HBM bound), "
        f"memory {entry['vs_baselines']['memory_vs_im2col_best_mode']:.3f} "
        f"(materialised im2win {entry['vs_baselines']['memory_vs_im2col_materialized']:.3f})")


def workloads_stride(sh):
    return sh.s if isinstance(sh.s, tuple) else (sh.s, sh.s)


def ingest_pmc(fetch_csv, write_csv, copy_bytes=1 << 30):
    """Per-launch HBM bytes of each kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE, KiB per dispatch), scaled so that the calibration
    copy reads and writes exactly its size. Writes profiles/traffic.json."""
    def per_kernel(path, counter):
        vals = {}
        for r in _read_csv(path):
            if r.get("Counter_Name") != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: float(np.mean(v)) for k, v in vals.items()}
    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    copy_k = [k for k in fetch if "copy" in k.lower() or "elementwise" in k.lower()]
    if not copy_k:
        raise SystemExit("no copy kernel found in the counter files")
    ck = max(copy_k, key=lambda k: fetch[k])
    f_scale = copy_bytes / (fetch[ck] * 1024.0)
    w_scale = copy_bytes / (write[ck] * 1024.0)
    out = {"copy_kernel": ck, "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    for k in fetch:
        if k in write:
            out["kernels"][k] = {"fetch_bytes": fetch[k] * 1024.0 * f_scale,
                                 "write_bytes": write[k] * 1024.0 * w_scale}
    return out


# Variants timed by --ablation: (label, mode, knobs, kernel) per precision.
# The knobs are the library's own planner overrides (im2win_set_knob); a row
# is timed only on layers where the knobs route the call to `kernel` (None:
# whatever the planner picks), so every row names the kernel it measured.
_ALL_F16_OFF = {"f16_reuse": -1, "f16_rows": -1, "f16_thin": -1, "f16_wide": -1, "f16_res": -1}
ABLATION = {
    "f32": [("matrix cores, planner's choice", "fused", {}, None),
            ("matrix cores, 4 waves/workgroup", "fused", {"f32_nw": 4, "f32_ksplit": 1}, None),
            ("matrix cores, 8 waves/workgroup", "fused", {"f32_nw": 8, "f32_ksplit": 1}, None),
            ("matrix cores, 12 waves/workgroup", "fused", {"f32_nw": 12, "f32_ksplit": 1}, None),
            ("matrix cores, K shared by 8 waves", "fused", {"f32_ksplit": 8}, None),
            ("vector ALU", "fused", {"f32_valu": 1}, None),
            ("materialised im2win tensor", "materialized", {}, None)],
    "f16": [("fused, filter gathered in-kernel (planner's kernel)", "fused", {}, None),
            ("fused, filter prepacked per call (planner's kernel)", "prepacked", {}, None),
            ("row-staged kernel (row reuse off)", "prepacked", {"f16_reuse": -1},
             "conv_f16_rows_kernel"),
            ("row-staged kernel, 4 waves", "prepacked", {"f16_reuse": -1, "f16_rows_nwv": 4},
             "conv_f16_rows_kernel"),
            ("row-staged kernel, 2 stage buffers", "prepacked",
             {"f16_reuse": -1, "f16_rows_bufs": 2}, "conv_f16_rows_kernel"),
            ("thin-layer kernel, 512-pixel tiles", "prepacked", {"f16_thin_nb": 4},
             "conv_f16_thin_kernel"),
            ("wide-tile kernel (resident-input kernel off)", "prepacked", {"f16_res": -1},
             "conv_f16_wide_kernel"),
            ("wide-tile kernel, 4 waves of 4 x 4 blocks", "prepacked",
             {"f16_res": -1, "f16_wide_nw": 4}, "conv_f16_wide_kernel"),
            ("channel-interleaved kernel", "prepacked", dict(_ALL_F16_OFF),
             "conv_f16_fused_kernel"),
            ("channel-interleaved, 8 waves along pixels", "prepacked",
             dict(_ALL_F16_OFF, f16_wpx=8), "conv_f16_fused_kernel"),
            ("channel-interleaved, >= 2 filter parts per group", "prepacked",
             dict(_ALL_F16_OFF, f16_nwh=2), "conv_f16_fused_kernel"),
            ("materialised im2win tensor", "materialized", {}, None),
            ("materialised, tiled kernel (staged kernel off)", "materialized", {"f16_ws": -1},
             "conv_f16_kernel")],
}


# The two switches every staged matrix-core kernel has, timed per layer and
# call mode: tiles in launch order instead of XCD-grouped (tile_order=1), and
# stages copied through registers and waited for before their MFMAs instead
# of loaded ahead while the previous stage computes (sync_staging=1).
SWITCHES = [("default", {}), ("tiles in launch order", {"tile_order": 1}),
            ("synchronous staging", {"sync_staging": 1}),
            ("launch order + synchronous staging", {"tile_order": 1, "sync_staging": 1})]
SWITCH_MODES = {"f32": ["fused"], "f16": ["fused", "prepacked", "materialized"]}
# Kernels with both switches; the small-problem fp32 kernel and the
# resident-input fp16 kernel stage their input once (no copy of it can
# overlap their MFMAs) and have only the tile order.
SWITCH_KERNELS = ("conv_f32_mfma_kernel", "conv_f16_reuse_kernel", "conv_f16_rows_kernel",
                  "conv_f16_thin_kernel", "conv_f16_wide_kernel", "conv_f16_fused_kernel",
                  "conv_f16_ws_kernel")
ORDER_ONLY_KERNELS = ("conv_f32_small_kernel", "conv_f16_res_kernel")


def ablation(keys, steps):
    """Times every layer under the two switches (per call mode) and under the
    ABLATION variants; prints two Markdown tables."""
    import torch
    import memory_efficient_im2win_amd as m
    m.load_library()
    sw_rows, rows = [], []
    for key in keys:
        sh = workloads.BY_KEY[key]
        peak = PEAK_FP32_MFMA_TFLOPS if sh.dtype == "f32" else PEAK_FP16_MFMA_TFLOPS
        for mode in SWITCH_MODES[sh.dtype]:
            kern = m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s,
                                      sh.elem_bytes, mode)
            variants = SWITCHES if kern in SWITCH_KERNELS else \
                SWITCHES[:2] if kern in ORDER_ONLY_KERNELS else SWITCHES[:1]
            res = time_variants(sh, mode, variants, steps)
            base = res[variants[0][0]]["ms_per_launch_median"]
            for label, _ in variants:
                r = res[label]
                us = r["ms_per_launch_median"] * 1e3
                sw_rows.append((key, mode, kern, label, r["tflops_median"], us,
                                r["ms_per_launch_median"] / base, r["tflops_median"] / peak))
                log(f"[ablation] {key} {mode} {kern} {label}: {us:.1f} us")
        todo = []
        for label, mode, kn, target in ABLATION[sh.dtype]:
            with m.knobs(**kn):
                kern = m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s,
                                          sh.elem_bytes, mode)
            if target is None or kern == target:
                todo.append((label, mode, kn, kern))
        res = {}
        for mode in dict.fromkeys(md for _, md, _, _ in todo):
            res.update(time_variants(sh, mode, [(lb, kn) for lb, md, kn, _ in todo
                                                if md == mode], steps))
        for label, _, _, kern in todo:
            r = res[label]
            rows.append((key, label, kern, r["tflops_median"], r["ms_per_launch_median"] * 1e3,
                         r["tflops_median"] / peak, r["workspace_bytes"]))
            log(f"[ablation] {key} {label}: {r['tflops_median']:.1f} TFLOP/s")
    torch.cuda.synchronize()
    print("| layer | mode | kernel | variant | TFLOP/s | us per call (median) "
          "| time / default | fraction of peak |")
    print("|---|---|---|---|---|---|---|---|")
    for key, mode, kern, label, tf, us, rel, fr in sw_rows:
        print(f"| {key} | {mode} | {kern} | {label} | {tf:.1f} | {us:.1f} | {rel:.3f} | {fr:.3f} |")
    print()
    print("| layer | variant | kernel | TFLOP/s | us per call (median) | fraction of peak "
          "| workspace bytes |")
    print("|---|---|---|---|---|---|---|")
    for key, label, kern, tf, us, fr, wsb in rows:
        print(f"| {key} | {label} | {kern} | {tf:.1f} | {us:.1f} | {fr:.3f} | {wsb:,} |")


def fill_rate(key, sh, steps, warmup):
    """torch's fill_ and copy_ over the fp32 output size of sh, timed with HIP
    events: the write (and read + write) rates that plain streaming kernels
    reach, beside which an output-bound convolution is read."""
    import torch
    dev = torch.device("cuda:0")
    import memory_efficient_im2win_amd as m
    Ho, Wo = m.output_dims(sh.Hi, sh.Wi, sh.Hf, sh.Wf, sh.s)
    n = sh.N * sh.Co * Ho * Wo
    y = torch.empty(n, dtype=torch.float32, device=dev)
    z = torch.empty(n, dtype=torch.float32, device=dev)
    for _ in range(warmup):
        y.fill_(1.0)
        z.copy_(y)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(steps):
        y.fill_(1.0)
    ev[1].record()
    for _ in range(steps):
        z.copy_(y)
    ev[2].record()
    torch.cuda.synchronize()
    f_us = ev[0].elapsed_time(ev[1]) / steps * 1e3
    c_us = ev[1].elapsed_time(ev[2]) / steps * 1e3
    return {"workload": key, "bytes": n * 4, "steps": steps, "fill_us": round(f_us, 2),
            "fill_TBps": round(n * 4 / f_us / 1e6, 3), "copy_us": round(c_us, 2),
            "copy_TBps_read_plus_write": round(2 * n * 4 / c_us / 1e6, 3)}


# Rates measured on this chip by measured_peaks() (filled in by main()).
MEASURED = {}
PROBE_ITERS = {"fp32_vector": 9000, "fp32_mfma": 4500, "fp16_mfma": 8000}


def measured_peaks():
    """The rates the chip sustains for each kind of arithmetic (the library's
    register-only rate probe, best of 2 and 4 waves per SIMD, 5 launches
    timed with HIP events after 2 warm-up) and the HBM rates of a 1 GiB fill
    and copy: the measured peaks beside the published ones."""
    import torch
    import memory_efficient_im2win_amd as m
    res = {}
    for kind, iters in PROBE_ITERS.items():
        best = 0.0
        for blocks in (512, 1024):
            out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
            for _ in range(2):
                m.peak_probe(kind, blocks, iters, out)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            ev[0].record()
            flops = 0.0
            for _ in range(5):
                flops += m.peak_probe(kind, blocks, iters, out)[1]
            ev[1].record()
            torch.cuda.synchronize()
            best = max(best, flops / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e12)
        res[kind + "_TFLOPs"] = round(best, 1)
    n = 1 << 28
    a = torch.empty(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        a.fill_(1.0)
        b.copy_(a)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(5):
        a.fill_(1.0)
    ev[1].record()
    for _ in range(5):
        b.copy_(a)
    ev[2].record()
    torch.cuda.synchronize()
    res["hbm_fill_GBps"] = round(5 * n * 4 / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9, 1)
    res["hbm_copy_GBps"] = round(5 * 2 * n * 4 / (ev[1].elapsed_time(ev[2]) * 1e-3) / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    return res


def measured_peak_of(sh, mode):
    """The measured rate of the arithmetic unit a layer's kernel runs on
    (None before measured_peaks() has run)."""
    bound, _ = peak_of(sh, mode)
    key = "fp32_vector_TFLOPs" if bound == "alu" else \
        "fp16_mfma_TFLOPs" if sh.dtype == "f16" else "fp32_mfma_TFLOPs"
    return MEASURED.get(key)


def alg_bytes(sh, mode):
    """(bytes read, bytes written) in HBM by one call, algorithmically: every
    tensor once. Fused: x, w read, y written (prepacked: plus the filter
    pack's read of w and write of the packed filter, and its read). The
    materialised mode: the transform reads x and writes the im2win tensor,
    the convolution reads it and w and writes y."""
    Ho = (sh.Hi - sh.Hf) // (sh.s[0] if isinstance(sh.s, tuple) else sh.s) + 1
    Wo = (sh.Wi - sh.Wf) // (sh.s[1] if isinstance(sh.s, tuple) else sh.s) + 1
    e = sh.elem_bytes
    x = sh.N * sh.Ci * sh.Hi * sh.Wi * e
    w = sh.Co * sh.Ci * sh.Hf * sh.Wf * e
    y = sh.N * sh.Co * Ho * Wo * 4
    ws = sh.N * sh.Ci * Ho * sh.Wi * sh.Hf * e
    if mode == "materialized":
        return x + ws + w, ws + y
    if mode == "prepacked":
        return x + 2 * w, y + w
    return x + w, y


def bound_of(sh, mode):
    """The roofline bound of a call: HBM when its algorithmic bytes at the
    HBM peak take longer than its flops at the arithmetic peak."""
    _, peak = peak_of(sh, mode)
    Ho = (sh.Hi - sh.Hf) // (sh.s[0] if isinstance(sh.s, tuple) else sh.s) + 1
    Wo = (sh.Wi - sh.Wf) // (sh.s[1] if isinstance(sh.s, tuple) else sh.s) + 1
    rd, wr = alg_bytes(sh, mode)
    t_bytes = (rd + wr) / (PEAK_HBM_GBS * 1e9)
    t_flops = flops(sh, Ho, Wo) / (peak * 1e12)
    return "hbm" if t_bytes > t_flops else peak_of(sh, mode)[0]


def peak_of(sh, mode):
    """(bound, peak TFLOP/s) of a layer's convolution kernel in a mode."""
    if sh.dtype == "f16":
        return "mfma", PEAK_FP16_MFMA_TFLOPS
    if mode == "fused_valu" or mode == "materialized":
        return "alu", PEAK_FP32_VECTOR_TFLOPS
    return "mfma", PEAK_FP32_MFMA_TFLOPS


def kernel_of(sh, mode):
    import memory_efficient_im2win_amd as m
    kmode = {"fused": "fused", "fused_valu": "fused", "prepacked": "prepacked",
             "materialized": "materialized"}[mode]
    with m.knobs(**_knobs_of(mode)):
        return m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s,
                                  sh.elem_bytes, kmode)


def roofline_of(key, sh, mode, r):
    """Roofline of a layer's dominant kernel. In the fused modes one call is
    one kernel launch, so the timed region's time per call (HIP events on the
    stream the library launches on, around the back-to-back calls) is that
    kernel's average launch time, gaps between launches included. In the
    prepacked mode a call is the filter prepack plus the convolution kernel,
    and in the materialised mode the im2win transform plus the convolution
    kernel; their per-call time includes those launches."""
    kern = kernel_of(sh, mode)
    t = r["ms_per_step"] * 1e-3   # the timed region's time per call
    bound = bound_of(sh, mode)
    if bound == "hbm":
        rd, wr = alg_bytes(sh, mode)
        achieved = (rd + wr) / t / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
        mp = MEASURED.get("hbm_fill_GBps" if wr > rd else "hbm_copy_GBps")
    else:
        _, peak = peak_of(sh, mode)
        achieved = r["flops"] / t / 1e12
        unit = "TFLOP/s"
        mp = measured_peak_of(sh, mode)
    return {
        "bound": bound,
        "achieved": round(achieved, 3),
        "peak": peak,
        "unit": unit,
        "frac": round(achieved / peak, 4),
        "measured_peak": mp,
        "frac_of_measured": round(achieved / mp, 4) if mp else None,
        "tflops": round(r["flops"] / t / 1e12, 3),
        "traffic": load_traffic(key, mode, kern),
        "kernel": kern,
        "launches_per_call": 1 if mode in ("fused", "fused_valu") else 2,
        "timed_us_per_call": round(r["ms_per_step"] * 1e3, 2),
        "launch_avg_us": round(r["ms_per_launch_avg"] * 1e3, 2),
        "launch_median_us": round(r["ms_per_launch_median"] * 1e3, 2),
        "launch_min_us": round(r["ms_per_launch_min"] * 1e3, 2),
    }


def layer_entry(key, args):
    """Every mode of one layer: per-call median, min and mean, TFLOP/s (on the
    median), the kernel and its roofline; the im2win transform alone; the
    baselines; the CPU oracle on a bounded sample."""
    lsh = workloads.BY_KEY[key]
    steps = LAYER_STEPS.get(key, 50)
    entry = {}
    modes = ("fused", "fused_valu", "materialized") if lsh.dtype == "f32" else \
        ("fused", "prepacked", "materialized")
    for mode in modes:
        r = time_layer(lsh, mode, steps, 5)
        _, peak = peak_of(lsh, mode)
        entry[mode] = {"tflops": round(r["tflops_median"], 3),
                       "us_per_call": round(r["ms_per_launch_median"] * 1e3, 2),
                       "us_min": round(r["ms_per_launch_min"] * 1e3, 2),
                       "us_mean": round(r["ms_per_launch_avg"] * 1e3, 2),
                       "frac_of_peak": round(r["tflops_median"] / peak, 4),
                       "workspace_bytes": r["workspace_bytes"],
                       "roofline": roofline_of(key, lsh, mode, r)}
        log(f"[bench] {key} {mode}: {r['tflops_median']:.2f} TFLOP/s "
            f"({r['ms_per_launch_median']*1e3:.1f} us/call median, "
            f"{r['ms_per_launch_min']*1e3:.1f} min, ws {r['workspace_bytes']} B, "
            f"{entry[mode]['roofline']['kernel']})")
    entry["pack"] = time_pack(lsh, steps, 5)
    log(f"[bench] {key} pack: {entry['pack']['us_median']} us, {entry['pack']['GBps']} GB/s")
    if not args.no_baselines:
        baselines(lsh, entry)
    if not args.no_cpu:
        entry["cpu_oracle"] = cpu_baseline(lsh, budget_s=2.5)
        log(f"[bench] {key} cpu oracle {entry['cpu_oracle']['value']*1e3:.2f} GFLOP/s")
    return entry


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(workloads.BY_KEY))
    ap.add_argument("--mode", default="fused", choices=MODES,
                    help="fused: no workspace; fused_valu: fp32 on the vector-ALU kernel; "
                         "prepacked: fused with the fp16 filter prepacked into a small "
                         "workspace; materialized: im2win tensor in HBM")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-layers", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-baselines", action="store_true",
                    help="skip the im2col + GEMM and direct-convolution baselines and the "
                         "NHWC lines per layer")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (for scaling rocprofv3 HBM counters)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs of this bench into "
                         "profiles/traffic.json for the current kernel sources, then exit")
    ap.add_argument("--fill-rate", action="store_true",
                    help="time a plain fill and a device copy of the workload's fp32 output "
                         "size (the write rate an HBM-bound kernel can reach), print one "
                         "JSON line and exit")
    ap.add_argument("--baseline", choices=["im2col", "direct", "nhwc_materialized", "nhwc_fused"],
                    help="time only this comparison mode on --workload (for a kernel trace of "
                         "it), print one JSON line and exit")
    ap.add_argument("--ablation", action="store_true",
                    help="time every layer under the library's variant switches and print a "
                         "Markdown table instead of the JSON line")
    args = ap.parse_args()

    if args.ablation:
        ablation(LAYER_KEYS, max(8, args.steps))
        return

    if args.ingest_pmc:
        t = ingest_pmc(*args.ingest_pmc)
        kern = [k for k in t["kernels"] if any(n in k for n in CONV_KERNELS)]
        if len(kern) != 1:
            raise SystemExit(f"expected one conv kernel in the counters, found {kern}")
        path = os.path.join(ROOT, "profiles", "traffic.json")
        d = json.load(open(path)) if os.path.exists(path) else {}
        kb = t["kernels"][kern[0]]
        import memory_efficient_im2win_amd as m
        m.load_library()
        name = kernel_of(workloads.BY_KEY[args.workload], args.mode)
        if name not in kern[0]:
            raise SystemExit(f"the counters are of {kern[0]}, the planner runs {name}")
        d[f"{args.workload}:{args.mode}"] = {
            "conv_kernel": name,
            "source_hash": kernel_source_hash(name),
            "kernel": kern[0][:120],
            "bytes_per_launch": round(kb["fetch_bytes"] + kb["write_bytes"]),
            "fetch_bytes": round(kb["fetch_bytes"]), "write_bytes": round(kb["write_bytes"]),
            "copy_scale": {"fetch": t["fetch_scale"], "write": t["write_scale"],
                           "copy_kernel": t["copy_kernel"][:120]},
        }
        with open(path, "w") as f:
            json.dump(d, f, indent=1)
        print(json.dumps(d[f"{args.workload}:{args.mode}"]))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the im2win forward convolution needs no "
              "collective and this build runs on a single MI355X; use --gpus 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    import memory_efficient_im2win_amd as m
    m.load_library()

    if args.calibrate_copy:
        calibrate_copy()

    if args.fill_rate:
        print(json.dumps(fill_rate(args.workload, workloads.BY_KEY[args.workload], args.steps,
                                   args.warmup)),
              flush=True)
        return

    if args.baseline:
        r = time_layer(workloads.BY_KEY[args.workload], args.baseline, args.steps, args.warmup)
        print(json.dumps({"workload": args.workload, "mode": args.baseline,
                          "us_per_call_median": round(r["ms_per_launch_median"] * 1e3, 2),
                          "us_per_call_min": round(r["ms_per_launch_min"] * 1e3, 2),
                          "workspace_bytes": r.get("workspace_bytes")}), flush=True)
        return

    MEASURED.update(measured_peaks())
    log(f"[bench] measured peaks {MEASURED}")
    sh = workloads.BY_KEY[args.workload]
    log(f"[bench] headline {sh.describe()} mode={args.mode} steps={args.steps} warmup={args.warmup}")
    head = time_layer(sh, args.mode, args.steps, args.warmup)
    log(f"[bench] headline {head['tflops']:.2f} TFLOP/s, {head['ms_per_step']*1e3:.1f} us/step")

    layers = {}
    if not args.no_layers:
        for key in LAYER_KEYS:
            layers[key] = layer_entry(key, args)

    roofline = roofline_of(args.workload, sh, args.mode, head)

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(sh)
        log(f"[bench] cpu oracle {cpu['value']*1e3:.3f} GFLOP/s on {cpu['cores']} threads")
    is_f32 = sh.dtype == "f32"

    out = {
        "metric": "conv TFLOPS (fp32 VALU, fp16 MFMA) + workspace bytes on cv1-cv5 shapes",
        "value": round(head["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if is_f32 else "f16 in, f32 accumulate",
        "data": "synthetic (seeded iid U[-1,1] at the Table I layer shapes)",
        "config": {
            "workload": f"{sh.name} forward conv, N={sh.N}, {sh.dtype}: input {sh.Ci}x{sh.Hi}x{sh.Wi}, "
                        f"filters {sh.Co}x{sh.Ci}x{sh.Hf}x{sh.Wf}, stride {sh.s}, "
                        f"output {sh.Co}x{head['Ho']}x{head['Wo']}",
            "mode": args.mode,
            "workspace_bytes": head["workspace_bytes"],
            "global_batch": sh.N,
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "measured_peaks": dict(MEASURED),
        "layers": layers,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
