"""Benchmark: im2win convolution TFLOPS and workspace bytes on one MI355X.

A step is one forward convolution call over one batch of seeded synthetic
input already resident in HBM: the im2win transform, the filter staging, the
windowed dot products and the fp32 output store, all inside the library's HIP
kernels. The headline workload is the cv1 layer of Table I ("Enabling
Memory-efficient Im2win Convolution with Multi-precision Support on GPU CUDA
and Tensor Cores"): N=32, 3x227x227 input, 96 11x11 filters, stride 4, fp32
inputs, products and accumulation (on the fp32 matrix instructions by
default; mode fused_valu forces the vector-ALU kernel). The other Table I
layers (cv5 fp32 N=1; cv5, cv3, cv4 fp16 on the matrix cores) are timed the
same way and reported under "layers".

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
KERNEL_SOURCES = ["conv_f32_mfma.hip", "conv_f32.hip", "conv_f16_fused.hip", "conv_f16_rows.hip",
                  "conv_f16_wide.hip", "conv_f16_thin.hip",
                  "conv_f16.hip", "conv_generic.hip", "pack.hip", "im2col.hip", "nhwc.hip",
                  "api.hip", "common.hpp", "kernels.hpp"]
# Modes: fused (no workspace), fused_valu (fp32 on the vector-ALU kernel),
# prepacked (fp16 filter prepacked into a small workspace), materialized
# (im2win tensor in HBM).
MODES = ["fused", "fused_valu", "prepacked", "materialized"]


CONV_KERNELS = ("conv_f32_mfma_kernel", "conv_f32_kernel", "conv_f16_fused_kernel",
                "conv_f16_rows_kernel", "conv_f16_thin_kernel", "conv_f16_wide_kernel",
                "conv_f16_kernel")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def flops(sh, Ho, Wo) -> int:
    return 2 * sh.N * sh.Co * Ho * Wo * sh.Ci * sh.Hf * sh.Wf


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "memory_efficient_im2win_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def time_layer(sh, mode, steps, warmup):
    """Returns dict with per-launch-averaged ms and workspace bytes."""
    if mode == "fused_valu":
        old = os.environ.get("IM2WIN_F32_PATH")
        os.environ["IM2WIN_F32_PATH"] = "valu"
        try:
            return time_layer(sh, "fused", steps, warmup)
        finally:
            if old is None:
                os.environ.pop("IM2WIN_F32_PATH", None)
            else:
                os.environ["IM2WIN_F32_PATH"] = old
    import torch
    import memory_efficient_im2win_amd as m
    dev = torch.device("cuda:0")
    x, w = workloads.make_inputs(sh, seed=0)
    if mode == "nhwc_materialized":
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
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    elif mode == "im2col":
        wsb = m.im2col_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s,
                                       sh.elem_bytes)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    elif mode != "fused" and mode != "direct":
        wsb = m.conv_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s,
                                     sh.elem_bytes, mode == "materialized")
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None

    def call():
        if mode == "nhwc_materialized":
            m.conv2d_nhwc(xt, wt, sh.s, ws=ws, out=y)
        elif mode == "im2col":
            m.conv2d_im2col(xt, wt, sh.s, ws=ws, out=y)
        elif mode == "direct":
            m.conv2d_direct(xt, wt, sh.s, out=y)
        else:
            m.conv2d(xt, wt, sh.s, ws=ws, out=y)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record()
    for i in range(steps):
        starts[i].record()
        call()
        ends[i].record()
    t_all1.record()
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    total_ms = t_all0.elapsed_time(t_all1)
    f = flops(sh, Ho, Wo)
    res = {
        "ms_per_step": total_ms / steps,
        "ms_per_launch_avg": float(np.mean(per)),
        "ms_per_launch_min": float(np.min(per)),
        "tflops": f / (total_ms / steps) / 1e9,
        "flops": f,
        "workspace_bytes": wsb,
        "Ho": Ho, "Wo": Wo,
    }
    del ws, y, xt, wt
    torch.cuda.empty_cache()
    return res


def cpu_baseline(sh, budget_s=12.0):
    """The oracle (plain C loops, fp64 accumulation) on the host cores, on a
    bounded sample of the workload: as many images as fit the time budget,
    and when the whole batch takes less than that, the whole batch repeated
    until the budget is used. Scaled to TFLOPS."""
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
    f = 2 * n * reps * sh.Co * Ho * Wo * sh.Ci * sh.Hf * sh.Wf
    what = f"{n} of {sh.N} images" + (f", {reps} times" if reps > 1 else "")
    return {
        "value": f / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": O.num_threads(),
        "kind": "oracle",
        "sample": f"{what}, of {sh.name} ({sh.dtype} inputs, fp64 accumulation), {dt:.2f} s",
    }


def load_traffic(key, mode):
    """HBM traffic measured with rocprofv3 counters for the current kernel
    sources, or None (no measurement, or the kernels changed since)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    ent = d.get(f"{key}:{mode}")
    if not ent or ent.get("source_hash") != kernel_source_hash():
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
    materialised im2win mode on a layer and adds them, and the im2win/im2col
    ratios, to its entry. Memory is the bytes a call touches in HBM:
    x + w + y + workspace."""
    peak = PEAK_FP32_MFMA_TFLOPS if sh.dtype == "f32" else PEAK_FP16_MFMA_TFLOPS
    for mode in ("im2col", "direct", "nhwc_materialized"):
        r = time_layer(sh, mode, 3, 1)
        entry[mode] = {"tflops": round(r["tflops"], 3), "us_per_call": round(r["ms_per_step"] * 1e3, 2),
                       "frac_of_peak": round(r["tflops"] / peak, 4),
                       "workspace_bytes": r["workspace_bytes"]}
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


# Variants timed by --ablation: (label, mode, environment) per precision. The
# environment switches are the library's own planner overrides.
ABLATION = {
    "f32": [("matrix cores, planner's choice", "fused", {}),
            ("matrix cores, 4 waves/workgroup", "fused", {"IM2WIN_F32_NW": "4"}),
            ("matrix cores, 8 waves/workgroup", "fused", {"IM2WIN_F32_NW": "8"}),
            ("matrix cores, 12 waves/workgroup", "fused", {"IM2WIN_F32_NW": "12"}),
            ("vector ALU", "fused", {"IM2WIN_F32_PATH": "valu"}),
            ("materialised im2win tensor", "materialized", {})],
    "f16": [("fused, filter gathered in-kernel", "fused", {}),
            ("fused, filter prepacked (planner's kernel)", "prepacked", {}),
            ("prepacked, row-staged kernel with 4 waves", "prepacked", {"IM2WIN_F16_ROWS_NWV": "4"}),
            ("prepacked, row-staged, tiles in launch order", "prepacked",
             {"IM2WIN_F16_ROWS_SWIZZLE": "0"}),
            ("prepacked, thin-layer kernel with 512-pixel tiles", "prepacked",
             {"IM2WIN_F16_THIN_NB": "4"}),
            ("prepacked, wide-tile kernel with 4 waves of 4 x 4 blocks", "prepacked",
             {"IM2WIN_F16_WIDE_NW": "4"}),
            ("prepacked, channel-interleaved kernel", "prepacked",
             {"IM2WIN_F16_ROWS": "0", "IM2WIN_F16_THIN": "0", "IM2WIN_F16_WIDE": "0"}),
            ("channel-interleaved, 8 waves along pixels", "prepacked",
             {"IM2WIN_F16_ROWS": "0", "IM2WIN_F16_THIN": "0", "IM2WIN_F16_WIDE": "0",
              "IM2WIN_F16_WPX": "8"}),
            ("channel-interleaved, >= 2 filter parts per group", "prepacked",
             {"IM2WIN_F16_ROWS": "0", "IM2WIN_F16_THIN": "0", "IM2WIN_F16_WIDE": "0",
              "IM2WIN_F16_NWH": "2"}),
            ("materialised im2win tensor", "materialized", {})],
}


def ablation(keys, steps):
    """Times every layer under the ABLATION variants; prints a Markdown table."""
    import torch
    import memory_efficient_im2win_amd as m
    m.load_library()
    rows = []
    for key in keys:
        sh = workloads.BY_KEY[key]
        for label, mode, env in ABLATION[sh.dtype]:
            saved = {k: os.environ.get(k) for k in env}
            os.environ.update(env)
            try:
                r = time_layer(sh, mode, steps, 3)
            finally:
                for k, v in saved.items():
                    if v is None:
                        os.environ.pop(k, None)
                    else:
                        os.environ[k] = v
            peak = PEAK_FP32_MFMA_TFLOPS if sh.dtype == "f32" else PEAK_FP16_MFMA_TFLOPS
            rows.append((key, label, r["tflops"], r["ms_per_launch_avg"] * 1e3, r["tflops"] / peak,
                         r["workspace_bytes"]))
            log(f"[ablation] {key} {label}: {r['tflops']:.1f} TFLOP/s")
    torch.cuda.synchronize()
    print("| layer | variant | TFLOP/s | us per call | fraction of peak | workspace bytes |")
    print("|---|---|---|---|---|---|")
    for key, label, tf, us, fr, wsb in rows:
        print(f"| {key} | {label} | {tf:.1f} | {us:.1f} | {fr:.3f} | {wsb:,} |")


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
    ap.add_argument("--ablation", action="store_true",
                    help="time every layer under the library's variant switches and print a "
                         "Markdown table instead of the JSON line")
    args = ap.parse_args()

    if args.ablation:
        ablation(LAYER_KEYS, max(5, args.steps // 2))
        return

    if args.ingest_pmc:
        t = ingest_pmc(*args.ingest_pmc)
        kern = [k for k in t["kernels"] if any(n in k for n in CONV_KERNELS)]
        if len(kern) != 1:
            raise SystemExit(f"expected one conv kernel in the counters, found {kern}")
        path = os.path.join(ROOT, "profiles", "traffic.json")
        d = json.load(open(path)) if os.path.exists(path) else {}
        kb = t["kernels"][kern[0]]
        d[f"{args.workload}:{args.mode}"] = {
            "source_hash": kernel_source_hash(),
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

    sh = workloads.BY_KEY[args.workload]
    log(f"[bench] headline {sh.describe()} mode={args.mode} steps={args.steps} warmup={args.warmup}")
    head = time_layer(sh, args.mode, args.steps, args.warmup)
    log(f"[bench] headline {head['tflops']:.2f} TFLOP/s, {head['ms_per_step']*1e3:.1f} us/step")

    layers = {}
    if not args.no_layers:
        for key in LAYER_KEYS:
            lsh = workloads.BY_KEY[key]
            entry = {}
            modes = ("fused", "fused_valu", "materialized") if lsh.dtype == "f32" else \
                ("fused", "prepacked", "materialized")
            for mode in modes:
                r = time_layer(lsh, mode, max(5, args.steps // 2), 3)
                peak = PEAK_FP32_MFMA_TFLOPS if lsh.dtype == "f32" else PEAK_FP16_MFMA_TFLOPS
                entry[mode] = {"tflops": round(r["tflops"], 3), "us_per_call": round(r["ms_per_step"] * 1e3, 2),
                               "frac_of_peak": round(r["tflops"] / peak, 4),
                               "workspace_bytes": r["workspace_bytes"]}
                log(f"[bench] {key} {mode}: {r['tflops']:.2f} TFLOP/s "
                    f"({r['ms_per_step']*1e3:.1f} us/call, ws {r['workspace_bytes']} B)")
            if not args.no_baselines:
                baselines(lsh, entry)
            layers[key] = entry

    # Roofline of the dominant kernel. For the headline (cv1, fused) one call
    # is exactly one kernel launch, so the per-launch event time, taken on the
    # stream the library launches on, is that kernel's time.
    is_f32 = sh.dtype == "f32"
    valu = args.mode == "fused_valu"
    achieved = head["flops"] / (head["ms_per_launch_avg"] * 1e-3) / 1e12
    peak = (PEAK_FP32_VECTOR_TFLOPS if valu else PEAK_FP32_MFMA_TFLOPS) if is_f32 \
        else PEAK_FP16_MFMA_TFLOPS
    # With a prepacked filter the library runs the row-staged fp16 kernel on
    # shapes with an even column stride, Wf <= 8, Wi % 8 == 0 and even Ci.
    sw = sh.s[1] if isinstance(sh.s, tuple) else sh.s
    rows = (args.mode == "prepacked" and sh.Wf <= 8 and sw % 2 == 0 and sh.Wi % 8 == 0
            and sh.Ci % 2 == 0)
    # Otherwise, with a prepacked filter, layers with fewer than 8 input
    # channels run the thin-layer kernel and layers with at least 128 output
    # channels the wide-tile kernel (when their tiles fit LDS).
    thin = (args.mode == "prepacked" and not rows and sh.Ci < 8 and sh.Wf <= 8 and sw % 2 == 0
            and sh.Ci * sh.Hf <= 64)
    wide = args.mode == "prepacked" and not rows and not thin and sh.Co >= 128
    kernel = ("conv_f32_kernel" if valu else "conv_f32_mfma_kernel") if is_f32 else \
        ("conv_f16_kernel" if args.mode == "materialized" else
         "conv_f16_rows_kernel" if rows else "conv_f16_thin_kernel" if thin else
         "conv_f16_wide_kernel" if wide else "conv_f16_fused_kernel")
    roofline = {
        "bound": "alu" if valu else "mfma",
        "achieved": round(achieved, 3),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": load_traffic(args.workload, args.mode),
        "kernel": kernel,
        "launch_avg_us": round(head["ms_per_launch_avg"] * 1e3, 2),
    }

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(sh)
        log(f"[bench] cpu oracle {cpu['value']*1e3:.3f} GFLOP/s on {cpu['cores']} threads")

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
        "layers": layers,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
