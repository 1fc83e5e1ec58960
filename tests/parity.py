"""Helpers shared by the GPU parity tests: device setup, running the HIP
path through the binding, and comparing with the oracle."""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-5, "f16": 2e-3}


def device():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (run with -m 'not gpu' on a CPU host)")
    return torch.device("cuda:0")


def note(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def assert_within(y, ref, absdot, tol, what):
    """|y - ref| <= tol * sum|x*w| for every output (NaN never passes)."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - ref)
    bound = tol * absdot
    ok = err <= bound
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        detail = ", ".join(f"{tuple(int(v) for v in i)}: gpu={y[tuple(i)]!r} ref={ref[tuple(i)]!r} "
                           f"bound={bound[tuple(i)]!r}" for i in bad)
        raise AssertionError(f"{what}: {int((~ok).sum())} outputs out of tolerance; {detail}")
    scale = float(np.max(absdot)) if absdot.size else 0.0
    return float(np.max(err)) / scale if scale > 0 else 0.0


def assert_exact(y, ref, what):
    y = np.asarray(y, dtype=np.float32)
    r = np.asarray(ref).astype(np.float32)
    if not np.array_equal(y, r):
        bad = np.argwhere(y != r)[:5]
        detail = ", ".join(f"{tuple(int(v) for v in i)}: gpu={y[tuple(i)]} ref={r[tuple(i)]}"
                           for i in bad)
        raise AssertionError(f"{what}: {int((y != r).sum())} outputs differ; {detail}")


# Workspace modes of a convolution call: None (fused, no workspace),
# "filter" (fp16 fused with its filter prepacked into a workspace by
# conv2d_fused; the same as None for fp32), "full" (materialised over the
# whole batch: exactly workspace_bytes(N)) and "one" (materialised one image
# at a time: workspace_bytes(1)).
WS_KINDS = [None, "filter", "full", "one"]


def workspace(sh, kind, dev):
    """The workspace tensor for mode `kind` of shape sh, or None."""
    import torch
    import memory_efficient_im2win_amd as m
    if kind is None or (kind == "filter" and sh.dtype == "f32"):
        return None
    if kind == "filter":
        nb = m.fused_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s)
    else:
        n = sh.N if kind == "full" else 1
        nb = m.workspace_bytes(n, sh.Ci, sh.Hi, sh.Wi, sh.Hf, sh.Wf, sh.s, sh.elem_bytes)
    return torch.empty(nb, dtype=torch.uint8, device=dev)


def call(sh, xt, wt, kind, dev, out=None, ws=None):
    """One convolution call through the binding in workspace mode `kind`
    (ws: a workspace tensor to use instead of a fresh one)."""
    import memory_efficient_im2win_amd as m
    if ws is None:
        ws = workspace(sh, kind, dev)
    if kind == "filter" and sh.dtype == "f16":
        return m.conv2d_fused(xt, wt, sh.s, fws=ws, out=out)
    return m.conv2d(xt, wt, sh.s, ws=ws, out=out)
