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
