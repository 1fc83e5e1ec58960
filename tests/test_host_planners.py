"""The library's host-side planning over many shapes, on a machine without a
GPU: every convolution entry point is called through the C ABI with stand-in
device pointers (never dereferenced on the host), so each call validates its
arguments, plans its kernels and chunks and then fails at the launch. A
planner mistake (a division by zero, a tile of no pixels) crashes the process
instead. Skipped when a GPU is visible: the stand-in pointers must never reach
a kernel.
"""
import ctypes
import random
import subprocess
import sys

import pytest

import memory_efficient_im2win_amd as m
from memory_efficient_im2win_amd import _lib

# Return codes a planned call may give without a GPU: the launch fails
# (IM2WIN_ELAUNCH), or the arguments or workspace are refused first.
ALLOWED = {_lib.IM2WIN_OK, _lib.IM2WIN_EINVAL, _lib.IM2WIN_EWORKSPACE, _lib.IM2WIN_ELAUNCH}

KNOB_SETS = [{}, {"f32_valu": 1}, {"f16_reuse": -1, "f16_thin": -1, "f16_res": -1},
             {"f16_reuse": -1, "f16_rows": -1, "f16_thin": -1, "f16_wide": -1}]


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


def _shapes(seed, n):
    rng = random.Random(seed)
    for _ in range(n):
        Hf = rng.choice([1, 2, 3, 5, 7, 9, 11, 13])
        Wf = rng.choice([1, 2, 3, 5, 7, 8, 11, 16])
        sh, sw = rng.choice([1, 2, 3, 4]), rng.choice([1, 2, 3, 4])
        yield (rng.choice([1, 2, 3, 8, 64]), rng.choice([1, 2, 3, 5, 8, 16, 64, 96, 130]),
               Hf + rng.randrange(0, 60), Wf + rng.randrange(0, rng.choice([40, 300, 3000])),
               rng.choice([1, 7, 32, 64, 96, 128, 256, 300]), Hf, Wf, sh, sw)


def _drive(seed, n):
    """Runs every entry point over n shapes; returns the set of codes seen."""
    L = _lib.load()
    fake = 1 << 40
    x, w, y, ws = (ctypes.c_void_p(fake + (i << 36)) for i in range(4))
    seen = set()
    for ks in KNOB_SETS:
        with m.knobs(**ks):
            for N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw in _shapes(seed, n):
                dims = (N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw)
                for f in (L.conv2d_im2win_fp32_strided, L.conv2d_im2win_fp16_strided):
                    for wsp, wsb in ((None, 0), (ws, 1 << 33), (ws, 1 << 22)):
                        seen.add(f(x, w, y, wsp, wsb, *dims, None))
                seen.add(L.conv2d_im2win_fp16_fused(x, w, y, ws, 1 << 24, N, Ci, Hi, Wi, Co, Hf,
                                                    Wf, sh, sw, None))
                for f in (L.conv2d_im2win_nhwc_fp32, L.conv2d_im2win_nhwc_fp16):
                    for wsp, wsb in ((None, 0), (ws, 1 << 33)):
                        seen.add(f(x, w, y, wsp, wsb, *dims, None))
                seen.add(L.conv2d_im2win_nhwc_fp16_fused(x, w, y, ws, 1 << 24, *dims, None))
                for f in (L.conv2d_im2col_fp32, L.conv2d_im2col_fp16):
                    seen.add(f(x, w, y, ws, 1 << 34, *dims, None))
    return seen


@pytest.mark.skipif(not _no_gpu(), reason="a GPU is visible: stand-in pointers must not reach it")
def test_planners_over_random_shapes():
    # In a child process, so a crash fails this test instead of the run.
    code = ("import sys; sys.path.insert(0, %r); import test_host_planners as t; "
            "print(sorted(t._drive(7, 60)))" % (str(__import__('pathlib').Path(__file__).parent)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    seen = set(eval(r.stdout.strip().splitlines()[-1]))
    assert seen <= ALLOWED, seen
    assert _lib.IM2WIN_ELAUNCH in seen   # shapes were planned as far as a launch
