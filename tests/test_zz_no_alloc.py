"""conv2d_im2win_fp16_fused_noalloc (filter scratch in the library's fixed
device array) against conv2d_im2win_fp16_fused (filter scratch in a caller
workspace), through the C ABI: the same kernels run, so the outputs must be
the same bits. Two calls in a row, the second with a smaller input, so the
second runs over the first's leftovers in the array."""
import ctypes

import numpy as np
import pytest

import memory_efficient_im2win_amd as m
import workloads
from parity import TOL, assert_within, device, note, to_dev

pytestmark = pytest.mark.gpu


def _c_call(fn, sh, xt, wt, y, fws=None):
    import torch
    st = ctypes.c_void_p(torch.cuda.current_stream(xt.device).cuda_stream)
    sh_, sw = m.strides(sh.s)
    args = [ctypes.c_void_p(xt.data_ptr()), ctypes.c_void_p(wt.data_ptr()),
            ctypes.c_void_p(y.data_ptr())]
    if fws is not None:
        args += [ctypes.c_void_p(fws.data_ptr()), fws.numel()]
    return fn(*args, sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh_, sw, st)


# Pairs (first call, second call with a smaller input): each fp16 kernel
# family and its filter layout (row-staged, thin-layer, wide-tile,
# channel-interleaved), then a different family in the second call.
PAIRS = [
    ((64, 64, 224, 224, 64, 7, 7, 2), (2, 64, 40, 40, 64, 7, 7, 2)),      # cv4, then a slice
    ((128, 96, 24, 24, 256, 5, 5, 1), (3, 13, 19, 21, 130, 3, 3, 1)),     # cv5, then wide-tile
    ((64, 3, 227, 227, 64, 7, 7, 2), (2, 12, 26, 40, 70, 3, 7, 2)),       # cv3, then interleaved
    ((4, 24, 40, 40, 96, 5, 5, 1), (1, 2, 9, 16, 64, 2, 2, 2)),           # interleaved, then rows
]


@pytest.mark.parametrize("first,second", PAIRS, ids=str)
def test_noalloc_matches_fused_with_workspace(first, second, orc):
    import torch
    dev = device()
    L = m.load_library()
    for i, t in enumerate((first, second)):
        sh = workloads.ConvShape("noalloc", *t, "f16")
        x, w = workloads.make_inputs(sh, seed=80 + i)
        xt, wt = to_dev(x, dev), to_dev(w, dev)
        Ho, Wo = m.output_dims(sh.Hi, sh.Wi, sh.Hf, sh.Wf, sh.s)
        fb = m.fused_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s)
        assert 0 < fb <= 4 << 20
        fws = torch.empty(fb, dtype=torch.uint8, device=dev)
        ya = torch.full((sh.N, sh.Co, Ho, Wo), float("nan"), dtype=torch.float32, device=dev)
        yb = torch.full_like(ya, float("nan"))
        note(f"noalloc call {i + 1} {sh.describe()}")
        assert _c_call(L.conv2d_im2win_fp16_fused, sh, xt, wt, ya, fws) == 0
        assert _c_call(L.conv2d_im2win_fp16_fused_noalloc, sh, xt, wt, yb) == 0
        torch.cuda.synchronize()
        assert torch.equal(ya, yb), f"call {i + 1}: {sh.describe()}"
        if sh.N * sh.Co * Ho * Wo <= 4_000_000:
            ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
            assert_within(yb.cpu().numpy(), ref, absd, TOL["f16"], sh.describe())
        else:
            assert bool(torch.isfinite(yb).all())
        del xt, wt, ya, yb, fws
    torch.cuda.synchronize()
