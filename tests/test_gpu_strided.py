"""Unequal row and column strides (sh != sw) on the GPU against the fp64
oracle, through every kernel: the fp32 matrix-core and vector-ALU kernels,
the fused fp16 kernel (filter gathered or prepacked), the materialised
kernels of both precisions, the plain fallback and the im2win transform.

Table I of "Enabling Memory-efficient Im2win Convolution with
Multi-precision Support on GPU CUDA and Tensor Cores" writes the stride per
axis, s_h(s_w); its rows all have the two equal, so these shapes are
synthetic. Bars as for equal strides: bit-exact for small-integer inputs,
otherwise |y - y_oracle| <= tol * sum|x*w| per output.
"""
import ctypes

import numpy as np
import pytest

import memory_efficient_im2win_amd as m
import workloads
from parity import WS_KINDS, TOL, assert_exact, assert_within, call, device, note, to_dev

pytestmark = pytest.mark.gpu

# (N, Ci, Hi, Wi, Co, Hf, Wf, (sh, sw)): each fp32 specialisation reached with a
# different row stride, sh below, equal to and above Hf, rectangles, 1x1,
# several tiles with ragged tails.
STRIDED = [
    (2, 5, 23, 29, 40, 3, 3, (1, 2)),
    (2, 3, 47, 45, 37, 11, 11, (4, 2)),
    (2, 3, 47, 45, 37, 11, 11, (2, 4)),
    (2, 16, 30, 29, 70, 7, 7, (3, 2)),
    (3, 24, 14, 18, 96, 5, 5, (2, 1)),
    (1, 13, 21, 17, 9, 2, 3, (1, 3)),
    (2, 6, 23, 11, 33, 4, 6, (3, 1)),
    (1, 9, 16, 16, 17, 2, 2, (5, 3)),
    (1, 64, 30, 30, 64, 7, 7, (1, 2)),
    (2, 3, 227, 227, 96, 11, 11, (4, 3)),
    (1, 96, 12, 12, 256, 5, 5, (1, 2)),
    (2, 8, 12, 40, 64, 1, 1, (2, 3)),
]

def _shape(t, dt):
    return workloads.ConvShape("strided", *t, dt)


def _run(sh, x, w, kind=None):
    import torch
    dev = device()
    y = call(sh, to_dev(x, dev), to_dev(w, dev), kind, dev).cpu().numpy()
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("t", STRIDED, ids=str)
def test_conv_strided(t, dt, orc):
    sh = _shape(t, dt)
    x, w = workloads.make_inputs(sh, seed=31)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    xi, wi = workloads.make_inputs(sh, seed=32, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    assert ref.shape[2:] == m.output_dims(sh.Hi, sh.Wi, sh.Hf, sh.Wf, sh.s)
    for kind in WS_KINDS:
        note(f"conv strided {sh.describe()} ws={kind}")
        assert_within(_run(sh, x, w, kind), ref, absd, TOL[dt], f"{sh.describe()} ws={kind}")
        assert_exact(_run(sh, xi, wi, kind), refi, f"{sh.describe()} ws={kind} integer")


@pytest.mark.parametrize("t", STRIDED, ids=str)
def test_conv_strided_f32_vector_alu(t, orc, knob):
    knob("f32_valu", 1)
    sh = _shape(t, "f32")
    x, w = workloads.make_inputs(sh, seed=33)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    note(f"conv strided fp32 vector ALU {sh.describe()}")
    assert_within(_run(sh, x, w), ref, absd, TOL["f32"], sh.describe())
    xi, wi = workloads.make_inputs(sh, seed=34, mode="int")
    assert_exact(_run(sh, xi, wi), orc.conv_direct(xi, wi, sh.s), sh.describe())


@pytest.mark.parametrize("nw", [4, 8, 12])
@pytest.mark.parametrize("t", [STRIDED[1], STRIDED[3], STRIDED[6], STRIDED[9]], ids=str)
def test_conv_strided_f32_matrix_waves(t, nw, orc, knob):
    knob("f32_ksplit", 1)
    knob("f32_nw", nw)
    sh = _shape(t, "f32")
    xi, wi = workloads.make_inputs(sh, seed=35, mode="int")
    note(f"conv strided fp32 NW={nw} {sh.describe()}")
    assert_exact(_run(sh, xi, wi), orc.conv_direct(xi, wi, sh.s), sh.describe())


@pytest.mark.parametrize("env", [{"f16_wpx": 1}, {"f16_nwh": 3}], ids=str)
@pytest.mark.parametrize("t", [STRIDED[0], STRIDED[3], STRIDED[8], STRIDED[9]], ids=str)
def test_conv_strided_f16_fused_tilings(t, env, orc, knob):
    for k, v in env.items():
        knob(k, v)
    # The prepacked calls reach the channel-interleaved kernel.
    knob("f16_thin", -1)
    knob("f16_wide", -1)
    sh = _shape(t, "f16")
    xi, wi = workloads.make_inputs(sh, seed=36, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    for kind in (None, "filter"):
        note(f"conv strided fp16 {env} {sh.describe()} ws={kind}")
        assert_exact(_run(sh, xi, wi, kind), refi, sh.describe())


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_conv_strided_generic_fallback(dt, orc):
    """A 13x13 filter over a wide row (outside the fp16 tiled kernels' LDS
    budget) with unequal strides."""
    sh = _shape((1, 9, 20, 600, 7, 13, 13, (3, 2)), dt)
    x, w = workloads.make_inputs(sh, seed=37)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    for kind in WS_KINDS:
        note(f"conv strided large filter {sh.describe()} ws={kind}")
        assert_within(_run(sh, x, w, kind), ref, absd, TOL[dt], sh.describe())


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_strided_entry_with_equal_strides_matches_single_stride_entry(dt):
    """conv2d_im2win_*_strided with sh == sw gives the single-stride result
    bit for bit (same kernels, same order)."""
    import torch
    dev = device()
    sh = _shape((2, 16, 30, 29, 70, 7, 7, 2), dt)
    x, w = workloads.make_inputs(sh, seed=38)
    xt, wt = to_dev(x, dev), to_dev(w, dev)
    a = m.conv2d(xt, wt, 2)
    b = torch.empty_like(a)
    L = m.load_library()
    f = L.conv2d_im2win_fp32_strided if dt == "f32" else L.conv2d_im2win_fp16_strided
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    note(f"conv strided entry, equal strides {sh.describe()}")
    rc = f(ctypes.c_void_p(xt.data_ptr()), ctypes.c_void_p(wt.data_ptr()),
           ctypes.c_void_p(b.data_ptr()), None, 0, *sh.x_shape, sh.Co, sh.Hf, sh.Wf, 2, 2, st)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("shape", [(2, 3, 19, 23, 3, 5, (2, 3)), (1, 5, 11, 8, 2, 5, (3, 1)),
                                   (2, 1, 50, 13, 3, 2, (5, 2)), (1, 2, 64, 301, 11, 11, (4, 2)),
                                   (1, 1, 9, 4001, 3, 3, (2, 1))], ids=str)
@pytest.mark.parametrize("width", [2, 4])
def test_pack_strided(shape, width, orc):
    import torch
    dev = device()
    N, Ci, Hi, Wi, Hf, Wf, s = shape
    note(f"pack strided {shape} width={width}")
    ut = np.uint16 if width == 2 else np.uint32
    rng = np.random.default_rng(7 + width)
    x = rng.integers(0, np.iinfo(ut).max, size=(N, Ci, Hi, Wi), dtype=ut, endpoint=True)
    xt = to_dev(x.view(np.int16 if width == 2 else np.int32), dev)
    got = m.pack(xt, Hf, Wf, s).cpu().numpy().view(ut)
    ref = orc.im2win_pack(x, Hf, Wf, s)
    assert got.shape == ref.shape and np.array_equal(got, ref)
    torch.cuda.synchronize()
