"""NHWC tensors on the GPU against the oracle: the NHWC im2win transform bit
for bit, and the convolution (direct, and materialised with the window runs
multiplied on the matrix cores) against the fp64 direct oracle, with x and y
permuted to NCHW on the host for the comparison."""
import numpy as np
import pytest

import memory_efficient_im2win_amd as m
import workloads
from parity import TOL, assert_exact, assert_within, device, note, to_dev

pytestmark = pytest.mark.gpu

# (N, Ci, Hi, Wi, Co, Hf, Wf, s): Ci a multiple of 16 (window runs unpadded
# in both precisions), of 8 only (unpadded in fp32, padded in fp16), and
# neither (runs padded to 32 bytes in both: Hf*Ci = 33 -> 40 floats or 48
# halves; 15 -> 16 in both).
SHAPES = [
    (2, 16, 19, 23, 40, 3, 5, 2),
    (1, 32, 14, 14, 70, 5, 5, 1),
    (2, 64, 30, 30, 64, 7, 7, 2),
    (3, 8, 17, 21, 33, 4, 3, (3, 1)),
    (2, 3, 47, 45, 37, 11, 11, 4),
    (1, 96, 12, 12, 256, 5, 5, (1, 2)),
    (2, 5, 13, 17, 20, 3, 2, (2, 1)),
]


def _shape(t, dt):
    return workloads.ConvShape("nhwc", *t, dt)


def _nhwc(a):
    return np.ascontiguousarray(a.transpose(0, 2, 3, 1))


@pytest.mark.parametrize("width", [2, 4])
@pytest.mark.parametrize("t", SHAPES, ids=str)
def test_pack_nhwc_bits(t, width, orc):
    import torch
    dev = device()
    N, Ci, Hi, Wi, Co, Hf, Wf, s = t
    note(f"pack nhwc {t} width={width}")
    ut = np.uint16 if width == 2 else np.uint32
    rng = np.random.default_rng(23 + width)
    x = rng.integers(0, np.iinfo(ut).max, size=(N, Hi, Wi, Ci), dtype=ut, endpoint=True)
    got = m.pack_nhwc(to_dev(x.view(np.int16 if width == 2 else np.int32), dev), Hf, Wf, s)
    got = got.cpu().numpy().view(ut)
    ref = orc.im2win_pack_nhwc(x, Hf, Wf, s)
    assert got.shape == ref.shape and np.array_equal(got, ref)
    torch.cuda.synchronize()


def _run(sh, x, w, ws_kind):
    import torch
    dev = device()
    ws = None
    if ws_kind is not None:
        n_img = sh.N if ws_kind == "full" else 1
        nb = m.nhwc_workspace_bytes(n_img, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s,
                                    sh.elem_bytes)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    y = m.conv2d_nhwc(to_dev(_nhwc(x), dev), to_dev(w, dev), sh.s, ws=ws).cpu().numpy()
    torch.cuda.synchronize()
    return np.ascontiguousarray(y.transpose(0, 3, 1, 2))


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("t", SHAPES, ids=str)
def test_conv_nhwc(t, dt, orc):
    sh = _shape(t, dt)
    x, w = workloads.make_inputs(sh, seed=61)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    xi, wi = workloads.make_inputs(sh, seed=62, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    for kind in (None, "full", "one"):
        note(f"conv nhwc {sh.describe()} ws={kind}")
        assert_within(_run(sh, x, w, kind), ref, absd, TOL[dt], f"{sh.describe()} ws={kind}")
        assert_exact(_run(sh, xi, wi, kind), refi, f"{sh.describe()} ws={kind} integer")


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_conv_nhwc_special_values(dt, orc):
    """Infinities and NaN reach exactly the outputs whose windows hold them
    on the matrix-core path (window runs of whole 16-byte slices)."""
    sh = _shape((2, 16, 13, 15, 40, 3, 5, 2), dt)
    x, w = workloads.make_inputs(sh, seed=63)
    x[0, 3, 4, 5] = np.inf
    x[1, 15, 12, 14] = -np.inf
    x[1, 0, 0, 0] = np.nan
    w = np.abs(w) + np.asarray(0.25, dtype=w.dtype)
    ref = orc.conv_direct(x, w, sh.s)
    note(f"conv nhwc special values {sh.describe()}")
    y = _run(sh, x, w, "full").astype(np.float64)
    assert np.array_equal(np.isnan(y), np.isnan(ref))
    assert np.array_equal(np.isposinf(y), np.isposinf(ref))
    assert np.array_equal(np.isneginf(y), np.isneginf(ref))


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("t", [SHAPES[4], SHAPES[6], SHAPES[3]], ids=str)
def test_conv_nhwc_padded_workspace_bits(t, dt, orc):
    """After a materialised call over the whole batch the workspace holds
    the filter rows and the im2win tensor with each column's Hf*Ci run padded
    with zeros to the pitch (Hf*Ci rounded up to 32 bytes): stripped of the
    padding, they are the oracle's NHWC transform and the filter in window
    order, bit for bit."""
    import torch
    dev = device()
    sh = _shape(t, dt)
    N, Ci, Hi, Wi, Co, Hf, Wf = sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf
    e = sh.elem_bytes
    x, w = workloads.make_inputs(sh, seed=64, mode="int")
    Ho, _ = m.output_dims(Hi, Wi, Hf, Wf, sh.s)
    HC = Hf * Ci
    q = 32 // e
    pitch = -(-HC // q) * q
    fb = -(-Co * Wf * pitch * e // 256) * 256
    nb = m.nhwc_workspace_bytes(N, Ci, Hi, Wi, Co, Hf, Wf, sh.s, e)
    assert nb == fb + N * Ho * Wi * pitch * e
    ws = torch.full((nb,), 0x5A, dtype=torch.uint8, device=dev)
    note(f"nhwc padded workspace {sh.describe()}")
    y = m.conv2d_nhwc(to_dev(_nhwc(x), dev), to_dev(w, dev), sh.s, ws=ws).cpu().numpy()
    assert_exact(np.ascontiguousarray(y.transpose(0, 3, 1, 2)), orc.conv_direct(x, w, sh.s),
                 sh.describe())
    ut = np.uint16 if e == 2 else np.uint32
    b = ws.cpu().numpy()
    wr = b[:Co * Wf * pitch * e].view(ut).reshape(Co, Wf, pitch)
    t_ = b[fb:].view(ut).reshape(N, Ho, Wi, pitch)
    xw = np.ascontiguousarray(w.transpose(0, 3, 2, 1)).view(ut).reshape(Co, Wf, HC)
    pk = orc.im2win_pack_nhwc(_nhwc(x).view(ut), Hf, Wf, sh.s).reshape(N, Ho, Wi, HC)
    assert np.array_equal(wr[..., :HC], xw) and not wr[..., HC:].any()
    assert np.array_equal(t_[..., :HC], pk) and not t_[..., HC:].any()
    torch.cuda.synchronize()


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("t", [SHAPES[0], SHAPES[4]], ids=str)
def test_conv_nhwc_materialised_x_at_element_offset(t, dt, orc):
    """x one element past a 16-byte boundary: the pack reads element by
    element (unpadded runs, Ci = 16, and padded ones, Ci = 3) and the GEMM
    runs on the packed tensor as for aligned x. Exact on integers."""
    import torch
    dev = device()
    sh = _shape(t, dt)
    xi, wi = workloads.make_inputs(sh, seed=65, mode="int")
    xn = _nhwc(xi)
    buf = torch.empty(xn.size + 1, dtype=torch.float16 if dt == "f16" else torch.float32,
                      device=dev)
    x_off = buf[1:].view(xn.shape)
    x_off.copy_(to_dev(xn, dev))
    assert x_off.data_ptr() % 16 != 0
    nb = m.nhwc_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, sh.elem_bytes)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    note(f"conv nhwc materialised, x at an element offset {sh.describe()}")
    y = m.conv2d_nhwc(x_off, to_dev(wi, dev), sh.s, ws=ws).cpu().numpy()
    assert_exact(np.ascontiguousarray(y.transpose(0, 3, 1, 2)), orc.conv_direct(xi, wi, sh.s),
                 f"{sh.describe()} x offset")
    torch.cuda.synchronize()


NHWC_FULL = ["cv5_f32_n1", "cv1_f32_n32", "cv5_f16_n128", "cv3_f16_n64", "cv4_f16_n64",
             "cv2_f32_n32"]


@pytest.mark.slow
@pytest.mark.parametrize("key", NHWC_FULL)
def test_conv_nhwc_full_size_every_output(key, orc):
    """The benchmark layers in NHWC at full size, as bench.py times them:
    materialised over the whole batch (window runs padded for the Ci = 3
    layers), and for cv5 fp16 the fused kernel with a prepacked filter.
    Every output against the oracle on small-integer inputs (exact), into an
    output pre-filled with NaN."""
    import torch
    dev = device()
    sh = workloads.BY_KEY[key]
    x, w = workloads.make_inputs(sh, seed=1, mode="int")
    note(f"nhwc full size {sh.describe()}: oracle")
    ref = np.ascontiguousarray(orc.conv_direct(x, w, sh.s).transpose(0, 2, 3, 1))
    xt, wt = to_dev(_nhwc(x), dev), to_dev(w, dev)
    y = torch.full(ref.shape, float("nan"), dtype=torch.float32, device=dev)
    nb = m.nhwc_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, sh.elem_bytes)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    note(f"conv nhwc materialised full {sh.describe()}")
    m.conv2d_nhwc(xt, wt, sh.s, ws=ws, out=y)
    assert_exact(y.cpu().numpy(), ref, f"{sh.describe()} nhwc materialised")
    del ws
    if key == "cv5_f16_n128":
        nb = m.nhwc_fused_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s)
        fws = torch.empty(nb, dtype=torch.uint8, device=dev)
        y.fill_(float("nan"))
        note(f"conv nhwc fused full {sh.describe()}")
        m.conv2d_nhwc_fused(xt, wt, sh.s, fws=fws, out=y)
        assert_exact(y.cpu().numpy(), ref, f"{sh.describe()} nhwc fused")
    torch.cuda.synchronize()


# Shapes of the fused NHWC kernel (resident input, prepacked filter): the
# cv5 layer, two channel tiles with Wi and Wo odd, row stride 2, a channel
# count that pads its last quad, 13- and 10-block one-row tiles, column
# stride 2, and the NHWC pack shape above.
RES_NHWC = [
    (3, 96, 24, 24, 256, 5, 5, 1),
    (2, 64, 17, 15, 512, 3, 5, 1),
    (2, 56, 21, 23, 256, 3, 5, (2, 1)),
    (1, 88, 13, 9, 256, 4, 5, 1),
    (2, 32, 6, 200, 256, 5, 5, 1),
    (1, 32, 5, 160, 256, 3, 9, 1),
    (2, 32, 20, 24, 256, 3, 2, (1, 2)),
    (1, 96, 12, 12, 256, 5, 5, (1, 2)),
]


def _run_fused(sh, x, w, out_nan=True):
    import torch
    dev = device()
    nb = m.nhwc_fused_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s)
    fws = torch.empty(nb, dtype=torch.uint8, device=dev)
    Ho, Wo = m.output_dims(sh.Hi, sh.Wi, sh.Hf, sh.Wf, sh.s)
    out = torch.full((sh.N, Ho, Wo, sh.Co), float("nan"), dtype=torch.float32, device=dev)
    y = m.conv2d_nhwc_fused(to_dev(_nhwc(x), dev), to_dev(w, dev), sh.s, fws=fws, out=out)
    y = y.cpu().numpy()
    torch.cuda.synchronize()
    return np.ascontiguousarray(y.transpose(0, 3, 1, 2))


@pytest.mark.parametrize("t", RES_NHWC, ids=str)
def test_conv_nhwc_fused(t, orc, knob):
    """The fused NHWC fp16 call on the resident-input kernel: exact on
    integer inputs, within tolerance on uniform ones, every output written
    (NaN-filled output), the same bits on a repeated call; with the kernel
    switched off (f16_res=-1) the call takes the direct kernel and gives the
    same integers."""
    sh = _shape(t, "f16")
    device()
    name = lambda: m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, 2,
                                      "nhwc_prepacked")
    assert name() == "conv_f16_res_kernel"
    x, w = workloads.make_inputs(sh, seed=71)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    xi, wi = workloads.make_inputs(sh, seed=72, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    note(f"conv nhwc fused {sh.describe()}")
    a = _run_fused(sh, x, w)
    assert_within(a, ref, absd, TOL["f16"], sh.describe())
    assert np.array_equal(_run_fused(sh, x, w), a)
    assert_exact(_run_fused(sh, xi, wi), refi, f"{sh.describe()} integer")
    knob("f16_res", -1)
    assert name() == "conv_direct_nhwc_kernel"
    assert_exact(_run_fused(sh, xi, wi), refi, f"{sh.describe()} integer, direct kernel")


def test_conv_nhwc_fused_special_values(orc):
    """Infinities and NaN reach exactly the outputs whose windows hold them
    through the fused NHWC kernel (its zero octets and padded K steps add
    nothing)."""
    sh = _shape((2, 88, 24, 24, 256, 5, 5, 1), "f16")
    device()
    assert m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, 2,
                              "nhwc_prepacked") == "conv_f16_res_kernel"
    x, w = workloads.make_inputs(sh, seed=73)
    x[0, 1, 4, 5] = np.inf
    x[1, 2, 7, 10] = -np.inf
    x[0, 0, 0, 6] = np.nan
    x[1, sh.Ci - 1, sh.Hi - 1, sh.Wi - 1] = np.inf
    w = (np.abs(w.astype(np.float32)) + np.float32(0.25)).astype(w.dtype)
    ref = orc.conv_direct(x, w, sh.s)
    fin = np.isfinite(ref)
    _, absd = orc.conv_direct(np.where(np.isfinite(x), x, 0).astype(x.dtype), w, sh.s,
                              with_absdot=True)
    note(f"conv nhwc fused special values {sh.describe()}")
    y = _run_fused(sh, x, w).astype(np.float64)
    assert np.array_equal(np.isnan(y), np.isnan(ref))
    assert np.array_equal(np.isposinf(y), np.isposinf(ref))
    assert np.array_equal(np.isneginf(y), np.isneginf(ref))
    assert_within(y[fin], ref[fin], absd[fin], TOL["f16"], "finite outputs")


def test_conv_nhwc_fused_outside_envelope_and_errors(orc):
    """Outside the kernel's envelope (Co not a multiple of 256) the fused
    NHWC call takes the direct kernel; without a workspace too; a workspace
    that is too small is refused before anything runs."""
    import torch
    dev = device()
    sh = _shape((2, 16, 13, 14, 40, 3, 3, 1), "f16")
    assert m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, 2,
                              "nhwc_prepacked") == "conv_direct_nhwc_kernel"
    xi, wi = workloads.make_inputs(sh, seed=74, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    note(f"conv nhwc fused fallback {sh.describe()}")
    assert_exact(_run_fused(sh, xi, wi), refi, sh.describe())
    xt, wt = to_dev(_nhwc(xi), dev), to_dev(wi, dev)
    y = m.conv2d_nhwc_fused(xt, wt, sh.s).cpu().numpy()
    assert_exact(np.ascontiguousarray(y.transpose(0, 3, 1, 2)), refi, f"{sh.describe()} no fws")
    sh2 = _shape((1, 96, 12, 12, 256, 5, 5, 1), "f16")
    nb = m.nhwc_fused_workspace_bytes(sh2.N, sh2.Ci, sh2.Hi, sh2.Wi, sh2.Co, sh2.Hf, sh2.Wf, sh2.s)
    x2, w2 = workloads.make_inputs(sh2, seed=75, mode="int")
    small = torch.empty(nb - 16, dtype=torch.uint8, device=dev)
    with pytest.raises(RuntimeError):
        m.conv2d_nhwc_fused(to_dev(_nhwc(x2), dev), to_dev(w2, dev), sh2.s, fws=small)
    torch.cuda.synchronize()
