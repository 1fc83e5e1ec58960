"""The baselines the GPU page compares im2win against, built here: the
im2col transform (bitwise against the oracle's), im2col + matrix-core GEMM
and direct convolution (against the fp64 oracle: exact for small integers,
otherwise |y - y_oracle| <= tol * sum|x*w|)."""
import numpy as np
import pytest

import memory_efficient_im2win_amd as m
import workloads
from parity import TOL, assert_exact, assert_within, device, note, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [
    (2, 3, 19, 23, 40, 3, 5, 2),
    (1, 13, 21, 17, 70, 2, 3, (1, 2)),
    (2, 16, 14, 14, 64, 5, 5, 1),
    (1, 3, 47, 45, 37, 11, 11, 4),
    (3, 6, 23, 11, 33, 4, 6, (3, 1)),
    (2, 8, 12, 40, 130, 1, 1, 1),
    (3, 2, 7, 9, 200, 3, 3, 1),         # K below one stage of the GEMM
    (2, 24, 20, 20, 64, 5, 5, 1),       # K across several stages and a partial last one
]


def _shape(t, dt):
    return workloads.ConvShape("baseline", *t, dt)


@pytest.mark.parametrize("width", [2, 4])
@pytest.mark.parametrize("t", SHAPES, ids=str)
def test_im2col_pack_bits(t, width, orc):
    import torch
    dev = device()
    N, Ci, Hi, Wi, Co, Hf, Wf, s = t
    note(f"im2col pack {t} width={width}")
    ut = np.uint16 if width == 2 else np.uint32
    rng = np.random.default_rng(17 + width)
    x = rng.integers(0, np.iinfo(ut).max, size=(N, Ci, Hi, Wi), dtype=ut, endpoint=True)
    got = m.im2col(to_dev(x.view(np.int16 if width == 2 else np.int32), dev), Hf, Wf, s)
    got = got.cpu().numpy().view(ut)
    step = 32 // width
    KP = -(-(Ci * Hf * Wf) // step) * step
    ref = orc.im2col_pack(x, Hf, Wf, s, KP=KP)
    assert got.shape == ref.shape and np.array_equal(got, ref)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("t", SHAPES, ids=str)
def test_conv_im2col_gemm(t, dt, orc):
    import torch
    dev = device()
    sh = _shape(t, dt)
    x, w = workloads.make_inputs(sh, seed=51)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    note(f"conv im2col+GEMM {sh.describe()}")
    y = m.conv2d_im2col(to_dev(x, dev), to_dev(w, dev), sh.s).cpu().numpy()
    assert_within(y, ref, absd, TOL[dt], sh.describe())
    xi, wi = workloads.make_inputs(sh, seed=52, mode="int")
    yi = m.conv2d_im2col(to_dev(xi, dev), to_dev(wi, dev), sh.s).cpu().numpy()
    assert_exact(yi, orc.conv_direct(xi, wi, sh.s), sh.describe())
    torch.cuda.synchronize()


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_conv_im2col_in_chunks(dt, orc):
    """A workspace for one image's rows: the batch goes in single-image chunks."""
    import torch
    dev = device()
    sh = _shape((3, 6, 20, 24, 70, 5, 3, 2), dt)
    x, w = workloads.make_inputs(sh, seed=53, mode="int")
    full = m.im2col_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, sh.elem_bytes)
    one = m.im2col_workspace_bytes(1, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, sh.elem_bytes)
    assert one < full
    note(f"conv im2col+GEMM chunked {sh.describe()}")
    ws = torch.empty(one, dtype=torch.uint8, device=dev)
    y = m.conv2d_im2col(to_dev(x, dev), to_dev(w, dev), sh.s, ws=ws).cpu().numpy()
    assert_exact(y, orc.conv_direct(x, w, sh.s), sh.describe())
    with pytest.raises(m.Im2winError):
        m.conv2d_im2col(to_dev(x, dev), to_dev(w, dev), sh.s, ws=ws[: one - 16])


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("t", SHAPES, ids=str)
def test_conv_direct(t, dt, orc):
    import torch
    dev = device()
    sh = _shape(t, dt)
    x, w = workloads.make_inputs(sh, seed=54)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    note(f"conv direct {sh.describe()}")
    assert_within(m.conv2d_direct(to_dev(x, dev), to_dev(w, dev), sh.s).cpu().numpy(), ref, absd,
                  TOL[dt], sh.describe())
    xi, wi = workloads.make_inputs(sh, seed=55, mode="int")
    assert_exact(m.conv2d_direct(to_dev(xi, dev), to_dev(wi, dev), sh.s).cpu().numpy(),
                 orc.conv_direct(xi, wi, sh.s), sh.describe())
    torch.cuda.synchronize()


@pytest.mark.slow
@pytest.mark.parametrize("key", ["cv1_f32_n32", "cv5_f16_n128", "cv4_f16_n64"])
def test_baselines_full_size(key, orc):
    """The benchmark layers through im2col + GEMM (cv4: 4.8 GB of im2col
    rows, in chunks below 4 GiB) and, for cv1 and cv5, direct convolution:
    every output against the oracle on small-integer inputs (exact), into an
    output pre-filled with NaN."""
    import torch
    dev = device()
    sh = workloads.BY_KEY[key]
    x, w = workloads.make_inputs(sh, seed=1, mode="int")
    note(f"baselines full size {sh.describe()}: oracle")
    ref = orc.conv_direct(x, w, sh.s)
    xt, wt = to_dev(x, dev), to_dev(w, dev)
    y = torch.full(ref.shape, float("nan"), dtype=torch.float32, device=dev)
    note(f"conv im2col+GEMM full {sh.describe()}")
    m.conv2d_im2col(xt, wt, sh.s, out=y)
    assert_exact(y.cpu().numpy(), ref, f"{sh.describe()} im2col")
    if key != "cv4_f16_n64":
        note(f"conv direct full {sh.describe()}")
        y.fill_(float("nan"))
        m.conv2d_direct(xt, wt, sh.s, out=y)
        assert_exact(y.cpu().numpy(), ref, f"{sh.describe()} direct")
    torch.cuda.synchronize()
