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

# (N, Ci, Hi, Wi, Co, Hf, Wf, s): Ci a multiple of 16 (matrix-core path in
# both precisions), of 8 only (fp32 matrix cores, fp16 direct), and neither.
SHAPES = [
    (2, 16, 19, 23, 40, 3, 5, 2),
    (1, 32, 14, 14, 70, 5, 5, 1),
    (2, 64, 30, 30, 64, 7, 7, 2),
    (3, 8, 17, 21, 33, 4, 3, (3, 1)),
    (2, 3, 47, 45, 37, 11, 11, 4),
    (1, 96, 12, 12, 256, 5, 5, (1, 2)),
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


@pytest.mark.slow
@pytest.mark.parametrize("key", ["cv4_f16_n64", "cv5_f16_n128"])
def test_conv_nhwc_full_size_sampled(key, orc):
    import torch
    dev = device()
    sh = workloads.BY_KEY[key]
    x, w = workloads.make_inputs(sh, seed=1, mode="int")
    Ho, Wo = m.output_dims(sh.Hi, sh.Wi, sh.Hf, sh.Wf, sh.s)
    idx = workloads.sample_output_indices(sh, Ho, Wo, 2000)
    ref, _ = orc.conv_points(x, w, sh.s, idx)
    nb = m.nhwc_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, sh.elem_bytes)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    note(f"conv nhwc full {sh.describe()}")
    y = m.conv2d_nhwc(to_dev(_nhwc(x), dev), to_dev(w, dev), sh.s, ws=ws)
    got = y.permute(0, 3, 1, 2).reshape(-1)[torch.from_numpy(idx).to(dev)].cpu().numpy()
    assert_exact(got, ref, sh.describe())
    torch.cuda.synchronize()
