"""im2win_pack on the GPU against the oracle's transform: bit for bit."""
import numpy as np
import pytest

import memory_efficient_im2win_amd as m
import workloads
from parity import device, note, to_dev

pytestmark = pytest.mark.gpu

# (N, Ci, Hi, Wi, Hf, Wf, s): row lengths that are odd/even, strides above and
# below the filter height, one output row, many rows per workgroup.
SHAPES = [
    (1, 3, 3, 3, 2, 2, 1),
    (2, 3, 19, 23, 3, 5, 2),
    (1, 5, 11, 8, 2, 5, 3),
    (3, 2, 31, 17, 7, 7, 1),
    (1, 4, 9, 40, 9, 3, 2),       # Ho = 1
    (2, 1, 50, 13, 3, 2, 5),      # s > Hf
    (1, 2, 64, 301, 11, 11, 4),
    (1, 1, 3, 4001, 3, 3, 1),     # long rows
]


@pytest.mark.parametrize("shape", SHAPES, ids=str)
@pytest.mark.parametrize("width", [2, 4])
def test_pack_bits_match_oracle(shape, width, orc):
    dev = device()
    N, Ci, Hi, Wi, Hf, Wf, s = shape
    note(f"pack {shape} width={width}")
    ut = np.uint16 if width == 2 else np.uint32
    rng = np.random.default_rng(hash((shape, width)) & 0xFFFF)
    x = rng.integers(0, np.iinfo(ut).max, size=(N, Ci, Hi, Wi), dtype=ut, endpoint=True)
    import torch
    xt = to_dev(x.view(np.int16 if width == 2 else np.int32), dev)
    got = m.pack(xt, Hf, Wf, s).cpu().numpy().view(ut)
    ref = orc.im2win_pack(x, Hf, Wf, s)
    assert got.shape == ref.shape and np.array_equal(got, ref)
    torch.cuda.synchronize()


def test_pack_leaves_bytes_outside_the_tensor_alone(orc):
    import torch
    dev = device()
    N, Ci, Hi, Wi, Hf, Wf, s = 2, 3, 17, 21, 5, 3, 2
    note("pack guard bands")
    x = np.random.default_rng(2).uniform(-1, 1, (N, Ci, Hi, Wi)).astype(np.float32)
    nb = m.workspace_bytes(N, Ci, Hi, Wi, Hf, Wf, s, 4)
    n = nb // 4
    big = torch.full((n + 2 * 37,), float("nan"), dtype=torch.float32, device=dev)
    ref = orc.im2win_pack(x, Hf, Wf, s)
    out = big[37:37 + n].view(ref.shape)
    m.pack(to_dev(x, dev), Hf, Wf, s, out=out)
    b = big.cpu().numpy()
    assert np.isnan(b[:37]).all() and np.isnan(b[37 + n:]).all()
    assert np.array_equal(b[37:37 + n].reshape(ref.shape).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("key", ["cv5_f32_n1", "cv1_f32_n32", "cv5_f16_n128", "cv3_f16_n64",
                                 "cv4_f16_n64", "cv2_f32_n32"])
def test_pack_full_size(key, orc):
    """The benchmark layers at full batch; images 0, N-1 and one in between
    are compared with the oracle bit for bit, the rest by their size."""
    import torch
    dev = device()
    sh = workloads.BY_KEY[key]
    note(f"pack full size {sh.describe()}")
    x, _ = workloads.make_inputs(sh, seed=0)
    xt = to_dev(x, dev)
    ws = m.pack(xt, sh.Hf, sh.Wf, sh.s)
    assert ws.numel() * ws.element_size() == m.workspace_bytes(
        sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Hf, sh.Wf, sh.s, sh.elem_bytes)
    for n in sorted({0, sh.N // 2, sh.N - 1}):
        got = ws[n:n + 1].cpu().numpy()
        ref = orc.im2win_pack(x[n:n + 1], sh.Hf, sh.Wf, sh.s)
        assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), n
    del ws
    torch.cuda.synchronize()
