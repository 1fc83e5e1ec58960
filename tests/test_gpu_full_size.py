"""The benchmark layers (Table I of "Enabling Memory-efficient Im2win
Convolution with Multi-precision Support on GPU CUDA and Tensor Cores") at
full size, in every launch configuration bench.py times, against the fp64
oracle output by output.

Bar: bit-exact on small-integer inputs; |y - y_oracle| <= tol * sum|x*w| for
every output on uniform inputs (tol 1e-5 fp32, 2e-3 fp16). Outputs are
pre-filled with NaN, so a tile a kernel never writes fails the comparison.
"""
import numpy as np
import pytest

import memory_efficient_im2win_amd as m
import workloads
from parity import TOL, assert_exact, assert_within, call, device, note, to_dev, workspace

pytestmark = pytest.mark.gpu

LAYERS = ["cv5_f32_n1", "cv1_f32_n32", "cv5_f16_n128", "cv3_f16_n64", "cv4_f16_n64",
          "cv2_f32_n32"]

# The modes bench.py times per precision: (name, workspace kind, knobs).
MODES = {
    "f32": [("fused", None, {}), ("fused_valu", None, {"f32_valu": 1}),
            ("materialized", "full", {})],
    "f16": [("fused", None, {}), ("prepacked", "filter", {}), ("materialized", "full", {})],
}


@pytest.mark.slow
@pytest.mark.parametrize("key", LAYERS)
@pytest.mark.parametrize("inputs", ["uniform", "int"])
def test_full_size_every_output(key, inputs, orc, knob):
    import torch
    dev = device()
    sh = workloads.BY_KEY[key]
    x, w = workloads.make_inputs(sh, seed=0 if inputs == "uniform" else 1, mode=inputs)
    note(f"full size {sh.describe()} {inputs}: oracle")
    if inputs == "uniform":
        ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    else:
        ref, absd = orc.conv_direct(x, w, sh.s), None
    xt, wt = to_dev(x, dev), to_dev(w, dev)
    y = torch.empty(ref.shape, dtype=torch.float32, device=dev)
    for name, kind, kn in MODES[sh.dtype]:
        for k, v in kn.items():
            knob(k, v)
        note(f"full size {sh.describe()} {inputs} mode={name}")
        y.fill_(float("nan"))
        call(sh, xt, wt, kind, dev, out=y)
        got = y.cpu().numpy()
        if inputs == "int":
            assert_exact(got, ref, f"{key} {name}")
        else:
            assert_within(got, ref, absd, TOL[sh.dtype], f"{key} {name}")
        for k in kn:
            knob(k, 0)
        del got
    torch.cuda.synchronize()


@pytest.mark.parametrize("t", [(1, 96, 24, 24, 256, 5, 5, 1), (64, 6, 20, 24, 40, 7, 7, 2),
                               (5, 3, 31, 29, 64, 7, 7, 2), (3, 8, 17, 16, 130, 3, 3, 1)],
                         ids=str)
@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_materialised_workspace_is_the_im2win_tensor(t, dt, orc):
    """A workspace of exactly im2win_workspace_bytes(N) runs the materialised
    mode over the whole batch: afterwards it holds the oracle's im2win tensor
    bit for bit (no filter or other data ahead of it), and the output is
    right. With room for k < N images it holds the last chunk's tensor."""
    import torch
    dev = device()
    sh = workloads.ConvShape("ws", *t, dt)
    x, w = workloads.make_inputs(sh, seed=70, mode="int")
    ref = orc.conv_direct(x, w, sh.s)
    pk = orc.im2win_pack(x, sh.Hf, sh.Wf, sh.s)
    ut = np.uint16 if dt == "f16" else np.uint32
    xt, wt = to_dev(x, dev), to_dev(w, dev)
    nb = m.workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Hf, sh.Wf, sh.s, sh.elem_bytes)
    assert nb == pk.size * sh.elem_bytes
    ws = torch.full((nb,), 0x5A, dtype=torch.uint8, device=dev)
    note(f"materialised workspace {sh.describe()} exact size")
    y = m.conv2d(xt, wt, sh.s, ws=ws)
    assert_exact(y.cpu().numpy(), ref, sh.describe())
    got = ws.cpu().numpy().view(ut).reshape(pk.shape)
    assert np.array_equal(got, pk.view(ut))
    if sh.N > 1:
        per = nb // sh.N
        k = max(1, (sh.N + 1) // 3)
        ws2 = torch.full((k * per + per - 1,), 0x5A, dtype=torch.uint8, device=dev)
        note(f"materialised workspace {sh.describe()} chunks of {k}")
        y2 = m.conv2d(xt, wt, sh.s, ws=ws2)
        assert_exact(y2.cpu().numpy(), ref, f"{sh.describe()} chunks of {k}")
        last0 = (sh.N - 1) // k * k
        nl = sh.N - last0
        got = ws2[:nl * per].cpu().numpy().view(ut).reshape((nl,) + pk.shape[1:])
        assert np.array_equal(got, pk[last0:].view(ut))
    torch.cuda.synchronize()


@pytest.mark.parametrize("key", LAYERS)
def test_repeat_calls_are_bitwise_identical(key, orc):
    """Every call of one mode on one layer gives the same bits (fixed
    summation order, no atomics): the small fp32 layer's K split included."""
    import torch
    dev = device()
    sh = workloads.BY_KEY[key]
    if sh.N > 32:
        sh = sh.with_batch(8)
    x, w = workloads.make_inputs(sh, seed=5)
    xt, wt = to_dev(x, dev), to_dev(w, dev)
    kinds = [None, "full"] + (["filter"] if sh.dtype == "f16" else [])
    for kind in kinds:
        note(f"repeat calls {sh.describe()} ws={kind}")
        ws = workspace(sh, kind, dev)
        a = call(sh, xt, wt, kind, dev, ws=ws)
        for _ in range(3):
            b = call(sh, xt, wt, kind, dev, ws=ws)
            assert torch.equal(a, b), f"{key} ws={kind}"
    torch.cuda.synchronize()


def test_fp32_kernel_names(knob):
    """The fp32 planner's choice as the kernel-name query reports it (it asks
    the device for occupancy)."""
    device()
    assert m.conv_kernel_name(32, 3, 227, 227, 96, 11, 11, 4, 4) == "conv_f32_mfma_kernel"
    assert m.conv_kernel_name(1, 96, 24, 24, 256, 5, 5, 1, 4) == "conv_f32_small_kernel"
    knob("f32_small", -1)
    assert m.conv_kernel_name(1, 96, 24, 24, 256, 5, 5, 1, 4) == "conv_f32_mfma_kernel"
    knob("f32_small", 0)
    assert m.conv_kernel_name(32, 3, 227, 227, 96, 11, 11, 4, 4, "materialized") == \
        "conv_f32_kernel"
    knob("f32_valu", 1)
    assert m.conv_kernel_name(32, 3, 227, 227, 96, 11, 11, 4, 4) == "conv_f32_kernel"
