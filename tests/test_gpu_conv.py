"""conv2d_im2win_fp32 / _fp16 on the GPU against the fp64 oracle.

Bar: bit-exact for small-integer inputs (every partial sum is an exact
integer below 2^24, so any summation order gives the same fp32 value);
otherwise |y - y_oracle| <= tol * sum|x*w| per output with tol 1e-5 (fp32)
and 2e-3 (fp16 inputs, fp32 accumulation).
"""
import numpy as np
import pytest

import memory_efficient_im2win_amd as m
import workloads
from parity import (TOL, WS_KINDS, assert_exact, assert_within, call, device, note, to_dev,
                    workspace)

pytestmark = pytest.mark.gpu

# (N, Ci, Hi, Wi, Co, Hf, Wf, s): several workgroup tiles with ragged tails in
# pixels and channels; each filter size the fp32 kernel specialises (11, 7, 5,
# 3) and the generic one; Ci and Co off the MFMA tile multiples.
SMALL = [
    (3, 5, 19, 19, 40, 3, 3, 1),
    (2, 3, 47, 45, 37, 11, 11, 4),
    (2, 16, 30, 29, 70, 7, 7, 2),
    (4, 24, 14, 14, 96, 5, 5, 1),
    (1, 13, 21, 17, 9, 2, 3, 2),      # rectangular, generic path
    (2, 8, 12, 40, 64, 1, 1, 1),      # 1x1
    (1, 3, 9, 9, 5, 9, 9, 1),         # filter covers the input: one output
    (2, 6, 23, 11, 33, 4, 6, 3),      # s < Hf, Wf; ragged (Hi-Hf) % s
    (1, 9, 16, 16, 17, 2, 2, 5),      # s > Hf, Wf
    (1, 64, 30, 30, 64, 7, 7, 2),     # cv4-like slice
    (1, 96, 12, 12, 256, 5, 5, 1),    # cv5-like slice
    (2, 3, 227, 227, 96, 11, 11, 4),  # cv1 images
]


def _ws(sh, kind, dev):
    return workspace(sh, kind, dev)


def _run(sh, mode, x, w, ws_kind=None):
    import torch
    dev = device()
    xt, wt = to_dev(x, dev), to_dev(w, dev)
    y = call(sh, xt, wt, ws_kind, dev)
    out = y.cpu().numpy()
    torch.cuda.synchronize()
    return out


def _shape(t, dt):
    return workloads.ConvShape("t", *t, dt)


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("t", SMALL, ids=str)
def test_conv_small_uniform(t, dt, orc):
    sh = _shape(t, dt)
    x, w = workloads.make_inputs(sh, seed=11)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    for kind in WS_KINDS:
        note(f"conv uniform {sh.describe()} ws={kind}")
        y = _run(sh, dt, x, w, kind)
        assert_within(y, ref, absd, TOL[dt], f"{sh.describe()} ws={kind}")


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("t", SMALL, ids=str)
def test_conv_small_integer_exact(t, dt, orc):
    sh = _shape(t, dt)
    x, w = workloads.make_inputs(sh, seed=12, mode="int")
    ref = orc.conv_direct(x, w, sh.s)
    for kind in WS_KINDS:
        note(f"conv integer {sh.describe()} ws={kind}")
        assert_exact(_run(sh, dt, x, w, kind), ref, f"{sh.describe()} ws={kind}")


@pytest.mark.parametrize("t", SMALL, ids=str)
def test_conv_f32_vector_alu_path(t, orc, knob):
    """fp32 on the vector-ALU kernel (the fallback of the matrix-core one)."""
    knob("f32_valu", 1)
    sh = _shape(t, "f32")
    x, w = workloads.make_inputs(sh, seed=16)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    for kind in (None, "one"):
        note(f"conv fp32 vector ALU {sh.describe()} ws={kind}")
        assert_within(_run(sh, "f32", x, w, kind), ref, absd, TOL["f32"], sh.describe())
    xi, wi = workloads.make_inputs(sh, seed=17, mode="int")
    note(f"conv fp32 vector ALU integer {sh.describe()}")
    assert_exact(_run(sh, "f32", xi, wi), orc.conv_direct(xi, wi, sh.s), sh.describe())


@pytest.mark.parametrize("t", [(1, 1, 12, 2000, 8, 11, 3, 1), (1, 2, 14, 1500, 4, 9, 5, (1, 2))],
                         ids=str)
def test_conv_f32_vector_alu_rows_past_lds(t, orc, knob):
    """Rows too long for the vector-ALU kernel's LDS (one im2win row set of a
    64-pixel tile above 64 KB): the call still gives the exact result, fused
    and from the materialised tensor (the planner declines and the generic
    kernel runs)."""
    knob("f32_valu", 1)
    sh = _shape(t, "f32")
    xi, wi = workloads.make_inputs(sh, seed=22, mode="int")
    ref = orc.conv_direct(xi, wi, sh.s)
    for kind in (None, "full"):
        note(f"conv fp32 vector ALU long rows {sh.describe()} ws={kind}")
        assert_exact(_run(sh, "f32", xi, wi, kind), ref, f"{sh.describe()} ws={kind}")


@pytest.mark.parametrize("ksplit", [1, 4, 8, 12])
@pytest.mark.parametrize("t", [(1, 96, 12, 12, 256, 5, 5, 1), (2, 16, 20, 20, 40, 3, 3, 1),
                               (3, 7, 26, 26, 33, 5, 5, 1), (1, 3, 40, 40, 20, 11, 11, 4),
                               (1, 5, 9, 9, 7, 3, 3, 2)], ids=str)
def test_conv_f32_k_split(t, ksplit, orc, knob):
    """The matrix-core fp32 kernel with K shared by 4, 8 or 12 waves of a
    workgroup (partial sums added through LDS in a fixed order; stages with
    fewer K pairs than waves included) and without a K split."""
    knob("f32_ksplit", ksplit)
    sh = _shape(t, "f32")
    x, w = workloads.make_inputs(sh, seed=18)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    note(f"conv fp32 ksplit={ksplit} {sh.describe()}")
    assert_within(_run(sh, "f32", x, w), ref, absd, TOL["f32"], sh.describe())
    xi, wi = workloads.make_inputs(sh, seed=19, mode="int")
    assert_exact(_run(sh, "f32", xi, wi), orc.conv_direct(xi, wi, sh.s), sh.describe())


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_conv_generic_fallback_large_filter(dt, orc):
    """A 13x13 filter over a wide row falls outside the tiled kernels' LDS
    budget in fp16; both precisions must still be right."""
    sh = _shape((1, 9, 20, 600, 7, 13, 13, 2), dt)
    x, w = workloads.make_inputs(sh, seed=13)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    for kind in WS_KINDS:
        note(f"conv large filter {sh.describe()} ws={kind}")
        assert_within(_run(sh, dt, x, w, kind), ref, absd, TOL[dt], sh.describe())


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_conv_special_values(dt, orc):
    """NaN and infinities propagate exactly to the outputs whose windows hold
    them (window padding never turns a neighbour's Inf into NaN)."""
    sh = _shape((2, 8, 13, 13, 9, 3, 3, 1), dt)
    x, w = workloads.make_inputs(sh, seed=14)
    x[0, 1, 4, 5] = np.inf
    x[1, 7, 12, 12] = -np.inf
    x[1, 0, 0, 0] = np.nan
    w = np.abs(w) + np.asarray(0.25, dtype=w.dtype)  # no zero taps, fixed signs
    ref = orc.conv_direct(x, w, sh.s)
    note(f"conv special values {sh.describe()}")
    for kind in WS_KINDS:
        y = _run(sh, dt, x, w, kind).astype(np.float64)
        assert np.array_equal(np.isnan(y), np.isnan(ref))
        assert np.array_equal(np.isposinf(y), np.isposinf(ref))
        assert np.array_equal(np.isneginf(y), np.isneginf(ref))
        fin = np.isfinite(ref)
        _, absd = orc.conv_direct(np.where(np.isfinite(x), x, 0).astype(x.dtype), w, sh.s,
                                  with_absdot=True)
        assert_within(y[fin], ref[fin], absd[fin], TOL[dt], "finite outputs")


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_conv_writes_only_its_output(dt, orc):
    """Outputs and workspaces sit between NaN / 0x7F guard bands that no
    call may touch, in every workspace mode."""
    import torch
    dev = device()
    sh = _shape((2, 12, 17, 15, 41, 3, 5, 2), dt)
    x, w = workloads.make_inputs(sh, seed=15)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    n = ref.size
    note(f"conv guard bands {sh.describe()}")
    xt, wt = to_dev(x, dev), to_dev(w, dev)
    for kind in WS_KINDS:
        big = torch.full((n + 2 * 129,), float("nan"), dtype=torch.float32, device=dev)
        out = big[129:129 + n].view(ref.shape)
        ws = _ws(sh, kind, dev)
        wsbig = None
        if ws is None:
            m.conv2d(xt, wt, sh.s, out=out)
        else:
            nb = ws.numel()
            wsbig = torch.full((nb + 4096,), 0x7F, dtype=torch.uint8, device=dev)
            if kind == "filter":
                m.conv2d_fused(xt, wt, sh.s, fws=wsbig, fws_bytes=nb, out=out)
            else:
                m.conv2d(xt, wt, sh.s, ws=wsbig, ws_bytes=nb, out=out)
        b = big.cpu().numpy()
        assert np.isnan(b[:129]).all() and np.isnan(b[129 + n:]).all()
        assert_within(b[129:129 + n].reshape(ref.shape), ref, absd, TOL[dt], f"guarded output {kind}")
        if wsbig is not None:
            assert (wsbig[nb:].cpu().numpy() == 0x7F).all()


@pytest.mark.parametrize("nw", [4, 8, 12])
@pytest.mark.parametrize("t", [(2, 3, 227, 227, 96, 11, 11, 4), (1, 16, 30, 30, 64, 7, 7, 2),
                               (3, 7, 26, 26, 33, 5, 5, 1), (2, 10, 19, 37, 130, 3, 3, 2),
                               (2, 5, 31, 40, 48, 3, 7, 2), (1, 8, 20, 33, 40, 7, 3, 3)], ids=str)
def test_conv_f32_matrix_waves(t, nw, orc, knob):
    """The fp32 matrix-core kernel forced to 4, 8 and 12 waves per workgroup
    (32*NW-pixel tiles: different tilings, row counts and item streams)."""
    knob("f32_ksplit", 1)
    knob("f32_nw", nw)
    sh = _shape(t, "f32")
    x, w = workloads.make_inputs(sh, seed=20)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    note(f"conv fp32 NW={nw} {sh.describe()}")
    assert_within(_run(sh, "f32", x, w), ref, absd, TOL["f32"], sh.describe())
    xi, wi = workloads.make_inputs(sh, seed=21, mode="int")
    assert_exact(_run(sh, "f32", xi, wi), orc.conv_direct(xi, wi, sh.s), sh.describe())


@pytest.mark.parametrize("kn", [{"f32_wco": 1}, {"f32_wco": 2}, {"f32_wco": 3}, {"f32_wco": 4},
                                {"f32_cb": 1}, {"f32_cb": 3}, {"f32_occ": 2}], ids=str)
@pytest.mark.parametrize("t", [(2, 3, 227, 227, 96, 11, 11, 4), (2, 16, 30, 30, 130, 5, 5, (2, 1))],
                         ids=str)
def test_conv_f32_matrix_tilings(t, kn, orc, knob):
    """The fp32 matrix-core kernel with its channel tile (32*WCO channels),
    channels per stage and workgroups per CU forced (the small-problem kernel
    off, so the tiled kernel runs)."""
    knob("f32_small", -1)
    for k, v in kn.items():
        knob(k, v)
    sh = _shape(t, "f32")
    device()
    assert m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, 4) == \
        "conv_f32_mfma_kernel"
    x, w = workloads.make_inputs(sh, seed=22)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    note(f"conv fp32 matrix tiling {kn} {sh.describe()}")
    assert_within(_run(sh, "f32", x, w), ref, absd, TOL["f32"], sh.describe())
    xi, wi = workloads.make_inputs(sh, seed=23, mode="int")
    assert_exact(_run(sh, "f32", xi, wi), orc.conv_direct(xi, wi, sh.s), sh.describe())


@pytest.mark.parametrize("env", [{"f16_wpx": 8}, {"f16_wpx": 1}, {"f16_nwh": 3}], ids=str)
@pytest.mark.parametrize("t", [(1, 64, 30, 30, 64, 7, 7, 2), (2, 24, 14, 14, 96, 5, 5, 1),
                               (2, 3, 47, 45, 37, 7, 7, 2), (2, 12, 26, 40, 70, 3, 7, 2),
                               (1, 16, 22, 19, 40, 5, 2, 1)], ids=str)
def test_conv_f16_fused_tilings(t, env, orc, knob):
    """The fused fp16 kernel with forced waves along pixels and filter stages
    per channel group, with and without the prepacked filter (the thin-layer
    and wide-tile kernels switched off, so the prepacked calls reach it)."""
    for k, v in env.items():
        knob(k, v)
    knob("f16_thin", -1)
    knob("f16_wide", -1)
    sh = _shape(t, "f16")
    x, w = workloads.make_inputs(sh, seed=22)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    for kind in (None, "filter"):
        note(f"conv fp16 {env} {sh.describe()} ws={kind}")
        assert_within(_run(sh, "f16", x, w, kind), ref, absd, TOL["f16"], sh.describe())
    xi, wi = workloads.make_inputs(sh, seed=23, mode="int")
    assert_exact(_run(sh, "f16", xi, wi, "filter"), orc.conv_direct(xi, wi, sh.s), sh.describe())


# Shapes the row-staged fp16 kernel takes with a prepacked filter (even column
# stride, Wf <= 8, Wi a multiple of 8, Ci even): several tiles and channel
# tiles, image breaks inside tiles, rectangles, Wf = 8 (no padded taps).
# Without a workspace, 8 waves gather the filter with dword loads up to 16
# per thread and stage, past that (and with 4 waves on the 7x7 shapes) one
# 16-byte entry per thread.
ROWS = [
    (2, 16, 30, 32, 70, 7, 7, 2),
    (1, 64, 40, 40, 64, 7, 7, 2),
    (3, 6, 23, 24, 33, 3, 5, (1, 2)),
    (2, 4, 17, 48, 40, 4, 8, (3, 4)),
    (4, 2, 9, 16, 64, 2, 2, 2),
    (5, 4, 12, 16, 64, 3, 3, 2),
    (2, 8, 20, 64, 128, 5, 3, (2, 2)),
    (2, 2, 65, 64, 40, 3, 3, 2),      # tiles aligned to images
    (2, 4, 24, 32, 64, 16, 8, 2),     # 16 dword gather loads per thread (8 waves)
    (2, 4, 24, 32, 64, 17, 8, 2),     # 17 would be needed: per-entry gather
]


def _filter_bytes(sh):
    return m.fused_workspace_bytes(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s)


def _layout_bytes(sh):
    """The two prepacked fp16 filter layouts, worked out independently of the
    library: (channel, filter row) slices of 8 taps for 64-channel tiles, and
    channel-interleaved 16-byte entries (8 input channels of a tap, taps
    rounded up to even) for 128-channel tiles."""
    slices = sh.Ci * sh.Hf * ((sh.Co + 63) // 64 * 64) * 16
    inter = -(-sh.Ci // 8) * ((sh.Hf * sh.Wf + 1) & ~1) * ((sh.Co + 127) // 128 * 128) * 16
    return slices, inter


@pytest.mark.parametrize("nwv", [8, 4])
@pytest.mark.parametrize("t", ROWS, ids=str)
def test_conv_f16_row_staged(t, nwv, orc, knob):
    """The fp16 kernel that copies input rows to LDS with direct loads (used
    with a prepacked filter): uniform and integer inputs, 8 and 4 waves. The
    filter workspace holds either layout, whatever the knobs. (The row-reuse
    kernel, which takes most of these shapes by default, is switched off.)"""
    knob("f16_reuse", -1)
    knob("f16_rows_nwv", nwv)
    sh = _shape(t, "f16")
    on = _filter_bytes(sh)
    knob("f16_rows", -1)
    knob("f16_thin", -1)
    off = _filter_bytes(sh)
    knob("f16_rows", 0)
    knob("f16_thin", 0)
    need = max(_layout_bytes(sh))
    assert on == off == -(-need // 256) * 256, (on, off, need)
    x, w = workloads.make_inputs(sh, seed=40)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    xi, wi = workloads.make_inputs(sh, seed=41, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    # With the filter prepacked, and gathered in the kernel (no workspace).
    for kind in ("filter", None):
        note(f"conv fp16 row-staged NWV={nwv} {sh.describe()} ws={kind}")
        assert_within(_run(sh, "f16", x, w, kind), ref, absd, TOL["f16"], sh.describe())
        assert_exact(_run(sh, "f16", xi, wi, kind), refi, sh.describe())


@pytest.mark.parametrize("bufs", [2, 3])
@pytest.mark.parametrize("t", ROWS, ids=str)
def test_conv_f16_row_staged_buffers(t, bufs, orc, knob):
    """Two stage buffers (loads one stage ahead; without a workspace the
    kernel picks them when a stage can then hold twice the channels) and
    three (two stages ahead), with the filter prepacked and gathered: exact
    on integer inputs."""
    knob("f16_reuse", -1)
    knob("f16_rows_bufs", bufs)
    sh = _shape(t, "f16")
    xi, wi = workloads.make_inputs(sh, seed=44, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    for kind in ("filter", None):
        note(f"conv fp16 row-staged buffers={bufs} {sh.describe()} ws={kind}")
        assert_exact(_run(sh, "f16", xi, wi, kind), refi, sh.describe())


@pytest.mark.parametrize("t", [(2, 4, 14, 16, 40, 3, 5, 2), (2, 4, 15, 24, 40, 3, 7, 2)], ids=str)
def test_conv_f16_row_staged_special_values(t, orc, knob):
    """Infinities and NaN in the input reach exactly the outputs whose windows
    hold them: the padded taps kw >= Wf never multiply a neighbour's Inf
    (Wf = 5 masks three dwords of each slice, Wf = 7 only the last)."""
    knob("f16_reuse", -1)
    sh = _shape(t, "f16")
    x, w = workloads.make_inputs(sh, seed=42)
    x[0, 1, 4, 5] = np.inf
    x[0, 2, 7, 13] = -np.inf
    x[1, 3, 0, 6] = np.nan
    x[1, 0, 13, 15] = np.inf
    x[0, 0, 2, 7] = np.inf
    x[-1, -1, -1, -1] = -np.inf     # x's last element
    w = np.abs(w) + np.asarray(0.25, dtype=w.dtype)
    ref = orc.conv_direct(x, w, sh.s)
    fin = np.isfinite(ref)
    _, absd = orc.conv_direct(np.where(np.isfinite(x), x, 0).astype(x.dtype), w, sh.s,
                              with_absdot=True)
    for kind in ("filter", None):
        note(f"conv fp16 row-staged special values {sh.describe()} ws={kind}")
        y = _run(sh, "f16", x, w, kind).astype(np.float64)
        assert np.array_equal(np.isnan(y), np.isnan(ref))
        assert np.array_equal(np.isposinf(y), np.isposinf(ref))
        assert np.array_equal(np.isneginf(y), np.isneginf(ref))
        assert_within(y[fin], ref[fin], absd[fin], TOL["f16"], "finite outputs")


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("t", [(11, 2, 65, 64, 40, 3, 3, 2), (40, 4, 21, 32, 70, 5, 5, 2)], ids=str)
def test_conv_f16_row_staged_tile_order(t, order, orc, knob):
    """XCD-grouped and launch-order tiling give the same (exact) results,
    with grids that are not a multiple of the 8 XCDs (partial last round)."""
    knob("tile_order", order)
    sh = _shape(t, "f16")
    xi, wi = workloads.make_inputs(sh, seed=43, mode="int")
    for reuse in (-1, 0):
        knob("f16_reuse", reuse)
        note(f"conv fp16 row-staged tile order={order} reuse={reuse} {sh.describe()}")
        assert_exact(_run(sh, "f16", xi, wi, "filter"), orc.conv_direct(xi, wi, sh.s), sh.describe())
    note(f"conv fp16 row-staged tile order={order} {sh.describe()}")
    assert_exact(_run(sh, "f16", xi, wi, "filter"), orc.conv_direct(xi, wi, sh.s), sh.describe())


# Shapes the row-reuse fp16 kernel takes (even column stride, Wf <= 8, Wi a
# multiple of 8, even Ci, a built (filter height, row stride) pair): every
# built pair; output heights not a multiple of the 4-row groups (partial last
# group); tiles crossing images (including several images per tile); one row
# group per image; Wf = 8 (no padded taps) and Wf = 1; column strides 2 and
# 4; channel counts that give stages of 4 and of 2 channels; Co off 64.
REUSE = [
    (2, 64, 40, 40, 64, 7, 7, 2),       # cv4-like
    (3, 6, 23, 24, 33, 3, 5, (1, 2)),
    (2, 16, 30, 32, 70, 7, 7, 2),
    (5, 4, 12, 16, 64, 3, 3, 2),
    (2, 8, 20, 64, 128, 5, 3, 2),
    (11, 2, 65, 64, 40, 3, 3, 2),
    (40, 4, 21, 32, 70, 5, 5, 2),       # several images per tile
    (7, 2, 7, 8, 5, 7, 3, (1, 2)),      # one output row per image
    (3, 2, 10, 8, 8, 3, 3, (1, 4)),
    (2, 6, 19, 24, 65, 5, 8, (1, 2)),   # Wf = 8
    (3, 10, 26, 16, 40, 7, 1, (1, 2)),  # Wf = 1, Hf 7 at row stride 1
    (1, 12, 33, 48, 130, 5, 5, 2),      # three channel tiles
]


@pytest.mark.parametrize("t", REUSE, ids=str)
def test_conv_f16_row_reuse(t, orc, knob):
    """The fp16 kernel that reuses each staged input row across the output
    rows sharing it, with the filter prepacked and gathered in the kernel
    (dword and, with w at an odd element offset, per-entry gathers): within
    tolerance on uniform inputs, exact on integer inputs, and the same bits
    as the row-staged kernel it replaces (knob f16_reuse=-1)."""
    import torch
    sh = _shape(t, "f16")
    assert m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, 2) == \
        "conv_f16_reuse_kernel"
    x, w = workloads.make_inputs(sh, seed=45)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    xi, wi = workloads.make_inputs(sh, seed=46, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    got = {}
    for kind in ("filter", None):
        note(f"conv fp16 row reuse {sh.describe()} ws={kind}")
        assert_within(_run(sh, "f16", x, w, kind), ref, absd, TOL["f16"], sh.describe())
        got[kind] = _run(sh, "f16", xi, wi, kind)
        assert_exact(got[kind], refi, f"{sh.describe()} ws={kind}")
    dev = device()
    big = torch.zeros(wi.size + 1, dtype=torch.float16, device=dev)
    big[1:] = torch.from_numpy(np.ascontiguousarray(wi).reshape(-1)).to(dev)
    note(f"conv fp16 row reuse {sh.describe()} filter at an odd offset")
    y = m.conv2d(to_dev(xi, dev), big[1:].view(wi.shape), sh.s).cpu().numpy()
    assert_exact(y, refi, f"{sh.describe()} odd filter offset")
    knob("f16_reuse", -1)
    for kind in ("filter", None):
        assert_exact(_run(sh, "f16", xi, wi, kind), got[kind], "row-staged kernel")


@pytest.mark.parametrize("t", [(2, 4, 14, 16, 40, 3, 5, 2), (2, 4, 19, 24, 40, 7, 7, 2),
                               (2, 2, 12, 16, 40, 5, 6, (1, 2))], ids=str)
def test_conv_f16_row_reuse_special_values(t, orc):
    """Infinities and NaN reach exactly the outputs whose windows hold them
    (padded taps are cleared in B, the rows of a partial row group past the
    image are zeros)."""
    sh = _shape(t, "f16")
    x, w = workloads.make_inputs(sh, seed=47)
    x[0, 1, 4, 5] = np.inf
    x[0, 2 % sh.Ci, 7, 13] = -np.inf
    x[1, 3 % sh.Ci, 0, 6] = np.nan
    x[1, 0, sh.Hi - 1, sh.Wi - 1] = np.inf
    x[0, 0, 2, 7] = np.inf
    x[-1, -1, -1, -1] = -np.inf     # x's last element
    w = np.abs(w) + np.asarray(0.25, dtype=w.dtype)
    ref = orc.conv_direct(x, w, sh.s)
    fin = np.isfinite(ref)
    _, absd = orc.conv_direct(np.where(np.isfinite(x), x, 0).astype(x.dtype), w, sh.s,
                              with_absdot=True)
    for kind in ("filter", None):
        note(f"conv fp16 row reuse special values {sh.describe()} ws={kind}")
        y = _run(sh, "f16", x, w, kind).astype(np.float64)
        assert np.array_equal(np.isnan(y), np.isnan(ref))
        assert np.array_equal(np.isposinf(y), np.isposinf(ref))
        assert np.array_equal(np.isneginf(y), np.isneginf(ref))
        assert_within(y[fin], ref[fin], absd[fin], TOL["f16"], "finite outputs")


# Shapes the fp16 kernel over the materialised tensor takes (sw*Hf even,
# packed rows a multiple of 8 elements): several slices per channel (Wf*Hf
# from 8 to 49, the last slice partly padding), stages of 4 and 2 channels,
# tiles crossing images, Co off 64 and above it, unequal strides.
WS = [
    (2, 16, 30, 32, 70, 7, 7, 2),
    (2, 64, 40, 40, 64, 7, 7, 2),
    (3, 6, 23, 24, 33, 3, 5, (1, 2)),
    (4, 8, 20, 16, 40, 2, 4, 2),
    (3, 4, 26, 32, 130, 4, 4, (3, 2)),
    (2, 12, 33, 48, 64, 5, 6, (2, 2)),
    (2, 8, 15, 24, 20, 1, 8, 2),
    (1, 10, 40, 64, 96, 3, 6, (2, 4)),
    (2, 16, 24, 40, 64, 7, 2, (1, 2)),
    # odd window steps sw*Hf (windows starting on odd elements)
    (2, 96, 24, 24, 256, 5, 5, 1),      # cv5 images: tiles across four images
    (2, 16, 14, 16, 70, 5, 5, 1),
    (3, 8, 12, 24, 40, 3, 3, 1),
    (2, 6, 20, 8, 33, 7, 3, 1),
    (3, 4, 15, 16, 64, 3, 3, (2, 3)),
]


@pytest.mark.parametrize("t", WS, ids=str)
def test_conv_f16_materialised_staged(t, orc, knob):
    """The fp16 kernel that copies each channel's window stretch of the
    materialised im2win tensor into LDS with direct loads, over the whole
    batch and one image at a time: within tolerance on uniform inputs, exact
    on integer inputs, and the same bits as the per-entry kernel it replaces
    (knob f16_ws=-1)."""
    sh = _shape(t, "f16")
    assert m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, 2,
                              "materialized") == "conv_f16_ws_kernel"
    x, w = workloads.make_inputs(sh, seed=48)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    xi, wi = workloads.make_inputs(sh, seed=49, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    got = {}
    for kind in ("full", "one"):
        note(f"conv fp16 materialised staged {sh.describe()} ws={kind}")
        assert_within(_run(sh, "f16", x, w, kind), ref, absd, TOL["f16"], sh.describe())
        got[kind] = _run(sh, "f16", xi, wi, kind)
        assert_exact(got[kind], refi, f"{sh.describe()} ws={kind}")
    knob("f16_ws", -1)
    assert_exact(_run(sh, "f16", xi, wi, "full"), got["full"], "per-entry kernel")


@pytest.mark.parametrize("t", [(2, 4, 19, 24, 40, 7, 7, 2), (2, 3, 14, 16, 40, 3, 4, (1, 2)),
                               (2, 4, 14, 16, 40, 5, 5, 1)], ids=str)
def test_conv_f16_materialised_staged_special_values(t, orc):
    """Infinities and NaN in the input reach exactly the outputs whose windows
    hold them: the padding of a channel's last slice (the next window's
    elements in the packed row) is masked."""
    sh = _shape(t, "f16")
    x, w = workloads.make_inputs(sh, seed=57)
    x[0, 1, 4, 5] = np.inf
    x[0, 2 % sh.Ci, 7, 13] = -np.inf
    x[1, 0, 0, 6] = np.nan
    x[1, 0, sh.Hi - 1, sh.Wi - 1] = np.inf
    x[0, 0, 2, 7] = np.inf
    x[-1, -1, -1, -1] = -np.inf     # x's last element
    w = np.abs(w) + np.asarray(0.25, dtype=w.dtype)
    ref = orc.conv_direct(x, w, sh.s)
    fin = np.isfinite(ref)
    _, absd = orc.conv_direct(np.where(np.isfinite(x), x, 0).astype(x.dtype), w, sh.s,
                              with_absdot=True)
    note(f"conv fp16 materialised staged special values {sh.describe()}")
    y = _run(sh, "f16", x, w, "full").astype(np.float64)
    assert np.array_equal(np.isnan(y), np.isnan(ref))
    assert np.array_equal(np.isposinf(y), np.isposinf(ref))
    assert np.array_equal(np.isneginf(y), np.isneginf(ref))
    assert_within(y[fin], ref[fin], absd[fin], TOL["f16"], "finite outputs")


# Shapes the wide-tile fp16 kernel takes with a prepacked filter (Co >= 128,
# or any Co with knob f16_wide=1; not taken by the row-staged kernel):
# tiles crossing images, Ci and Co off the multiples of 8 and 128, odd Wi
# (single-column staging), column strides 2 and 3, unequal strides, tiles
# aligned to images, a 1x1 filter, odd and even tap counts.
WIDE = [
    (2, 96, 24, 24, 256, 5, 5, 1),      # cv5 images
    (3, 13, 19, 21, 130, 3, 3, 1),
    (2, 16, 30, 28, 136, 3, 5, 2),
    (1, 8, 40, 40, 128, 4, 4, 3),
    (2, 24, 36, 36, 160, 2, 6, (1, 3)),
    (2, 8, 32, 36, 128, 3, 3, 1),       # tiles aligned to images
    (2, 8, 12, 40, 200, 1, 1, 1),
    (2, 24, 14, 14, 96, 5, 5, 1),       # Co < 128 (forced)
    (1, 16, 20, 20, 384, 3, 3, 1),      # one image, three channel tiles
    (3, 9, 5, 64, 128, 5, 3, 1),        # one output row per image
]


def _wide_plan(sh):
    """The wide kernel's envelope, worked out independently of the library:
    (applies, LDS bytes, staging units)."""
    sh_, sw = sh.s if isinstance(sh.s, tuple) else (sh.s, sh.s)
    Ho, Wo = (sh.Hi - sh.Hf) // sh_ + 1, (sh.Wi - sh.Wf) // sw + 1
    P = 512
    plane = Ho * Wo
    rows_max = min((P - 1) // Wo + 2, sh.N * Ho)
    tpi = -(-plane // P)
    aligned = tpi * P <= 1.05 * plane
    kmax = 0 if aligned or rows_max <= 1 else min(sh.N - 1, -(-(rows_max - 1) // Ho))
    rin = (rows_max - 1) * sh_ + sh.Hf + kmax * max(0, sh.Hf - sh_)
    rs = sw * -(-sh.Wi // sw)
    units = rin * (sh.Wi // 2) if sh.Wi % 2 == 0 else rin * sh.Wi
    cap = 4 * 256 if sh.Wi % 2 == 0 else 6 * 256
    hwp = (sh.Hf * sh.Wf + 1) & ~1
    kt = (hwp + 8 + 3) & ~3
    lds = 2 * (hwp * 128 * 16 + rin * rs * 16) + (kt * 4 + 15) // 16 * 16 + 8192
    return units <= cap and lds <= 160 * 1024, lds, units


@pytest.mark.parametrize("nw", [8, 4])
@pytest.mark.parametrize("t", WIDE, ids=str)
def test_conv_f16_wide_tiles(t, nw, orc, knob):
    """The fp16 kernel with 128-channel wave tiles (8 waves of 4 x 2 blocks or
    4 waves of 4 x 4), the filter copied to LDS by direct loads from the
    prepacked copy or gathered from w (no workspace): uniform and integer
    inputs; switching it off (knob f16_wide=-1) gives the
    channel-interleaved kernel's results."""
    knob("f16_wide_nw", nw)
    sh = _shape(t, "f16")
    ok, lds, units = _wide_plan(sh)
    assert ok, (lds, units)
    if sh.Co < 128:
        knob("f16_wide", 1)
    x, w = workloads.make_inputs(sh, seed=50)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    xi, wi = workloads.make_inputs(sh, seed=51, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    yi = {}
    for kind in ("filter", None):
        note(f"conv fp16 wide tiles NW={nw} {sh.describe()} ws={kind} (LDS {lds} B)")
        assert_within(_run(sh, "f16", x, w, kind), ref, absd, TOL["f16"], sh.describe())
        yi[kind] = _run(sh, "f16", xi, wi, kind)
        assert_exact(yi[kind], refi, sh.describe())
    knob("f16_wide", -1)
    for kind in ("filter", None):
        assert_exact(_run(sh, "f16", xi, wi, kind), yi[kind], "channel-interleaved kernel")


@pytest.mark.parametrize("t", [(2, 13, 19, 21, 130, 3, 3, 1), (2, 16, 14, 14, 128, 5, 5, 1)],
                         ids=str)
def test_conv_f16_wide_special_values(t, orc):
    """Infinities and NaN reach exactly the outputs whose windows hold them;
    the zero partner of the last tap (odd tap count) never multiplies one."""
    sh = _shape(t, "f16")
    assert _wide_plan(sh)[0]
    x, w = workloads.make_inputs(sh, seed=52)
    x[0, 1, 4, 5] = np.inf
    x[0, 2, 7, 13] = -np.inf
    x[1, 3, 0, 6] = np.nan
    x[1, 0, 13, 13] = np.inf
    x[0, 0, 2, 7] = np.inf
    x[-1, -1, -1, -1] = -np.inf     # x's last element
    w = np.abs(w) + np.asarray(0.25, dtype=w.dtype)
    ref = orc.conv_direct(x, w, sh.s)
    fin = np.isfinite(ref)
    _, absd = orc.conv_direct(np.where(np.isfinite(x), x, 0).astype(x.dtype), w, sh.s,
                              with_absdot=True)
    for kind in ("filter", None):
        note(f"conv fp16 wide special values {sh.describe()} ws={kind}")
        y = _run(sh, "f16", x, w, kind).astype(np.float64)
        assert np.array_equal(np.isnan(y), np.isnan(ref))
        assert np.array_equal(np.isposinf(y), np.isposinf(ref))
        assert np.array_equal(np.isneginf(y), np.isneginf(ref))
        assert_within(y[fin], ref[fin], absd[fin], TOL["f16"], "finite outputs")


@pytest.mark.parametrize("t", [(1, 10, 40, 40, 24, 17, 17, 1), (2, 12, 21, 40, 136, 16, 16, 1),
                               (1, 20, 30, 32, 70, 16, 8, 2)], ids=str)
def test_conv_f16_filter_pack_tap_counts(t, orc):
    """The filter packs on both sides of their LDS limit (256 taps): 17 x 17
    (289 taps, packed one entry per thread), 16 x 16 (256 taps, through LDS)
    and a 16 x 8 filter for the row-staged layout, bit-exact on integer
    inputs."""
    sh = _shape(t, "f16")
    xi, wi = workloads.make_inputs(sh, seed=53, mode="int")
    note(f"conv fp16 filter pack taps={sh.Hf * sh.Wf} {sh.describe()}")
    assert_exact(_run(sh, "f16", xi, wi, "filter"), orc.conv_direct(xi, wi, sh.s), sh.describe())


# Shapes the thin-layer fp16 kernel takes with a prepacked filter (Ci < 8,
# Ci*Hf <= 64, Wf <= 8, even column stride; not taken by the row-staged
# kernel): odd and even slice counts, odd widths (shifted dword-aligned row loads) and
# widths that are multiples of 8 (16-byte row loads), several channel tiles,
# row strides below and above the filter height, a 1x1 filter, cv3 images.
THIN = [
    (2, 3, 47, 45, 37, 7, 7, 2),      # odd filter length: per-entry gather without a workspace
    (3, 3, 35, 64, 64, 7, 7, 2),
    (2, 1, 30, 31, 70, 5, 3, (1, 2)),
    (2, 5, 20, 40, 130, 3, 8, 2),
    (1, 7, 19, 25, 16, 1, 1, 2),
    (4, 2, 15, 17, 64, 6, 4, (3, 2)),
    (3, 3, 227, 227, 64, 7, 7, 2),    # cv3 images
    (1, 3, 7, 40, 64, 7, 7, 2),       # one output row
    (5, 4, 9, 9, 200, 9, 8, 2),       # filter covers the input height: one output per image
]


def _thin_plan(sh, P=512):
    """The thin-layer kernel's envelope for tiles of P pixels, worked out
    independently of the library: (applies, LDS bytes)."""
    sh_, sw = sh.s if isinstance(sh.s, tuple) else (sh.s, sh.s)
    if sh.Ci >= 8 or sh.Wf > 8 or sw % 2 or sh.Hf * sh.Wf > 256 or sh.Ci * sh.Hf > 64:
        return False, 0
    S = sh.Ci * sh.Hf
    Sp = (S + 1) & ~1
    Ho, Wo = (sh.Hi - sh.Hf) // sh_ + 1, (sh.Wi - sh.Wf) // sw + 1
    plane = Ho * Wo
    rows_max = min((P - 1) // Wo + 2, sh.N * Ho)
    tpi = -(-plane // P)
    aligned = tpi * P <= 1.05 * plane
    kmax = 0 if aligned or rows_max <= 1 else min(sh.N - 1, -(-(rows_max - 1) // Ho))
    rin = (rows_max - 1) * sh_ + sh.Hf + kmax * max(0, sh.Hf - sh_)
    rp = -(-max(sh.Wi, (Wo - 1) * sw + 8) // 8) * 8
    kt = (Sp + 8 + 3) & ~3
    # filter slices, rows, slice table; an even slice count reads 2 KB past the filter
    lds = max(Sp * 1024 + sh.Ci * rin * (rp // 8) * 16 + (kt * 4 + 15) // 16 * 16,
              (Sp + (2 if S % 2 == 0 else 0)) * 1024)
    return lds <= 160 * 1024, lds


@pytest.mark.parametrize("nb", [4, 2])
@pytest.mark.parametrize("t", THIN, ids=str)
def test_conv_f16_thin_layers(t, nb, orc, knob):
    """The fp16 kernel that keeps a thin layer's whole filter in LDS as
    (channel, filter row) slices, with 4 and 2 pixel blocks per wave, the
    filter prepacked or gathered in the kernel (no workspace): uniform and
    integer inputs, and the same exact results as the kernels it replaces
    (knob f16_thin=-1)."""
    knob("f16_thin_nb", nb)
    sh = _shape(t, "f16")
    ok, lds = _thin_plan(sh, 32 * 4 * int(nb))
    assert ok, lds
    on = _filter_bytes(sh)
    assert on == -(-max(_layout_bytes(sh)) // 256) * 256, on
    x, w = workloads.make_inputs(sh, seed=60)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    xi, wi = workloads.make_inputs(sh, seed=61, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    yi = {}
    for kind in ("filter", None):
        note(f"conv fp16 thin {sh.describe()} ws={kind} (LDS {lds} B)")
        assert_within(_run(sh, "f16", x, w, kind), ref, absd, TOL["f16"], sh.describe())
        yi[kind] = _run(sh, "f16", xi, wi, kind)
        assert_exact(yi[kind], refi, sh.describe())
    knob("f16_thin", -1)
    assert _filter_bytes(sh) == on
    for kind in ("filter", None):
        assert_exact(_run(sh, "f16", xi, wi, kind), yi[kind], "kernels without the thin path")


@pytest.mark.parametrize("t", [(2, 3, 15, 17, 40, 7, 7, 2), (2, 2, 14, 17, 40, 3, 5, 2)], ids=str)
def test_conv_f16_thin_special_values(t, orc):
    """Infinities and NaN reach exactly the outputs whose windows hold them:
    padded taps (kw >= Wf) and the zero partner of an odd slice count never
    multiply one."""
    sh = _shape(t, "f16")
    assert _thin_plan(sh)[0]
    x, w = workloads.make_inputs(sh, seed=62)
    x[0, 1, 4, 5] = np.inf
    x[0, 0, 7, 13] = -np.inf
    x[1, 1, 0, 6] = np.nan
    x[1, 0, 13, 15] = np.inf
    x[0, 0, 2, 7] = np.inf
    x[-1, -1, -1, -1] = -np.inf     # x's last element (its row chunk is loaded half by half)
    w = np.abs(w) + np.asarray(0.25, dtype=w.dtype)
    ref = orc.conv_direct(x, w, sh.s)
    fin = np.isfinite(ref)
    _, absd = orc.conv_direct(np.where(np.isfinite(x), x, 0).astype(x.dtype), w, sh.s,
                              with_absdot=True)
    for kind in ("filter", None):
        note(f"conv fp16 thin special values {sh.describe()} ws={kind}")
        y = _run(sh, "f16", x, w, kind).astype(np.float64)
        assert np.array_equal(np.isnan(y), np.isnan(ref))
        assert np.array_equal(np.isposinf(y), np.isposinf(ref))
        assert np.array_equal(np.isneginf(y), np.isneginf(ref))
        assert_within(y[fin], ref[fin], absd[fin], TOL["f16"], "finite outputs")


@pytest.mark.parametrize("t", [(2, 24, 14, 14, 96, 5, 5, 1), (2, 16, 14, 14, 128, 5, 5, 1),
                               (2, 3, 47, 45, 37, 7, 7, 2), (3, 3, 35, 64, 64, 7, 7, 2),
                               (1, 64, 40, 40, 64, 7, 7, 2), (2, 9, 13, 21, 40, 3, 3, 1)],
                         ids=str)
def test_conv_f16_input_at_odd_element_offset(t, orc):
    """An fp16 input that starts 2 bytes past a 4-byte boundary (a view at an
    odd element offset) gives the exact results with every kernel a call can
    reach: fused, prepacked (channel-interleaved, wide-tile, thin-layer,
    row-staged) and materialised."""
    import torch
    dev = device()
    sh = _shape(t, "f16")
    xi, wi = workloads.make_inputs(sh, seed=63, mode="int")
    ref = orc.conv_direct(xi, wi, sh.s)
    big = torch.zeros(xi.size + 1, dtype=torch.float16, device=dev)
    big[1:] = torch.from_numpy(np.ascontiguousarray(xi).reshape(-1)).to(dev)
    xv = big[1:].view(xi.shape)
    assert xv.data_ptr() % 4 == 2
    wt = to_dev(wi, dev)
    for kind in (None, "filter", "full"):
        note(f"conv fp16 input at odd offset {sh.describe()} ws={kind}")
        y = call(sh, xv, wt, kind, dev).cpu().numpy()
        assert_exact(y, ref, f"{sh.describe()} ws={kind}")
    torch.cuda.synchronize()


@pytest.mark.parametrize("t", [(2, 24, 14, 14, 96, 5, 5, 1), (2, 16, 14, 14, 128, 5, 5, 1),
                               (3, 3, 35, 64, 64, 7, 7, 2), (1, 64, 40, 40, 64, 7, 7, 2),
                               (2, 4, 24, 32, 64, 16, 8, 2), (2, 9, 13, 21, 40, 3, 3, 1)],
                         ids=str)
def test_conv_f16_filter_at_odd_element_offset(t, orc):
    """An fp16 filter that starts 2 bytes past a 4-byte boundary gives the
    exact results when the kernels gather it themselves (no workspace; the
    row-staged kernel's dword-wide gather needs a 4-byte-aligned filter and
    takes its per-entry gather here) and when it is prepacked."""
    import torch
    dev = device()
    sh = _shape(t, "f16")
    xi, wi = workloads.make_inputs(sh, seed=64, mode="int")
    ref = orc.conv_direct(xi, wi, sh.s)
    big = torch.zeros(wi.size + 1, dtype=torch.float16, device=dev)
    big[1:] = torch.from_numpy(np.ascontiguousarray(wi).reshape(-1)).to(dev)
    wv = big[1:].view(wi.shape)
    assert wv.data_ptr() % 4 == 2
    xt = to_dev(xi, dev)
    for kind in (None, "filter"):
        note(f"conv fp16 filter at odd offset {sh.describe()} ws={kind}")
        y = call(sh, xt, wv, kind, dev).cpu().numpy()
        assert_exact(y, ref, f"{sh.describe()} ws={kind}")
    torch.cuda.synchronize()


def _random_f16_shapes(count_per_family=12, seed=2024):
    """Seeded random small shapes aimed at each fp16 kernel family: row-staged
    (even Ci, Wi % 8 = 0, even column stride, Wf <= 8), thin-layer (Ci < 8,
    even column stride, Wf <= 8), wide-tile (Co >= 128) and the
    channel-interleaved kernel (the rest). Strides may differ per axis."""
    rng = np.random.default_rng(seed)
    out = []

    def pick(family):
        for _ in range(1000):
            N = int(rng.integers(1, 4))
            Hf, Wf = int(rng.integers(1, 8)), int(rng.integers(1, 9))
            sh, sw = int(rng.integers(1, 4)), int(rng.integers(1, 4))
            Hi = int(rng.integers(Hf, Hf + 24))
            Wi = int(rng.integers(Wf, Wf + 40))
            if family == "rows":
                Ci, Co, sw = 2 * int(rng.integers(1, 9)), int(rng.integers(1, 130)), 2 * int(rng.integers(1, 3))
                Wi = max(8, (Wi + 7) // 8 * 8)
            elif family == "thin":
                Ci, Co, sw = int(rng.integers(1, 8)), int(rng.integers(1, 200)), 2 * int(rng.integers(1, 3))
                if Ci % 2 == 0 and Wi % 8 == 0:
                    Wi += 1
            elif family == "wide":
                Ci, Co = int(rng.integers(8, 40)), int(rng.integers(128, 300))
                Hf, Wf = min(Hf, 5), min(Wf, 5)
            else:
                Ci, Co = int(rng.integers(8, 40)), int(rng.integers(1, 128))
            if Wi < Wf or Hi < Hf:
                continue
            s = sh if sh == sw else (sh, sw)
            return (N, Ci, Hi, Wi, Co, Hf, Wf, s)
        raise RuntimeError(family)

    for family in ("rows", "thin", "wide", "interleaved"):
        for _ in range(count_per_family):
            out.append((family, pick(family)))
    return out


@pytest.mark.parametrize("family,t", _random_f16_shapes(), ids=lambda v: str(v))
def test_conv_f16_random_shapes(family, t, orc):
    """Seeded random shapes for every fp16 kernel family, bit-exact on
    integer inputs with the filter prepacked and gathered in the kernel (no
    workspace), and within tolerance on uniform inputs."""
    sh = _shape(t, "f16")
    xi, wi = workloads.make_inputs(sh, seed=64, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    for kind in ("filter", None):
        note(f"conv fp16 random {family} {sh.describe()} ws={kind}")
        assert_exact(_run(sh, "f16", xi, wi, kind), refi, f"{family} {sh.describe()} ws={kind}")
    x, w = workloads.make_inputs(sh, seed=65)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    assert_within(_run(sh, "f16", x, w, "filter"), ref, absd, TOL["f16"], sh.describe())


def _random_f32_shapes(count=24, seed=2025):
    """Seeded random small fp32 shapes: thin and wide channel counts, filters
    up to 11 x 11, strides up to 4 per axis."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        N = int(rng.integers(1, 4))
        Ci, Co = int(rng.integers(1, 40)), int(rng.integers(1, 200))
        Hf, Wf = int(rng.integers(1, 12)), int(rng.integers(1, 12))
        sh, sw = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        Hi, Wi = int(rng.integers(Hf, Hf + 30)), int(rng.integers(Wf, Wf + 40))
        out.append((N, Ci, Hi, Wi, Co, Hf, Wf, sh if sh == sw else (sh, sw)))
    return out


@pytest.mark.parametrize("t", _random_f32_shapes(), ids=str)
def test_conv_f32_random_shapes(t, orc, knob):
    """Seeded random fp32 shapes, bit-exact on integer inputs through the
    matrix-core kernel, the vector-ALU kernel and the materialised mode."""
    sh = _shape(t, "f32")
    xi, wi = workloads.make_inputs(sh, seed=66, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    for kind in (None, "full"):
        note(f"conv fp32 random {sh.describe()} ws={kind}")
        assert_exact(_run(sh, "f32", xi, wi, kind), refi, f"{sh.describe()} ws={kind}")
    knob("f32_valu", 1)
    note(f"conv fp32 random {sh.describe()} vector ALU")
    assert_exact(_run(sh, "f32", xi, wi, None), refi, f"{sh.describe()} vector ALU")


# One case per kernel that has the ablation switches (tile_order=1: tiles in
# launch order instead of XCD-grouped; sync_staging=1: each stage copied
# through registers and waited for before its MFMAs), with the knobs that
# route the shape to it: (shape, dtype, workspace kind, knobs, kernel).
SWITCH_CASES = [
    ((2, 64, 40, 40, 64, 7, 7, 2), "f16", "filter", {}, "conv_f16_reuse_kernel"),
    ((40, 4, 21, 32, 70, 5, 5, 2), "f16", None, {}, "conv_f16_reuse_kernel"),
    ((2, 64, 40, 40, 64, 7, 7, 2), "f16", "filter", {"f16_reuse": -1}, "conv_f16_rows_kernel"),
    ((40, 4, 21, 32, 70, 5, 5, 2), "f16", None, {"f16_reuse": -1, "f16_rows_bufs": 2},
     "conv_f16_rows_kernel"),
    ((3, 3, 35, 64, 64, 7, 7, 2), "f16", "filter", {}, "conv_f16_thin_kernel"),
    ((2, 3, 47, 45, 37, 7, 7, 2), "f16", None, {}, "conv_f16_thin_kernel"),
    ((2, 96, 24, 24, 256, 5, 5, 1), "f16", "filter", {}, "conv_f16_res_kernel"),
    ((2, 96, 24, 24, 256, 5, 5, 1), "f16", "filter", {"f16_res": -1}, "conv_f16_wide_kernel"),
    ((3, 13, 19, 21, 130, 3, 3, 1), "f16", None, {}, "conv_f16_wide_kernel"),
    ((1, 64, 30, 30, 64, 7, 7, 2), "f16", "filter", {}, "conv_f16_fused_kernel"),
    ((2, 24, 14, 14, 96, 5, 5, 1), "f16", None, {"f16_nwh": 3}, "conv_f16_fused_kernel"),
    ((2, 16, 30, 32, 70, 7, 7, 2), "f16", "full", {}, "conv_f16_ws_kernel"),
    ((3, 6, 23, 24, 33, 3, 5, (1, 2)), "f16", "one", {}, "conv_f16_ws_kernel"),
    ((2, 3, 99, 99, 96, 11, 11, 4), "f32", None, {"f32_small": -1}, "conv_f32_mfma_kernel"),
    ((1, 96, 12, 12, 256, 5, 5, 1), "f32", None, {"f32_ksplit": 4}, "conv_f32_mfma_kernel"),
    ((1, 96, 24, 24, 256, 5, 5, 1), "f32", None, {}, "conv_f32_small_kernel"),
    # 271 items on a grid of at most 256 workgroups: items in turn
    ((24, 4, 40, 40, 32, 3, 3, 1), "f32", None, {"f32_nw": 4, "f32_occ": 1},
     "conv_f32_mfma_kernel"),
]
_MODE_OF_KIND = {None: "fused", "filter": "prepacked", "full": "materialized",
                 "one": "materialized"}


@pytest.mark.parametrize("case", SWITCH_CASES, ids=lambda c: f"{c[4]}-{c[0]}-{c[2]}")
def test_ablation_switches_keep_results(case, orc, knob):
    """The two ablation switches change how a kernel stages its operands and
    orders its tiles, never what it sums or in which order: every switch
    setting runs the same kernel, exact on integer inputs, and gives the same
    bits as the default on uniform inputs."""
    import torch
    t, dt, kind, kn, kernel = case
    sh = _shape(t, dt)
    for k, v in kn.items():
        knob(k, v)
    name = m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s,
                              sh.elem_bytes, _MODE_OF_KIND[kind])
    assert name == kernel
    dev = device()
    x, w = workloads.make_inputs(sh, seed=61)
    xi, wi = workloads.make_inputs(sh, seed=62, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    xt, wt, xit, wit = to_dev(x, dev), to_dev(w, dev), to_dev(xi, dev), to_dev(wi, dev)
    note(f"ablation switches {kernel} {sh.describe()} ws={kind}: default")
    base = call(sh, xt, wt, kind, dev).cpu()
    for order, sync in ((1, 0), (0, 1), (1, 1)):
        knob("tile_order", order)
        knob("sync_staging", sync)
        note(f"ablation switches {kernel} {sh.describe()} ws={kind} tile_order={order} "
             f"sync_staging={sync}")
        assert m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s,
                                  sh.elem_bytes, _MODE_OF_KIND[kind]) == kernel
        assert_exact(call(sh, xit, wit, kind, dev).cpu().numpy(), refi,
                     f"{sh.describe()} order={order} sync={sync}")
        got = call(sh, xt, wt, kind, dev).cpu()
        assert torch.equal(got, base), f"{sh.describe()} order={order} sync={sync}"
    torch.cuda.synchronize()


# Shapes too small to fill the chip with 32 x 32 fp32 tiles, which the
# one-stage small-problem kernel takes: the 5x5 layer at N=1; K a multiple of
# 4 and not (16-byte and 4-byte filter loads); Wi a multiple of 4 and not;
# unequal strides; Co off 16; planes off 32 pixels; several images; K at the
# 8 x 24-chunk limit.
SMALL_F32 = [
    (1, 96, 24, 24, 256, 5, 5, 1),
    (1, 16, 20, 20, 40, 3, 3, 1),
    (2, 7, 19, 23, 33, 3, 5, (2, 1)),
    (1, 3, 30, 30, 20, 7, 7, 2),
    (3, 5, 9, 10, 17, 4, 2, (1, 3)),
    (1, 128, 12, 12, 64, 3, 3, 1),
    (1, 120, 10, 10, 32, 5, 5, 1),
]


@pytest.mark.parametrize("t", SMALL_F32, ids=str)
def test_conv_f32_small_problem_kernel(t, orc, knob):
    """The small-problem fp32 kernel: exact on integer inputs, within
    tolerance on uniform inputs, the same bits on repeated calls, and the
    same (exact) integer results as the K split it replaces (knob
    f32_small=-1)."""
    import torch
    sh = _shape(t, "f32")
    dev = device()
    assert m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, 4) == \
        "conv_f32_small_kernel"
    x, w = workloads.make_inputs(sh, seed=81)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    xi, wi = workloads.make_inputs(sh, seed=82, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    note(f"conv fp32 small problem {sh.describe()}")
    xt, wt = to_dev(x, dev), to_dev(w, dev)
    a = m.conv2d(xt, wt, sh.s)
    assert_within(a.cpu().numpy(), ref, absd, TOL["f32"], sh.describe())
    for _ in range(3):
        assert torch.equal(m.conv2d(xt, wt, sh.s), a)
    yi = _run(sh, "f32", xi, wi)
    assert_exact(yi, refi, sh.describe())
    knob("f32_small", -1)
    assert m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, 4) == \
        "conv_f32_mfma_kernel"
    assert_exact(_run(sh, "f32", xi, wi), refi, f"{sh.describe()} K split")


@pytest.mark.parametrize("t", [(1, 12, 14, 15, 40, 3, 5, 1), (1, 16, 12, 12, 64, 5, 5, 1)],
                         ids=str)
def test_conv_f32_small_problem_special_values(t, orc):
    """Infinities and NaN in the input reach exactly the outputs whose windows
    hold them (taps past K read a zero entry with a zero filter value)."""
    sh = _shape(t, "f32")
    device()
    assert m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, 4) == \
        "conv_f32_small_kernel"
    x, w = workloads.make_inputs(sh, seed=83)
    x[0, 1, 4, 5] = np.inf
    x[0, 2, 7, 10] = -np.inf
    x[0, 0, 0, 6] = np.nan
    x[0, sh.Ci - 1, sh.Hi - 1, sh.Wi - 1] = np.inf
    w = np.abs(w) + np.float32(0.25)
    ref = orc.conv_direct(x, w, sh.s)
    fin = np.isfinite(ref)
    _, absd = orc.conv_direct(np.where(np.isfinite(x), x, 0).astype(x.dtype), w, sh.s,
                              with_absdot=True)
    note(f"conv fp32 small problem special values {sh.describe()}")
    y = _run(sh, "f32", x, w).astype(np.float64)
    assert np.array_equal(np.isnan(y), np.isnan(ref))
    assert np.array_equal(np.isposinf(y), np.isposinf(ref))
    assert np.array_equal(np.isneginf(y), np.isneginf(ref))
    assert_within(y[fin], ref[fin], absd[fin], TOL["f32"], "finite outputs")


@pytest.mark.parametrize("kind", ["fp32_vector", "fp32_mfma", "fp16_mfma"])
def test_peak_probe_runs(kind):
    """The rate probe runs and reports finite values and a positive flop
    count (its rate is a measurement, checked against nothing)."""
    import torch
    device()
    out, flops = m.peak_probe(kind, 8, 16)
    torch.cuda.synchronize()
    assert flops > 0
    assert torch.isfinite(out).all()


# Shapes of the resident-input fp16 kernel (prepacked filter; 256 output
# channels per tile, whole output rows of one image): the cv5 layer, a
# channel count that pads its last octet, two channel tiles, row stride 2,
# column stride 2, a last quad with a zero octet, a filter taller than wide,
# row tiles that do not divide the output, and one-row tiles of 13 and 10
# pixel blocks (wide outputs).
RES_F16 = [
    (3, 96, 24, 24, 256, 5, 5, 1),
    (1, 32, 6, 200, 256, 5, 5, 1),
    (1, 32, 5, 160, 256, 3, 9, 1),
    (2, 60, 17, 16, 512, 3, 5, 1),
    (2, 32, 21, 24, 256, 3, 5, (2, 1)),
    (2, 31, 20, 24, 256, 3, 2, (1, 2)),
    (1, 88, 13, 8, 256, 4, 5, 1),
    (2, 32, 12, 16, 256, 7, 5, 1),
]


@pytest.mark.parametrize("t", RES_F16, ids=str)
def test_conv_f16_resident_kernel(t, orc, knob):
    """The resident-input fp16 kernel: exact on integer inputs, within
    tolerance on uniform inputs, the same bits on repeated calls, and the
    same (exact) integer results as the kernel it replaces (f16_res=-1)."""
    import torch
    sh = _shape(t, "f16")
    dev = device()
    name = lambda: m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, 2,
                                      "prepacked")
    assert name() == "conv_f16_res_kernel"
    x, w = workloads.make_inputs(sh, seed=91)
    ref, absd = orc.conv_direct(x, w, sh.s, with_absdot=True)
    xi, wi = workloads.make_inputs(sh, seed=92, mode="int")
    refi = orc.conv_direct(xi, wi, sh.s)
    note(f"conv fp16 resident-input {sh.describe()}")
    xt, wt = to_dev(x, dev), to_dev(w, dev)
    ws = workspace(sh, "filter", dev)
    y = torch.full(ref.shape, float("nan"), dtype=torch.float32, device=dev)
    a = call(sh, xt, wt, "filter", dev, ws=ws, out=y).clone()
    assert_within(a.cpu().numpy(), ref, absd, TOL["f16"], sh.describe())
    for _ in range(2):
        assert torch.equal(call(sh, xt, wt, "filter", dev, ws=ws), a)
    assert_exact(_run(sh, "f16", xi, wi, "filter"), refi, sh.describe())
    knob("f16_res", -1)
    assert name() != "conv_f16_res_kernel"
    assert_exact(_run(sh, "f16", xi, wi, "filter"), refi, f"{sh.describe()} f16_res=-1")


def test_conv_f16_resident_kernel_special_values(orc):
    """Infinities and NaN in the input reach exactly the outputs whose windows
    hold them: the zero octets and the zero filter fragments of the padded K
    steps add nothing."""
    sh = _shape((2, 88, 24, 24, 256, 5, 5, 1), "f16")
    device()
    assert m.conv_kernel_name(sh.N, sh.Ci, sh.Hi, sh.Wi, sh.Co, sh.Hf, sh.Wf, sh.s, 2,
                              "prepacked") == "conv_f16_res_kernel"
    x, w = workloads.make_inputs(sh, seed=93)
    x[0, 1, 4, 5] = np.inf
    x[1, 2, 7, 10] = -np.inf
    x[0, 0, 0, 6] = np.nan
    x[1, sh.Ci - 1, sh.Hi - 1, sh.Wi - 1] = np.inf
    w = (np.abs(w.astype(np.float32)) + np.float32(0.25)).astype(w.dtype)
    ref = orc.conv_direct(x, w, sh.s)
    fin = np.isfinite(ref)
    _, absd = orc.conv_direct(np.where(np.isfinite(x), x, 0).astype(x.dtype), w, sh.s,
                              with_absdot=True)
    note(f"conv fp16 resident-input special values {sh.describe()}")
    y = _run(sh, "f16", x, w, "filter").astype(np.float64)
    assert np.array_equal(np.isnan(y), np.isnan(ref))
    assert np.array_equal(np.isposinf(y), np.isposinf(ref))
    assert np.array_equal(np.isneginf(y), np.isneginf(ref))
    assert_within(y[fin], ref[fin], absd[fin], TOL["f16"], "finite outputs")
