"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch. tests/test_oracle.py runs them on the oracle as built;
tests/test_oracle_mutants.py runs them on copies of the oracle with a planted
mistake and expects at least one pin to fail for each.

None of these re-types the oracle's own loops: each compares against a
printed value (Table I, Fig. 1), a library routine (scipy correlate2d, torch
conv2d, numpy transpose), or a closed form that holds for a special input.

Run as a script, ``python tests/oracle_pins.py LIB.so`` runs every pin on that
library and exits 1 if any fails.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")

# Small shapes covering rectangles, s > Wf, ragged (Hi-Hf) % s, Ho = 1, Ci = 1,
# and unequal row and column strides.
# (N, Ci, Hi, Wi, Co, Hf, Wf, s) with s an int or (sh, sw)
SWEEP = [
    (1, 3, 3, 3, 2, 2, 2, 1),     # the Fig. 1 shapes
    (2, 2, 7, 9, 3, 3, 2, 1),
    (1, 5, 11, 8, 2, 2, 5, 2),
    (2, 1, 12, 12, 4, 5, 3, 3),
    (1, 3, 9, 10, 2, 1, 2, 4),    # s > Wf and s > Hf
    (1, 2, 5, 12, 3, 5, 1, 2),    # Ho = 1
    (2, 3, 10, 7, 1, 3, 3, 2),    # ragged (Hi-Hf) % s
    (1, 4, 6, 6, 5, 6, 6, 1),     # filter covers the whole input
    (1, 2, 13, 11, 2, 2, 3, 4),
    (1, 2, 11, 9, 3, 3, 2, (2, 1)),
    (2, 3, 10, 13, 2, 3, 3, (1, 3)),
    (1, 2, 12, 7, 2, 2, 5, (3, 2)),    # sh > Hf, Wo = 2
    (1, 1, 9, 14, 2, 4, 2, (4, 1)),
]


def _st(s):
    """(sh, sw) of a SWEEP stride entry."""
    return (s, s) if isinstance(s, int) else tuple(s)


def _rand(rng, shape, integer=False):
    if integer:
        return rng.integers(-4, 5, size=shape).astype(np.float32)
    return rng.uniform(-1, 1, size=shape).astype(np.float32)


def _case(cfg, seed, integer=False):
    N, Ci, Hi, Wi, Co, Hf, Wf, s = cfg
    rng = np.random.default_rng(seed)
    return _rand(rng, (N, Ci, Hi, Wi), integer), _rand(rng, (Co, Ci, Hf, Wf), integer)


# --------------------------------------------------------------------------
# Printed shapes
# --------------------------------------------------------------------------
def pin_table1_extents(O):
    """Output extents reproduce every Table I row (cv4 needs the floor)."""
    with open(os.path.join(GOLDEN, "table1_shapes.json")) as f:
        rows = json.load(f)["rows"]
    for r in rows:
        Ci, Hi, Wi = r["input"]
        Co, Hf, Wf = r["filter"]
        s = r["stride"]
        assert O.out_hw(Hi, Wi, Hf, Wf, s) == tuple(r["output"][1:]), r["name"]
        assert r["output"][0] == Co


def pin_fig1_sizes(O):
    """Fig. 1: 1x3x3x3 input, 2x3x2x2 filter, 1x2x2x2 output.

    Sizes the transforms must have there: the input has 27 elements; each of
    the 3 channels has 2 output rows of windows, each im2win row keeps all 3
    columns of its 2 input rows (6), so 36 elements; im2col has one column of
    3*2*2 = 12 per output pixel, 4 pixels, so 48.
    """
    with open(os.path.join(GOLDEN, "fig1_example.json")) as f:
        g = json.load(f)
    N, Ci, Hi, Wi = g["input"]
    Co, Ci2, Hf, Wf = g["filter"]
    s = g["stride"]
    assert Ci2 == Ci
    assert (N, Co) + O.out_hw(Hi, Wi, Hf, Wf, s) == tuple(g["output"])
    assert O.im2win_elems(N, Ci, Hi, Wi, Hf, Wf, s) == 36
    assert O.im2col_elems(N, Ci, Hi, Wi, Hf, Wf, s) == 48


# --------------------------------------------------------------------------
# Library special cases
# --------------------------------------------------------------------------
def pin_scipy_correlate(O):
    """Stride-1 'valid' cross-correlation per channel (scipy), summed over
    channels and subsampled by (sh, sw), equals the oracle (to fp64 rounding)."""
    from scipy.signal import correlate2d
    for k, cfg in enumerate(SWEEP):
        N, Ci, Hi, Wi, Co, Hf, Wf, s = cfg
        sh, sw = _st(s)
        x, w = _case(cfg, 100 + k)
        y = O.conv_direct(x, w, s)
        ref = np.zeros_like(y)
        for n in range(N):
            for co in range(Co):
                full = sum(correlate2d(x[n, ci].astype(np.float64), w[co, ci].astype(np.float64),
                                       mode="valid") for ci in range(Ci))
                ref[n, co] = full[::sh, ::sw][: y.shape[2], : y.shape[3]]
        assert y.shape == ref.shape, cfg
        scale = np.abs(ref).max() + 1e-30
        assert np.max(np.abs(y - ref)) <= 1e-12 * scale, cfg


def pin_torch_conv2d(O):
    """torch.nn.functional.conv2d in float64 on the CPU equals the oracle,
    including the absolute-product sums (conv2d of |x| and |w|)."""
    import torch
    import torch.nn.functional as F
    for k, cfg in enumerate(SWEEP):
        s = cfg[-1]
        st = _st(s)
        x, w = _case(cfg, 200 + k)
        y, a = O.conv_direct(x, w, s, with_absdot=True)
        xt = torch.from_numpy(x.astype(np.float64))
        wt = torch.from_numpy(w.astype(np.float64))
        ref = F.conv2d(xt, wt, stride=st).numpy()
        aref = F.conv2d(xt.abs(), wt.abs(), stride=st).numpy()
        assert y.shape == ref.shape, cfg
        assert np.max(np.abs(y - ref)) <= 1e-12 * (np.abs(ref).max() + 1e-30), cfg
        assert np.max(np.abs(a - aref)) <= 1e-12 * (aref.max() + 1e-30), cfg


def pin_integer_exact(O):
    """Small-integer inputs: every partial sum is an exact integer, so the
    oracle equals torch conv2d exactly, in fp64 and with a float accumulator."""
    import torch
    import torch.nn.functional as F
    for k, cfg in enumerate(SWEEP):
        s = cfg[-1]
        x, w = _case(cfg, 300 + k, integer=True)
        ref = F.conv2d(torch.from_numpy(x.astype(np.float64)),
                       torch.from_numpy(w.astype(np.float64)), stride=_st(s)).numpy()
        assert np.array_equal(O.conv_direct(x, w, s), ref), cfg
        assert np.array_equal(O.conv_direct_f32acc(x, w, s), ref.astype(np.float32)), cfg


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------
def pin_delta_filter(O):
    """A one-hot filter (channel c, tap (kh0, kw0)) turns the convolution into
    the strided crop x[n, c, kh0::sh, kw0::sw] -- exactly."""
    rng = np.random.default_rng(5)
    for cfg in SWEEP:
        N, Ci, Hi, Wi, Co, Hf, Wf, s = cfg
        sh, sw = _st(s)
        x = rng.uniform(-1, 1, size=(N, Ci, Hi, Wi)).astype(np.float32)
        w = np.zeros((Co, Ci, Hf, Wf), np.float32)
        picks = []
        for co in range(Co):
            c, kh0, kw0 = rng.integers(Ci), rng.integers(Hf), rng.integers(Wf)
            w[co, c, kh0, kw0] = 1.0
            picks.append((c, kh0, kw0))
        y = O.conv_direct(x, w, s)
        Ho, Wo = y.shape[2:]
        for co, (c, kh0, kw0) in enumerate(picks):
            crop = x[:, c, kh0::sh, kw0::sw][:, :Ho, :Wo].astype(np.float64)
            assert np.array_equal(y[:, co], crop), (cfg, co)


def pin_constant_input(O):
    """x == c everywhere gives y[n, co] == c * sum(w[co]) at every pixel."""
    for k, cfg in enumerate(SWEEP):
        N, Ci, Hi, Wi, Co, Hf, Wf, s = cfg
        _, w = _case(cfg, 400 + k, integer=True)
        x = np.full((N, Ci, Hi, Wi), 3.0, np.float32)
        y = O.conv_direct(x, w, s)
        expect = 3.0 * w.astype(np.float64).reshape(Co, -1).sum(1)
        assert np.array_equal(y, np.broadcast_to(expect[None, :, None, None], y.shape)), cfg


def pin_ramp_input(O):
    """x[n, ci, h, w] = a*h + b*w + c[ci] is affine in (h, w), so
    y[n, co, ho, wo] = (a*sh*ho + b*sw*wo)*S + a*Kh + b*Kw + Cc with
    S = sum w[co], Kh = sum kh*w[co,..,kh,kw], Kw = sum kw*w[co,..,kh,kw],
    Cc = sum_ci c[ci]*sum w[co,ci]. Integer values keep it exact; a != b
    separates the two axes."""
    a, b = 3.0, 7.0
    for k, cfg in enumerate(SWEEP):
        N, Ci, Hi, Wi, Co, Hf, Wf, s = cfg
        sh, sw = _st(s)
        _, w = _case(cfg, 500 + k, integer=True)
        c = np.arange(1, Ci + 1, dtype=np.float64) * 5.0
        hh = np.arange(Hi, dtype=np.float64)[:, None]
        ww = np.arange(Wi, dtype=np.float64)[None, :]
        x = (a * hh + b * ww)[None, None] + c[None, :, None, None]
        x = np.broadcast_to(x, (N, Ci, Hi, Wi)).astype(np.float32)
        y = O.conv_direct(x, w, s)
        Ho, Wo = y.shape[2:]
        wd = w.astype(np.float64)
        S = wd.sum(axis=(1, 2, 3))
        Kh = (wd * np.arange(Hf)[None, None, :, None]).sum(axis=(1, 2, 3))
        Kw = (wd * np.arange(Wf)[None, None, None, :]).sum(axis=(1, 2, 3))
        Cc = (wd.sum(axis=(2, 3)) * c[None, :]).sum(axis=1)
        ho = np.arange(Ho)[:, None]
        wo = np.arange(Wo)[None, :]
        expect = (a * sh * ho + b * sw * wo)[None] * S[:, None, None] + \
            (a * Kh + b * Kw + Cc)[:, None, None]
        assert np.array_equal(y, np.broadcast_to(expect[None], y.shape)), cfg


# --------------------------------------------------------------------------
# The im2win transform
# --------------------------------------------------------------------------
def pin_pack_rows_are_transposed_strips(O):
    """Each im2win row (n, ci, ho) is the Hf x Wi strip of input rows
    ho*sh .. ho*sh+Hf-1 read column by column (numpy transpose, flattened)."""
    for k, cfg in enumerate(SWEEP):
        N, Ci, Hi, Wi, Co, Hf, Wf, s = cfg
        sh, _ = _st(s)
        x, _ = _case(cfg, 600 + k)
        ws = O.im2win_pack(x, Hf, Wf, s)
        Ho = ws.shape[2]
        assert ws.shape == (N, Ci, Ho, Wi * Hf)
        for ho in range(Ho):
            strip = x[:, :, ho * sh: ho * sh + Hf, :]          # N, Ci, Hf, Wi
            assert np.array_equal(ws[:, :, ho, :], strip.transpose(0, 1, 3, 2).reshape(N, Ci, -1))


def pin_pack_windows_contiguous(O):
    """The defining property: the Hf x Wf window of output (ho, wo) is the
    one contiguous run of Wf*Hf elements at wo*sw*Hf in im2win row (n, ci, ho)."""
    for k, cfg in enumerate(SWEEP):
        N, Ci, Hi, Wi, Co, Hf, Wf, s = cfg
        sh, sw = _st(s)
        x, _ = _case(cfg, 700 + k)
        ws = O.im2win_pack(x, Hf, Wf, s)
        Ho, Wo = O.out_hw(Hi, Wi, Hf, Wf, s)
        for ho in range(Ho):
            for wo in range(Wo):
                run = ws[:, :, ho, wo * sw * Hf: wo * sw * Hf + Wf * Hf]
                win = x[:, :, ho * sh: ho * sh + Hf, wo * sw: wo * sw + Wf]
                assert np.array_equal(run.reshape(N, Ci, Wf, Hf).transpose(0, 1, 3, 2), win)


def pin_pack_is_bit_copy(O):
    """The transform moves bits: NaN payloads, infinities and subnormals of
    2- and 4-byte elements come through unchanged."""
    rng = np.random.default_rng(9)
    for dt in (np.uint16, np.uint32):
        for cfg in SWEEP[:4] + SWEEP[-2:]:
            N, Ci, Hi, Wi, Co, Hf, Wf, s = cfg
            sh, _ = _st(s)
            x = rng.integers(0, np.iinfo(dt).max, size=(N, Ci, Hi, Wi), dtype=dt, endpoint=True)
            ws = O.im2win_pack(x, Hf, Wf, s)
            ref = np.stack([x[:, :, ho * sh: ho * sh + Hf, :].transpose(0, 1, 3, 2).reshape(N, Ci, -1)
                            for ho in range(ws.shape[2])], axis=2)
            assert ws.dtype == dt and np.array_equal(ws, ref)
    x = np.array([np.nan, np.inf, -np.inf, 1e-45, -0.0, 3.0, 6e-8, 65504.0, 1.0],
                 np.float32).reshape(1, 1, 3, 3)
    for dt in (np.float32, np.float16):
        xx = x.astype(dt)
        ws = O.im2win_pack(xx, 2, 2, 1)
        ref = np.stack([xx[:, :, h: h + 2, :].transpose(0, 1, 3, 2).reshape(1, 1, -1)
                        for h in range(2)], axis=2)
        assert np.array_equal(ws.view(np.uint8), ref.view(np.uint8))


def pin_pack_nhwc_is_nchw_pack_permuted(O):
    """The NHWC transform of x.transpose(0, 2, 3, 1) is the NCHW transform of x
    with its axes permuted: ws_nhwc[n, ho, w, kh, c] = ws[n, c, ho, w*Hf + kh]."""
    for k, cfg in enumerate(SWEEP):
        N, Ci, Hi, Wi, Co, Hf, Wf, s = cfg
        x, _ = _case(cfg, 1100 + k)
        nchw = O.im2win_pack(x, Hf, Wf, s)
        Ho = nchw.shape[2]
        nhwc = O.im2win_pack_nhwc(np.ascontiguousarray(x.transpose(0, 2, 3, 1)), Hf, Wf, s)
        assert nhwc.shape == (N, Ho, Wi, Hf, Ci)
        assert np.array_equal(nhwc, nchw.reshape(N, Ci, Ho, Wi, Hf).transpose(0, 2, 3, 4, 1)), cfg


def pin_pack_nhwc_windows_contiguous(O):
    """NHWC: the window of output (ho, wo) is the contiguous run of Wf*Hf*Ci
    elements at wo*sw*Hf*Ci in row (n, ho), ordered (kw, kh, c)."""
    for k, cfg in enumerate(SWEEP):
        N, Ci, Hi, Wi, Co, Hf, Wf, s = cfg
        sh, sw = _st(s)
        x, _ = _case(cfg, 1200 + k)
        ws = O.im2win_pack_nhwc(np.ascontiguousarray(x.transpose(0, 2, 3, 1)), Hf, Wf, s)
        Ho, Wo = O.out_hw(Hi, Wi, Hf, Wf, s)
        L = Wf * Hf * Ci
        for n in range(N):
            for ho in range(Ho):
                row = ws[n, ho].reshape(-1)
                for wo in range(Wo):
                    run = row[wo * sw * Hf * Ci: wo * sw * Hf * Ci + L].reshape(Wf, Hf, Ci)
                    win = x[n, :, ho * sh: ho * sh + Hf, wo * sw: wo * sw + Wf]   # Ci, Hf, Wf
                    assert np.array_equal(run.transpose(2, 1, 0), win), (cfg, n, ho, wo)


def pin_im2col_rows_are_windows(O):
    """Each im2col row is one output pixel's receptive field x[n, :, ho*sh:+Hf,
    wo*sw:+Wf] flattened in (ci, kh, kw) order (numpy slicing), then zeros;
    and the im2col matrix times the flattened filters is the convolution."""
    for k, cfg in enumerate(SWEEP):
        N, Ci, Hi, Wi, Co, Hf, Wf, s = cfg
        sh, sw = _st(s)
        x, w = _case(cfg, 1000 + k, integer=True)
        K = Ci * Hf * Wf
        col = O.im2col_pack(x, Hf, Wf, s, KP=K + 3)
        Ho, Wo = O.out_hw(Hi, Wi, Hf, Wf, s)
        assert col.shape == (N * Ho * Wo, K + 3)
        assert not col[:, K:].any()
        q = 0
        for n in range(N):
            for ho in range(Ho):
                for wo in range(Wo):
                    win = x[n, :, ho * sh: ho * sh + Hf, wo * sw: wo * sw + Wf].reshape(-1)
                    assert np.array_equal(col[q, :K], win), (cfg, q)
                    q += 1
        y = (col[:, :K].astype(np.float64) @ w.reshape(Co, K).astype(np.float64).T)
        y = y.reshape(N, Ho, Wo, Co).transpose(0, 3, 1, 2)
        assert np.array_equal(y, O.conv_direct(x, w, s)), cfg


def pin_im2win_conv_equals_direct(O):
    """Convolving the packed tensor gives bit-identical results to the direct
    loops (same terms, same order), in fp64 and with a float accumulator."""
    for k, cfg in enumerate(SWEEP):
        N, Ci, Hi, Wi, Co, Hf, Wf, s = cfg
        x, w = _case(cfg, 800 + k)
        ws = O.im2win_pack(x, Hf, Wf, s)
        assert np.array_equal(O.conv_im2win(ws, w, Hi, Wi, s), O.conv_direct(x, w, s)), cfg
        assert np.array_equal(O.conv_im2win_f32acc(ws, w, Hi, Wi, s),
                              O.conv_direct_f32acc(x, w, s)), cfg


def pin_points_match_full(O):
    """Single outputs computed one by one equal the full run bit for bit."""
    for k, cfg in enumerate(SWEEP):
        x, w = _case(cfg, 900 + k)
        s = cfg[-1]
        y, a = O.conv_direct(x, w, s, with_absdot=True)
        idx = np.arange(y.size, dtype=np.int64)[::3]
        py, pa = O.conv_points(x, w, s, idx)
        assert np.array_equal(py, y.reshape(-1)[idx]) and np.array_equal(pa, a.reshape(-1)[idx])


def pin_workspace_sizes(O):
    """Element counts: im2win N*Ci*Ho*Wi*Hf, im2col N*Ci*Hf*Wf*Ho*Wo, so their
    ratio is Wi/(Wf*Wo) -- and the byte counts at the benchmark layers."""
    expect_bytes = {  # (N, Ci, Hi, Wi, Hf, Wf, s, elem): im2win bytes
        # sh=3, sw=2: Ho = (20-4)//3 + 1 = 6, 2*3*6*17*4 elements
        (2, 3, 20, 17, 4, 3, (3, 2), 4): 9_792,
        (1, 96, 24, 24, 5, 5, 1, 4): 921_600,
        (32, 3, 227, 227, 11, 11, 4, 4): 52_736_640,
        (128, 96, 24, 24, 5, 5, 1, 2): 58_982_400,
        (64, 3, 227, 227, 7, 7, 2, 2): 67_729_536,
        (64, 64, 224, 224, 7, 7, 2, 2): 1_400_111_104,
    }
    for (N, Ci, Hi, Wi, Hf, Wf, s, e), b in expect_bytes.items():
        win = O.im2win_elems(N, Ci, Hi, Wi, Hf, Wf, s)
        col = O.im2col_elems(N, Ci, Hi, Wi, Hf, Wf, s)
        Ho, Wo = O.out_hw(Hi, Wi, Hf, Wf, s)
        assert win * e == b
        assert win * Wf * Wo == col * Wi


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


def main(argv):
    sys.path.insert(0, os.path.dirname(HERE))
    import oracle
    O = oracle.Oracle(argv[1])
    failed = []
    for p in PINS:
        try:
            p(O)
        except AssertionError as e:
            failed.append(f"{p.__name__}: {e}")
    for f in failed:
        print("FAIL", f)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
