"""The C-ABI library on the host: it loads, exports every declared symbol,
and rejects bad arguments before touching the GPU (no GPU needed)."""
import ctypes
import os
import re

import pytest

import memory_efficient_im2win_amd as m
from memory_efficient_im2win_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "im2win.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(im2win_\w+|im2col_\w+|conv2d_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    single = ["im2win_workspace_bytes", "im2win_output_dims", "im2win_pack",
              "conv2d_im2win_fp32", "conv2d_im2win_fp16"]
    assert declared_functions() == sorted(
        single + [f + "_strided" for f in single] + ["im2win_status_string", "im2win_last_error"] +
        ["conv2d_im2win_fp16_fused_workspace_bytes", "conv2d_im2win_fp16_fused",
         "conv2d_im2win_fp16_fused_noalloc",
         "im2win_set_knob", "im2win_get_knob", "im2win_knob_name", "im2win_conv_kernel_name",
         "im2win_peak_probe", "im2win_peak_probe_flops"] +
        ["conv2d_im2col_workspace_bytes", "im2col_pack", "conv2d_im2col_fp32", "conv2d_im2col_fp16",
         "conv2d_direct_fp32", "conv2d_direct_fp16", "conv2d_im2win_nhwc_workspace_bytes",
         "im2win_pack_nhwc", "conv2d_im2win_nhwc_fp32", "conv2d_im2win_nhwc_fp16",
         "conv2d_im2win_nhwc_fp16_fused_workspace_bytes", "conv2d_im2win_nhwc_fp16_fused"])


def test_library_exports_every_declared_symbol():
    L = m.load_library()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(_lib.EXPORTS)


def test_workspace_bytes_at_the_benchmark_layers():
    # N*Ci*Ho*(Wi*Hf)*elem for cv5/cv1 (fp32) and cv5/cv3/cv4 (fp16)
    assert m.workspace_bytes(1, 96, 24, 24, 5, 5, 1, 4) == 921_600
    assert m.workspace_bytes(32, 3, 227, 227, 11, 11, 4, 4) == 52_736_640
    assert m.workspace_bytes(128, 96, 24, 24, 5, 5, 1, 2) == 58_982_400
    assert m.workspace_bytes(64, 3, 227, 227, 7, 7, 2, 2) == 67_729_536
    assert m.workspace_bytes(64, 64, 224, 224, 7, 7, 2, 2) == 1_400_111_104


def test_workspace_bytes_agrees_with_oracle(orc):
    import random
    rnd = random.Random(1)
    for _ in range(200):
        Hf, Wf, s = rnd.randint(1, 6), rnd.randint(1, 6), rnd.randint(1, 5)
        Hi, Wi = rnd.randint(Hf, 40), rnd.randint(Wf, 40)
        N, Ci = rnd.randint(1, 4), rnd.randint(1, 9)
        for e in (2, 4):
            assert m.workspace_bytes(N, Ci, Hi, Wi, Hf, Wf, s, e) == \
                orc.im2win_elems(N, Ci, Hi, Wi, Hf, Wf, s) * e
            assert m.output_dims(Hi, Wi, Hf, Wf, s) == orc.out_hw(Hi, Wi, Hf, Wf, s)


def test_strided_sizes_agree_with_oracle(orc):
    import random
    rnd = random.Random(2)
    for _ in range(200):
        Hf, Wf, sh, sw = rnd.randint(1, 6), rnd.randint(1, 6), rnd.randint(1, 5), rnd.randint(1, 5)
        Hi, Wi = rnd.randint(Hf, 40), rnd.randint(Wf, 40)
        N, Ci = rnd.randint(1, 4), rnd.randint(1, 9)
        st = (sh, sw)
        assert m.output_dims(Hi, Wi, Hf, Wf, st) == orc.out_hw(Hi, Wi, Hf, Wf, st)
        for e in (2, 4):
            assert m.workspace_bytes(N, Ci, Hi, Wi, Hf, Wf, st, e) == \
                orc.im2win_elems(N, Ci, Hi, Wi, Hf, Wf, st) * e


def test_single_stride_entry_points_equal_their_strided_twins():
    L = m.load_library()
    for (Hi, Wi, Hf, Wf, s) in [(224, 224, 7, 7, 2), (227, 227, 11, 11, 4), (24, 24, 5, 5, 1),
                                (13, 17, 3, 5, 3)]:
        a, b, c, d = (ctypes.c_int() for _ in range(4))
        assert L.im2win_output_dims(Hi, Wi, Hf, Wf, s, ctypes.byref(a), ctypes.byref(b)) == 0
        assert L.im2win_output_dims_strided(Hi, Wi, Hf, Wf, s, s, ctypes.byref(c),
                                            ctypes.byref(d)) == 0
        assert (a.value, b.value) == (c.value, d.value)
        for e in (2, 4):
            assert L.im2win_workspace_bytes(3, 5, Hi, Wi, Hf, Wf, s, e) == \
                L.im2win_workspace_bytes_strided(3, 5, Hi, Wi, Hf, Wf, s, s, e)


def test_unequal_strides_axes():
    # Ho follows the row stride, Wo the column stride; the im2win tensor
    # depends on the row stride only.
    assert m.output_dims(20, 17, 4, 3, (3, 2)) == (6, 8)
    assert m.output_dims(17, 20, 3, 4, (2, 3)) == (8, 6)
    assert m.workspace_bytes(2, 3, 20, 17, 4, 3, (3, 2), 4) == 2 * 3 * 6 * 17 * 4 * 4
    assert m.workspace_bytes(2, 3, 20, 17, 4, 3, (3, 5), 4) == 2 * 3 * 6 * 17 * 4 * 4
    with pytest.raises(ValueError):
        m.strides((1, 2, 3))


@pytest.mark.parametrize("args", [
    (0, 1, 4, 4, 2, 2, 1, 4),      # N = 0
    (1, 1, 4, 4, 5, 2, 1, 4),      # Hf > Hi
    (1, 1, 4, 4, 2, 5, 1, 4),      # Wf > Wi
    (1, 1, 4, 4, 2, 2, 0, 4),      # s = 0
    (1, 1, 4, 4, 2, 2, 1, 3),      # element size
    (1, 1 << 16, 1 << 8, 1 << 8, 1, 1, 1, 2),  # one image beyond 2^31 elements
])
def test_workspace_bytes_invalid(args):
    assert m.workspace_bytes(*args) == 0


@pytest.mark.parametrize("sh,sw", [(0, 1), (1, 0), (-1, 2)])
def test_strided_rejects_a_zero_or_negative_stride(sh, sw):
    L = m.load_library()
    assert L.im2win_workspace_bytes_strided(1, 1, 8, 8, 2, 2, sh, sw, 4) == 0
    assert L.conv2d_im2win_fp16_fused_workspace_bytes(1, 1, 8, 8, 1, 2, 2, sh, sw) == 0
    assert L.im2win_output_dims_strided(8, 8, 2, 2, sh, sw, None, None) == _lib.IM2WIN_EINVAL
    assert L.im2win_pack_strided(FAKE, FAKE, 1, 1, 8, 8, 2, 2, sh, sw, 4, None) == \
        _lib.IM2WIN_EINVAL
    for f in (L.conv2d_im2win_fp32_strided, L.conv2d_im2win_fp16_strided):
        assert f(FAKE, FAKE, FAKE, None, 0, 1, 3, 8, 8, 4, 3, 3, sh, sw, None) == \
            _lib.IM2WIN_EINVAL


def test_output_dims_table1_floor():
    assert m.output_dims(224, 224, 7, 7, 2) == (109, 109)
    with pytest.raises(m.Im2winError):
        m.output_dims(4, 4, 5, 5, 1)


def test_status_strings():
    L = m.load_library()
    for st in (0, -1, -2, -3, 7):
        assert L.im2win_status_string(st)
    assert L.im2win_last_error() == b"no error"


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails its checks first


@pytest.mark.parametrize("fn", ["conv2d_im2win_fp32", "conv2d_im2win_fp16"])
def test_conv_rejects_bad_arguments_before_launch(fn):
    L = m.load_library()
    f = getattr(L, fn)
    ok = (1, 3, 8, 8, 4, 3, 3, 1)
    # NULL tensors
    assert f(None, FAKE, FAKE, None, 0, *ok, None) == _lib.IM2WIN_EINVAL
    assert f(FAKE, None, FAKE, None, 0, *ok, None) == _lib.IM2WIN_EINVAL
    assert f(FAKE, FAKE, None, None, 0, *ok, None) == _lib.IM2WIN_EINVAL
    # bad shapes
    assert f(FAKE, FAKE, FAKE, None, 0, 1, 3, 8, 8, 4, 9, 3, 1, None) == _lib.IM2WIN_EINVAL
    assert f(FAKE, FAKE, FAKE, None, 0, 1, 3, 8, 8, 4, 3, 3, 0, None) == _lib.IM2WIN_EINVAL
    assert f(FAKE, FAKE, FAKE, None, 0, 1, 0, 8, 8, 4, 3, 3, 1, None) == _lib.IM2WIN_EINVAL
    # misaligned tensors
    odd = ctypes.c_void_p(0x10001)
    assert f(odd, FAKE, FAKE, None, 0, *ok, None) == _lib.IM2WIN_EINVAL
    # workspace: NULL with a size, or smaller than one image's im2win rows
    e = 4 if fn.endswith("32") else 2
    smallest = m.workspace_bytes(1, 3, 8, 8, 3, 3, 1, e)
    assert f(FAKE, FAKE, FAKE, None, 64, *ok, None) == _lib.IM2WIN_EWORKSPACE
    assert f(FAKE, FAKE, FAKE, FAKE, smallest - 1, *ok, None) == _lib.IM2WIN_EWORKSPACE
    assert f(FAKE, FAKE, FAKE, FAKE, 0, *ok, None) == _lib.IM2WIN_EWORKSPACE
    # workspace not 16-byte aligned
    assert f(FAKE, FAKE, FAKE, ctypes.c_void_p(0x10008), smallest, *ok, None) == _lib.IM2WIN_EINVAL


def test_fused_workspace_query():
    """The fp16 filter scratch holds either prepacked layout (slices of 8 taps
    for 64-channel tiles, or 16-byte entries of 8 input channels for
    128-channel tiles; worked out here independently), rounded up to 256
    bytes, and depends on the shape only (no knob changes it)."""
    for (N, Ci, Hi, Wi, Co, Hf, Wf, s) in [(64, 64, 224, 224, 64, 7, 7, 2),
                                           (128, 96, 24, 24, 256, 5, 5, 1),
                                           (64, 3, 227, 227, 64, 7, 7, 2),
                                           (1, 10, 40, 40, 24, 17, 17, 1)]:
        slices = Ci * Hf * (-(-Co // 64) * 64) * 16 if Wf <= 8 and Hf * Wf <= 256 else 0
        inter = -(-Ci // 8) * ((Hf * Wf + 1) & ~1) * (-(-Co // 128) * 128) * 16
        F = m.fused_workspace_bytes(N, Ci, Hi, Wi, Co, Hf, Wf, s)
        assert F == -(-max(slices, inter) // 256) * 256, (F, slices, inter)
        with m.knobs(f16_rows=-1, f16_thin=-1, f16_wide=-1):
            assert m.fused_workspace_bytes(N, Ci, Hi, Wi, Co, Hf, Wf, s) == F
    assert m.fused_workspace_bytes(1, 3, 4, 4, 2, 5, 5, 1) == 0   # invalid shape


def test_fused_rejects_bad_arguments_before_launch():
    L = m.load_library()
    f = L.conv2d_im2win_fp16_fused
    ok = (1, 3, 8, 8, 4, 3, 3, 1, 1)
    F = L.conv2d_im2win_fp16_fused_workspace_bytes(*ok)
    assert f(None, FAKE, FAKE, None, 0, *ok, None) == _lib.IM2WIN_EINVAL
    assert f(FAKE, FAKE, FAKE, None, 0, 1, 3, 8, 8, 4, 9, 3, 1, 1, None) == _lib.IM2WIN_EINVAL
    assert f(FAKE, FAKE, FAKE, None, 64, *ok, None) == _lib.IM2WIN_EWORKSPACE
    assert f(FAKE, FAKE, FAKE, FAKE, F - 1, *ok, None) == _lib.IM2WIN_EWORKSPACE
    assert f(FAKE, FAKE, FAKE, ctypes.c_void_p(0x10008), F, *ok, None) == _lib.IM2WIN_EINVAL


def test_knobs():
    names = m.knob_names()
    assert len(names) == len(set(names)) and "f32_valu" in names and "tile_order" in names
    L = m.load_library()
    assert L.im2win_knob_name(len(names)) is None and L.im2win_knob_name(-1) is None
    assert L.im2win_set_knob(len(names), 1) == _lib.IM2WIN_EINVAL
    assert all(m.get_knob(n) == 0 for n in names)
    with m.knobs(f32_nw=8, tile_order=1):
        assert m.get_knob("f32_nw") == 8 and m.get_knob("tile_order") == 1
    assert m.get_knob("f32_nw") == 0 and m.get_knob("tile_order") == 0
    with pytest.raises(ValueError):
        m.set_knob("no_such_knob", 1)


def test_pack_rejects_bad_arguments_before_launch():
    L = m.load_library()
    assert L.im2win_pack(None, FAKE, 1, 1, 4, 4, 2, 2, 1, 4, None) == _lib.IM2WIN_EINVAL
    assert L.im2win_pack(FAKE, None, 1, 1, 4, 4, 2, 2, 1, 4, None) == _lib.IM2WIN_EINVAL
    assert L.im2win_pack(FAKE, FAKE, 1, 1, 4, 4, 2, 2, 1, 8, None) == _lib.IM2WIN_EINVAL
    assert L.im2win_pack(FAKE, FAKE, 1, 1, 4, 4, 5, 2, 1, 4, None) == _lib.IM2WIN_EINVAL
    assert L.im2win_pack(ctypes.c_void_p(0x10002), FAKE, 1, 1, 4, 4, 2, 2, 1, 4, None) == \
        _lib.IM2WIN_EINVAL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()


def test_one_hip_runtime_when_the_library_loads_before_torch():
    """Using the binding before importing torch must not map a second HIP
    runtime into the process (the library must bind to torch's)."""
    import subprocess
    import sys
    code = (
        "import memory_efficient_im2win_amd as m\n"
        "m.output_dims(8, 8, 3, 3, 1)\n"
        "import torch\n"
        "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
        "print(len(paths))\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "1", r.stdout


def test_im2col_workspace_bytes():
    # [filter padded to KP, 256-byte aligned | N*Ho*Wo rows of KP]; K = Ci*Hf*Wf
    # padded to 32 bytes. cv4 fp16: K = 3136 (already a multiple of 16).
    fb = -(-64 * 3136 * 2 // 256) * 256
    assert m.im2col_workspace_bytes(64, 64, 224, 224, 64, 7, 7, 2, 2) == fb + 64 * 109 * 109 * 3136 * 2
    # cv1 fp32: K = 363 -> 368
    fb = -(-96 * 368 * 4 // 256) * 256
    assert m.im2col_workspace_bytes(32, 3, 227, 227, 96, 11, 11, 4, 4) == fb + 32 * 55 * 55 * 368 * 4
    assert m.im2col_workspace_bytes(1, 3, 4, 4, 2, 5, 5, 1, 2) == 0
    assert m.im2col_workspace_bytes(1, 3, 8, 8, 2, 3, 3, (2, 1), 3) == 0


@pytest.mark.parametrize("fn", ["conv2d_im2col_fp32", "conv2d_im2col_fp16"])
def test_im2col_conv_rejects_bad_arguments(fn):
    L = m.load_library()
    f = getattr(L, fn)
    ok = (1, 3, 8, 8, 4, 3, 3, 1, 1)
    assert f(None, FAKE, FAKE, FAKE, 1 << 20, *ok, None) == _lib.IM2WIN_EINVAL
    assert f(FAKE, FAKE, FAKE, None, 0, *ok, None) == _lib.IM2WIN_EWORKSPACE
    assert f(FAKE, FAKE, FAKE, FAKE, 64, *ok, None) == _lib.IM2WIN_EWORKSPACE
    assert f(FAKE, FAKE, FAKE, FAKE, 1 << 20, 1, 3, 8, 8, 4, 3, 3, 0, 1, None) == _lib.IM2WIN_EINVAL
    assert f(FAKE, FAKE, FAKE, ctypes.c_void_p(0x10008), 1 << 20, *ok, None) == _lib.IM2WIN_EINVAL


def test_direct_and_im2col_pack_reject_bad_arguments():
    L = m.load_library()
    for f in (L.conv2d_direct_fp32, L.conv2d_direct_fp16):
        assert f(None, FAKE, FAKE, 1, 3, 8, 8, 4, 3, 3, 1, 1, None) == _lib.IM2WIN_EINVAL
        assert f(FAKE, FAKE, FAKE, 1, 3, 8, 8, 4, 9, 3, 1, 1, None) == _lib.IM2WIN_EINVAL
    assert L.im2col_pack(FAKE, None, 1, 1, 4, 4, 2, 2, 1, 1, 4, None) == _lib.IM2WIN_EINVAL
    assert L.im2col_pack(FAKE, FAKE, 1, 1, 4, 4, 2, 2, 1, 1, 8, None) == _lib.IM2WIN_EINVAL


def test_nhwc_workspace_bytes():
    # [filter in window order, 256-aligned | N * Ho*Wi*Hf*Ci]: the NHWC im2win
    # tensor has the size of the NCHW one.
    fb = -(-64 * 64 * 49 * 2 // 256) * 256
    assert m.nhwc_workspace_bytes(64, 64, 224, 224, 64, 7, 7, 2, 2) == \
        fb + m.workspace_bytes(64, 64, 224, 224, 7, 7, 2, 2)
    assert m.nhwc_workspace_bytes(64, 64, 224, 224, 64, 7, 7, 2, 2, materialize=False) == 0
    assert m.nhwc_workspace_bytes(1, 3, 4, 4, 2, 5, 5, 1, 2) == 0
    # Ci = 3, Hf = 11: each column's 33-element run padded to 32 bytes, 40
    # floats or 48 halves, in the filter rows and the tensor (Ho = 10).
    for e, pitch in ((4, 40), (2, 48)):
        fb = -(-37 * 11 * pitch * e // 256) * 256
        assert m.nhwc_workspace_bytes(2, 3, 47, 45, 37, 11, 11, 4, e) == fb + 2 * 10 * 45 * pitch * e


def test_nhwc_fused_workspace_bytes():
    """The fused NHWC call's workspace is the channel-interleaved filter:
    ceil(Ci/8) x (taps rounded up to even) x Co rounded up to 128 x 16 bytes,
    256-aligned; 0 for an invalid shape."""
    assert m.nhwc_fused_workspace_bytes(128, 96, 24, 24, 256, 5, 5, 1) == 12 * 26 * 256 * 16
    assert m.nhwc_fused_workspace_bytes(2, 13, 9, 9, 40, 3, 3, 1) == \
        -(-(2 * 10 * 128 * 16) // 256) * 256
    assert m.nhwc_fused_workspace_bytes(1, 3, 4, 4, 2, 5, 5, 1) == 0


def test_nhwc_fused_rejects_bad_arguments():
    L = m.load_library()
    f = L.conv2d_im2win_nhwc_fp16_fused
    ok = (1, 96, 12, 12, 256, 5, 5, 1, 1)
    assert f(None, FAKE, FAKE, None, 0, *ok, None) == _lib.IM2WIN_EINVAL
    assert f(FAKE, FAKE, FAKE, None, 64, *ok, None) == _lib.IM2WIN_EWORKSPACE
    need = L.conv2d_im2win_nhwc_fp16_fused_workspace_bytes(*ok)
    assert f(FAKE, FAKE, FAKE, FAKE, need - 16, *ok, None) == _lib.IM2WIN_EWORKSPACE
    assert f(FAKE, FAKE, FAKE, None, 0, 1, 96, 12, 12, 256, 5, 5, 1, 0, None) == _lib.IM2WIN_EINVAL


@pytest.mark.parametrize("fn", ["conv2d_im2win_nhwc_fp32", "conv2d_im2win_nhwc_fp16"])
def test_nhwc_conv_rejects_bad_arguments(fn):
    L = m.load_library()
    f = getattr(L, fn)
    ok = (1, 16, 8, 8, 4, 3, 3, 1, 1)
    assert f(None, FAKE, FAKE, None, 0, *ok, None) == _lib.IM2WIN_EINVAL
    assert f(FAKE, FAKE, FAKE, None, 64, *ok, None) == _lib.IM2WIN_EWORKSPACE
    assert f(FAKE, FAKE, FAKE, FAKE, 64, *ok, None) == _lib.IM2WIN_EWORKSPACE
    assert f(FAKE, FAKE, FAKE, None, 0, 1, 16, 8, 8, 4, 3, 3, 1, 0, None) == _lib.IM2WIN_EINVAL
    assert L.im2win_pack_nhwc(FAKE, None, 1, 1, 4, 4, 2, 2, 1, 1, 4, None) == _lib.IM2WIN_EINVAL


def test_binding_checks_workspace_extent():
    """A workspace byte count past the tensor, or a tensor on another device,
    is refused before the library is called (stand-in tensor objects; no GPU
    needed)."""
    from memory_efficient_im2win_amd import _ws_arg

    class Dev:
        def __init__(self, i):
            self.i = i

        def __eq__(self, o):
            return self.i == o.i

    class T:
        is_cuda = True

        def __init__(self, n, dev=0):
            self.n, self.device = n, Dev(dev)

        def is_contiguous(self):
            return True

        def numel(self):
            return self.n

        def element_size(self):
            return 1

        def data_ptr(self):
            return 0x10000

    x = T(1)
    assert _ws_arg(T(100), None, x, "ws")[1] == 100
    assert _ws_arg(T(100), 60, x, "ws")[1] == 60
    with pytest.raises(ValueError):
        _ws_arg(T(100), 101, x, "ws")
    with pytest.raises(ValueError):
        _ws_arg(T(100, dev=1), None, x, "ws")
    with pytest.raises(ValueError):
        _ws_arg(None, 64, x, "ws")


def test_conv_kernel_name():
    """The fp16 kernel a call runs, as the planners pick it (no GPU needed;
    the fp32 planner asks the device for occupancy, so its names are checked
    on the GPU)."""
    assert m.conv_kernel_name(64, 64, 224, 224, 64, 7, 7, 2, 2) == "conv_f16_reuse_kernel"
    with m.knobs(f16_reuse=-1):
        assert m.conv_kernel_name(64, 64, 224, 224, 64, 7, 7, 2, 2) == "conv_f16_rows_kernel"
    assert m.conv_kernel_name(64, 3, 227, 227, 64, 7, 7, 2, 2) == "conv_f16_thin_kernel"
    assert m.conv_kernel_name(128, 96, 24, 24, 256, 5, 5, 1, 2) == "conv_f16_wide_kernel"
    assert m.conv_kernel_name(128, 96, 24, 24, 256, 5, 5, 1, 2, "prepacked") == \
        "conv_f16_res_kernel"
    assert m.conv_kernel_name(128, 96, 24, 24, 256, 5, 5, 1, 2, "nhwc_prepacked") == \
        "conv_f16_res_kernel"
    assert m.conv_kernel_name(64, 64, 224, 224, 64, 7, 7, 2, 2, "nhwc_prepacked") == \
        "conv_direct_nhwc_kernel"
    with m.knobs(f16_res=-1):
        assert m.conv_kernel_name(128, 96, 24, 24, 256, 5, 5, 1, 2, "prepacked") == \
            "conv_f16_wide_kernel"
    with m.knobs(f16_rows=-1, f16_thin=-1, f16_wide=-1):
        assert m.conv_kernel_name(64, 64, 224, 224, 64, 7, 7, 2, 2, "prepacked") == \
            "conv_f16_fused_kernel"
    assert m.conv_kernel_name(64, 64, 224, 224, 64, 7, 7, 2, 2, "materialized") == \
        "conv_f16_ws_kernel"
    assert m.conv_kernel_name(128, 96, 24, 24, 256, 5, 5, 1, 2, "materialized") == \
        "conv_f16_ws_kernel"
    assert m.conv_kernel_name(64, 3, 227, 227, 64, 7, 7, 2, 2, "materialized") == "conv_f16_kernel"
    with m.knobs(f16_ws=-1):
        assert m.conv_kernel_name(64, 64, 224, 224, 64, 7, 7, 2, 2, "materialized") == \
            "conv_f16_kernel"
    with pytest.raises(ValueError):
        m.conv_kernel_name(1, 3, 4, 4, 2, 5, 5, 1, 2)


def test_noalloc_rejects_before_launch():
    """The entry point without allocation refuses bad arguments and shapes
    whose filter scratch exceeds its 4 MiB before touching the GPU."""
    L = m.load_library()
    f = L.conv2d_im2win_fp16_fused_noalloc
    ok = (1, 3, 8, 8, 4, 3, 3, 1, 1)
    assert f(None, FAKE, FAKE, *ok, None) == _lib.IM2WIN_EINVAL
    assert f(FAKE, FAKE, FAKE, 1, 3, 8, 8, 4, 9, 3, 1, 1, None) == _lib.IM2WIN_EINVAL
    assert f(ctypes.c_void_p(0x10001), FAKE, FAKE, *ok, None) == _lib.IM2WIN_EINVAL
    big = (1, 512, 16, 16, 512, 7, 7, 1, 1)   # filter scratch > 4 MiB
    assert L.conv2d_im2win_fp16_fused_workspace_bytes(*big) > 4 << 20
    assert f(FAKE, FAKE, FAKE, *big, None) == _lib.IM2WIN_EWORKSPACE


def test_peak_probe_host_side():
    """The rate probe's flop count (host arithmetic) and its argument checks
    (rejected before anything is enqueued)."""
    L = m.load_library()
    assert L.im2win_peak_probe_flops(2, 512, 10) == 512 * 4 * 10 * 4 * 32 * 32 * 16 * 2
    assert L.im2win_peak_probe_flops(1, 1, 1) == 4 * 4 * 32 * 32 * 2 * 2
    assert L.im2win_peak_probe_flops(0, 1, 1) == 4 * 64 * 4 * 8 * 2
    assert L.im2win_peak_probe_flops(3, 1, 1) == 0.0
    assert L.im2win_peak_probe(3, 1, 1, ctypes.c_void_p(256), None) == _lib.IM2WIN_EINVAL
    assert L.im2win_peak_probe(2, 1, 1, None, None) == _lib.IM2WIN_EINVAL
    assert L.im2win_peak_probe(2, 0, 1, ctypes.c_void_p(256), None) == _lib.IM2WIN_EINVAL
