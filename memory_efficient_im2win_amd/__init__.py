"""im2win convolution for AMD Instinct MI355X (gfx950).

A thin binding over libim2win.so: it checks tensor dtypes, devices and
layouts, allocates outputs with torch, and passes raw device pointers and
torch's current HIP stream to the C ABI. Every step of the computation runs
in the library's HIP kernels.

    y = conv2d(x, w, stride)                 # fused: im2win rows built in LDS
    y = conv2d(x, w, stride, ws=workspace)   # materialised im2win tensor
    y = conv2d_fused(x, w, stride, fws=f)    # fp16 fused, filter prepacked into f
    ws = pack(x, Hf, Wf, stride)             # the im2win transform itself
    with knobs(f16_rows=-1): ...             # planner overrides (tests, ablation)

A stride is one int (both axes) or a pair (sh, sw): row stride, then column
stride. Equal strides go through the single-stride entry points of the C ABI,
unequal ones through their *_strided twins.
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import Im2winError, status_string  # noqa: F401

__all__ = ["conv2d", "conv2d_fused", "pack", "workspace_bytes", "fused_workspace_bytes",
           "output_dims", "strides", "knob_names", "set_knob", "get_knob", "knobs",
           "conv_kernel_name",
           "im2col", "im2col_workspace_bytes", "conv2d_im2col", "conv2d_direct",
           "pack_nhwc", "conv2d_nhwc", "nhwc_workspace_bytes",
           "Im2winError", "status_string", "load_library"]


def load_library():
    """The loaded ctypes library (raises ImportError if it was not built)."""
    return _lib.load()


def strides(s):
    """(sh, sw) of a stride given as one int or a pair."""
    if isinstance(s, (tuple, list)):
        if len(s) != 2:
            raise ValueError("a stride pair is (sh, sw)")
        return int(s[0]), int(s[1])
    return int(s), int(s)


def _entry(name, s):
    """The C entry point for stride s and the stride arguments to pass it."""
    sh, sw = strides(s)
    L = _lib.load()
    if sh == sw:
        return getattr(L, name), (sh,)
    return getattr(L, name + "_strided"), (sh, sw)


def output_dims(Hi: int, Wi: int, Hf: int, Wf: int, s):
    ho, wo = ctypes.c_int(), ctypes.c_int()
    fn, st = _entry("im2win_output_dims", s)
    _lib.check(fn(Hi, Wi, Hf, Wf, *st, ctypes.byref(ho), ctypes.byref(wo)), "output_dims")
    return ho.value, wo.value


def workspace_bytes(N, Ci, Hi, Wi, Hf, Wf, s, elem_bytes) -> int:
    """Bytes of the im2win tensor of the whole batch (0 for an invalid shape)."""
    fn, st = _entry("im2win_workspace_bytes", s)
    return fn(N, Ci, Hi, Wi, Hf, Wf, *st, elem_bytes)


def fused_workspace_bytes(N, Ci, Hi, Wi, Co, Hf, Wf, s) -> int:
    """Bytes conv2d_fused needs for its prepacked fp16 filter (0 for an
    invalid shape)."""
    sh, sw = strides(s)
    return _lib.load().conv2d_im2win_fp16_fused_workspace_bytes(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw)


def conv_kernel_name(N, Ci, Hi, Wi, Co, Hf, Wf, s, elem_bytes, mode: str = "fused") -> str:
    """Name of the main kernel a call runs (mode "fused", "prepacked" for
    conv2d_fused with a filter workspace, "materialized", or "nhwc_prepacked"
    for conv2d_nhwc_fused with a filter workspace, fp16)."""
    sh, sw = strides(s)
    code = {"fused": 0, "prepacked": 1, "materialized": 2, "nhwc_prepacked": 3}[mode]
    if code == 1 and elem_bytes == 4:
        code = 0
    r = _lib.load().im2win_conv_kernel_name(elem_bytes, code, N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw)
    if r is None:
        raise ValueError("invalid shape or mode")
    return r.decode()


PROBE_KINDS = {"fp32_vector": 0, "fp32_mfma": 1, "fp16_mfma": 2}


def peak_probe(kind: str, blocks: int, iters: int, out=None):
    """Enqueues the library's rate probe of `kind` (fp32_vector, fp32_mfma,
    fp16_mfma) on torch's current stream; returns (out, flops of the launch).
    out: a float32 device tensor of at least blocks * 256 elements."""
    torch = _torch()
    k = PROBE_KINDS[kind]
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    _check_tensor(out, "out", (torch.float32,), 1)
    if out.numel() < blocks * 256:
        raise ValueError("out holds fewer than blocks * 256 floats")
    L = _lib.load()
    _lib.check(L.im2win_peak_probe(k, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                                   _stream_handle(out)), "im2win_peak_probe")
    return out, L.im2win_peak_probe_flops(k, blocks, iters)


# ---- tuning knobs ------------------------------------------------------------
def knob_names():
    """Names of the library's tuning knobs, in the order of their ids."""
    L = _lib.load()
    out = []
    while True:
        n = L.im2win_knob_name(len(out))
        if n is None:
            return out
        out.append(n.decode())


def _knob_id(name: str) -> int:
    names = knob_names()
    if name not in names:
        raise ValueError(f"unknown knob {name!r}; known: {names}")
    return names.index(name)


def set_knob(name: str, value: int) -> None:
    """Sets a planner knob (0: the planner's choice). Process-wide; change
    knobs only while no call is running."""
    _lib.check(_lib.load().im2win_set_knob(_knob_id(name), int(value)), f"set_knob({name})")


def get_knob(name: str) -> int:
    return _lib.load().im2win_get_knob(_knob_id(name))


class knobs:
    """Context manager: ``with knobs(f16_rows=-1, tile_order=1): ...`` sets
    the given knobs and restores their previous values on exit."""

    def __init__(self, **values):
        self.values = values
        self.saved = {}

    def __enter__(self):
        for k, v in self.values.items():
            self.saved[k] = get_knob(k)
            set_knob(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self.saved.items():
            set_knob(k, v)
        return False


def _torch():
    import torch
    return torch


def _stream_handle(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check_tensor(t, name, dtypes, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def pack(x, Hf: int, Wf: int, s, out=None):
    """The im2win tensor of x (N, Ci, Hi, Wi) as (N, Ci, Ho, Wi*Hf), same dtype.

    Any 2- or 4-byte dtype works (the transform is a bit copy).
    """
    torch = _torch()
    _check_tensor(x, "x", (torch.float16, torch.float32, torch.int16, torch.int32,
                           torch.bfloat16, torch.uint16, torch.uint32), 4)
    N, Ci, Hi, Wi = x.shape
    Ho, _ = output_dims(Hi, Wi, Hf, Wf, s)
    shape = (N, Ci, Ho, Wi * Hf)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    fn, st = _entry("im2win_pack", s)
    _lib.check(fn(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                  N, Ci, Hi, Wi, Hf, Wf, *st, x.element_size(), _stream_handle(x)), fn.__name__)
    return out


def _ws_arg(ws, ws_bytes, x, name):
    """(pointer, byte count) of an optional workspace tensor on x's device;
    ws_bytes may name a prefix of it, never more."""
    if ws is None:
        if ws_bytes:
            raise ValueError(f"{name}_bytes given without {name}")
        return None, 0
    if not getattr(ws, "is_cuda", False) or not ws.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    if ws.device != x.device:
        raise ValueError(f"{name} must be on x's device")
    size = ws.numel() * ws.element_size()
    nbytes = size if ws_bytes is None else int(ws_bytes)
    if nbytes < 0 or nbytes > size:
        raise ValueError(f"{name}_bytes={nbytes} is outside the {size}-byte {name} tensor")
    return ctypes.c_void_p(ws.data_ptr()), nbytes


def conv2d(x, w, stride=1, ws=None, ws_bytes: int | None = None, out=None):
    """Forward convolution (cross-correlation, no padding) of x (N,Ci,Hi,Wi)
    with w (Co,Ci,Hf,Wf); fp32 output (N,Co,Ho,Wo).

    float32 inputs run on the fp32 matrix instructions (the vector-ALU kernel
    with knob f32_valu=1), float16 inputs on the fp16 matrix instructions
    with fp32 accumulation. Without ``ws`` the im2win rows are built in LDS
    (fused). With ``ws`` (a device tensor of at least one image's im2win
    bytes; ``workspace_bytes(N, ...)`` for the whole batch) the im2win tensor
    is materialised in it, in chunks of as many images as fit. ``ws_bytes``
    may restrict the call to a prefix of ``ws``.
    """
    torch = _torch()
    _check_tensor(x, "x", (torch.float32, torch.float16), 4)
    _check_tensor(w, "w", (x.dtype,), 4)
    if w.device != x.device:
        raise ValueError("x and w must be on the same device")
    N, Ci, Hi, Wi = x.shape
    Co, Ci2, Hf, Wf = w.shape
    if Ci2 != Ci:
        raise ValueError("x and w disagree on the input channel count")
    Ho, Wo = output_dims(Hi, Wi, Hf, Wf, stride)
    if out is None:
        out = torch.empty((N, Co, Ho, Wo), dtype=torch.float32, device=x.device)
    elif (tuple(out.shape) != (N, Co, Ho, Wo) or out.dtype != torch.float32
          or not out.is_contiguous() or out.device != x.device):
        raise ValueError("out has the wrong shape, dtype, device or layout")
    ws_ptr, nbytes = _ws_arg(ws, ws_bytes, x, "ws")
    fn, st = _entry("conv2d_im2win_fp32" if x.dtype == torch.float32 else "conv2d_im2win_fp16",
                    stride)
    _lib.check(fn(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                  ctypes.c_void_p(out.data_ptr()), ws_ptr, nbytes,
                  N, Ci, Hi, Wi, Co, Hf, Wf, *st, _stream_handle(x)), fn.__name__)
    return out


def conv2d_fused(x, w, stride=1, fws=None, fws_bytes: int | None = None, out=None):
    """fp16 fused convolution with the filter prepacked per call into ``fws``
    (a device tensor of at least fused_workspace_bytes(...) bytes), then
    copied from there by the matrix-core kernel. Without ``fws`` the kernel
    gathers the filter from w, as conv2d does without a workspace."""
    torch = _torch()
    dims, out = _conv_args(x, w, stride, out)
    if x.dtype != torch.float16:
        raise TypeError("conv2d_fused takes float16 inputs")
    ptr, nbytes = _ws_arg(fws, fws_bytes, x, "fws")
    L = _lib.load()
    _lib.check(L.conv2d_im2win_fp16_fused(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                                          ctypes.c_void_p(out.data_ptr()), ptr, nbytes, *dims,
                                          _stream_handle(x)), "conv2d_im2win_fp16_fused")
    return out


# ---- baselines: im2col + GEMM and direct convolution ------------------------
def im2col_workspace_bytes(N, Ci, Hi, Wi, Co, Hf, Wf, s, elem_bytes) -> int:
    """Workspace of conv2d_im2col for the whole batch (padded filter + im2col
    rows); 0 for an invalid shape."""
    sh, sw = strides(s)
    return _lib.load().conv2d_im2col_workspace_bytes(N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, elem_bytes)


def im2col(x, Hf: int, Wf: int, s):
    """The im2col matrix of x (N, Ci, Hi, Wi): (N*Ho*Wo, KP) rows of
    Ci*Hf*Wf elements in (ci, kh, kw) order, zero-padded to 32 bytes."""
    torch = _torch()
    _check_tensor(x, "x", (torch.float16, torch.float32, torch.int16, torch.int32,
                           torch.bfloat16, torch.uint16, torch.uint32), 4)
    N, Ci, Hi, Wi = x.shape
    Ho, Wo = output_dims(Hi, Wi, Hf, Wf, s)
    e = x.element_size()
    K = Ci * Hf * Wf
    KP = -(-K // (32 // e)) * (32 // e)
    out = torch.empty((N * Ho * Wo, KP), dtype=x.dtype, device=x.device)
    sh, sw = strides(s)
    _lib.check(_lib.load().im2col_pack(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                       N, Ci, Hi, Wi, Hf, Wf, sh, sw, e, _stream_handle(x)),
               "im2col_pack")
    return out


def _conv_args(x, w, stride, out=None):
    torch = _torch()
    _check_tensor(x, "x", (torch.float32, torch.float16), 4)
    _check_tensor(w, "w", (x.dtype,), 4)
    if w.device != x.device:
        raise ValueError("x and w must be on the same device")
    N, Ci, Hi, Wi = x.shape
    Co, Ci2, Hf, Wf = w.shape
    if Ci2 != Ci:
        raise ValueError("x and w disagree on the input channel count")
    Ho, Wo = output_dims(Hi, Wi, Hf, Wf, stride)
    if out is None:
        out = torch.empty((N, Co, Ho, Wo), dtype=torch.float32, device=x.device)
    elif (tuple(out.shape) != (N, Co, Ho, Wo) or out.dtype != torch.float32
          or not out.is_contiguous() or out.device != x.device):
        raise ValueError("out has the wrong shape, dtype, device or layout")
    return (N, Ci, Hi, Wi, Co, Hf, Wf) + strides(stride), out


def conv2d_im2col(x, w, stride=1, ws=None, out=None):
    """Baseline: im2col into the workspace, then a matrix-core GEMM (fp32
    output). ws defaults to the whole batch's im2col_workspace_bytes."""
    torch = _torch()
    dims, out = _conv_args(x, w, stride, out)
    if ws is None:
        nb = _lib.load().conv2d_im2col_workspace_bytes(*dims, x.element_size())
        ws = torch.empty(nb, dtype=torch.uint8, device=x.device)
    fn = _lib.load().conv2d_im2col_fp32 if x.dtype == torch.float32 else _lib.load().conv2d_im2col_fp16
    _lib.check(fn(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                  ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                  ws.numel() * ws.element_size(), *dims, _stream_handle(x)), fn.__name__)
    return out


def conv2d_direct(x, w, stride=1, out=None):
    """Baseline: direct convolution, one thread per output (fp32 output)."""
    torch = _torch()
    dims, out = _conv_args(x, w, stride, out)
    fn = _lib.load().conv2d_direct_fp32 if x.dtype == torch.float32 else _lib.load().conv2d_direct_fp16
    _lib.check(fn(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                  ctypes.c_void_p(out.data_ptr()), *dims, _stream_handle(x)), fn.__name__)
    return out


# ---- NHWC tensors ------------------------------------------------------------
def nhwc_workspace_bytes(N, Ci, Hi, Wi, Co, Hf, Wf, s, elem_bytes, materialize: bool = True) -> int:
    """Workspace of conv2d_nhwc: 0 without materialize, else the filter in
    window order plus the NHWC im2win tensor of the whole batch."""
    sh, sw = strides(s)
    return _lib.load().conv2d_im2win_nhwc_workspace_bytes(1 if materialize else 0, N, Ci, Hi, Wi, Co,
                                                          Hf, Wf, sh, sw, elem_bytes)


def pack_nhwc(x, Hf: int, Wf: int, s):
    """The NHWC im2win tensor of x (N, Hi, Wi, Ci) as (N, Ho, Wi, Hf, Ci)."""
    torch = _torch()
    _check_tensor(x, "x", (torch.float16, torch.float32, torch.int16, torch.int32,
                           torch.bfloat16, torch.uint16, torch.uint32), 4)
    N, Hi, Wi, Ci = x.shape
    Ho, _ = output_dims(Hi, Wi, Hf, Wf, s)
    out = torch.empty((N, Ho, Wi, Hf, Ci), dtype=x.dtype, device=x.device)
    sh, sw = strides(s)
    _lib.check(_lib.load().im2win_pack_nhwc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                            N, Ci, Hi, Wi, Hf, Wf, sh, sw, x.element_size(),
                                            _stream_handle(x)), "im2win_pack_nhwc")
    return out


def nhwc_fused_workspace_bytes(N, Ci, Hi, Wi, Co, Hf, Wf, s) -> int:
    """Workspace of conv2d_nhwc_fused (fp16): the prepacked filter's bytes;
    0 for an invalid shape."""
    sh, sw = strides(s)
    return _lib.load().conv2d_im2win_nhwc_fp16_fused_workspace_bytes(N, Ci, Hi, Wi, Co, Hf, Wf,
                                                                     sh, sw)


def conv2d_nhwc_fused(x, w, stride=1, fws=None, fws_bytes: int | None = None, out=None):
    """fp16 NHWC convolution without an im2win tensor: x (N, Hi, Wi, Ci), w
    (Co, Ci, Hf, Wf), fp32 NHWC output (N, Ho, Wo, Co). With ``fws`` (at
    least nhwc_fused_workspace_bytes(...) bytes) the filter is prepacked into
    it and the resident-input kernel runs where its envelope allows; without
    it, and outside the envelope, the direct NHWC kernel."""
    torch = _torch()
    _check_tensor(x, "x", (torch.float16,), 4)
    _check_tensor(w, "w", (torch.float16,), 4)
    if w.device != x.device:
        raise ValueError("x and w must be on the same device")
    N, Hi, Wi, Ci = x.shape
    Co, Ci2, Hf, Wf = w.shape
    if Ci2 != Ci:
        raise ValueError("x and w disagree on the input channel count")
    Ho, Wo = output_dims(Hi, Wi, Hf, Wf, stride)
    if out is None:
        out = torch.empty((N, Ho, Wo, Co), dtype=torch.float32, device=x.device)
    elif (tuple(out.shape) != (N, Ho, Wo, Co) or out.dtype != torch.float32
          or not out.is_contiguous() or out.device != x.device):
        raise ValueError("out has the wrong shape, dtype, device or layout")
    ptr, nbytes = _ws_arg(fws, fws_bytes, x, "fws")
    sh, sw = strides(stride)
    _lib.check(_lib.load().conv2d_im2win_nhwc_fp16_fused(
        ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        ptr, nbytes, N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw, _stream_handle(x)),
        "conv2d_im2win_nhwc_fp16_fused")
    return out


def conv2d_nhwc(x, w, stride=1, ws=None, out=None):
    """Convolution of an NHWC x (N, Hi, Wi, Ci) with w (Co, Ci, Hf, Wf); fp32
    NHWC output (N, Ho, Wo, Co). Without ws: direct; with ws (see
    nhwc_workspace_bytes): the NHWC im2win tensor is materialised and
    multiplied on the matrix cores."""
    torch = _torch()
    _check_tensor(x, "x", (torch.float32, torch.float16), 4)
    _check_tensor(w, "w", (x.dtype,), 4)
    if w.device != x.device:
        raise ValueError("x and w must be on the same device")
    N, Hi, Wi, Ci = x.shape
    Co, Ci2, Hf, Wf = w.shape
    if Ci2 != Ci:
        raise ValueError("x and w disagree on the input channel count")
    Ho, Wo = output_dims(Hi, Wi, Hf, Wf, stride)
    if out is None:
        out = torch.empty((N, Ho, Wo, Co), dtype=torch.float32, device=x.device)
    elif (tuple(out.shape) != (N, Ho, Wo, Co) or out.dtype != torch.float32
          or not out.is_contiguous() or out.device != x.device):
        raise ValueError("out has the wrong shape, dtype, device or layout")
    if ws is None:
        ws_ptr, nbytes = None, 0
    else:
        if not ws.is_cuda or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous GPU tensor")
        ws_ptr, nbytes = ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()
    sh, sw = strides(stride)
    fn = _lib.load().conv2d_im2win_nhwc_fp32 if x.dtype == torch.float32 else \
        _lib.load().conv2d_im2win_nhwc_fp16
    _lib.check(fn(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                  ctypes.c_void_p(out.data_ptr()), ws_ptr, nbytes, N, Ci, Hi, Wi, Co, Hf, Wf, sh, sw,
                  _stream_handle(x)), fn.__name__)
    return out
