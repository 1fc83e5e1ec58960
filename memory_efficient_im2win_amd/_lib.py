"""ctypes declarations of libim2win.so (the C ABI in include/im2win.h).

Loading fails loudly if the library has not been built: there is no
fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libim2win.so")

IM2WIN_OK = 0
IM2WIN_EINVAL = -1
IM2WIN_EWORKSPACE = -2
IM2WIN_ELAUNCH = -3

_i = ctypes.c_int
_sz = ctypes.c_size_t
_p = ctypes.c_void_p

EXPORTS = {
    "im2win_workspace_bytes": ([_i] * 7 + [_sz], _sz),
    "im2win_output_dims": ([_i] * 5 + [ctypes.POINTER(_i), ctypes.POINTER(_i)], _i),
    "im2win_pack": ([_p, _p] + [_i] * 7 + [_sz, _p], _i),
    "conv2d_im2win_fp32": ([_p, _p, _p, _p, _sz] + [_i] * 8 + [_p], _i),
    "conv2d_im2win_fp16": ([_p, _p, _p, _p, _sz] + [_i] * 8 + [_p], _i),
    "im2win_workspace_bytes_strided": ([_i] * 8 + [_sz], _sz),
    "im2win_output_dims_strided": ([_i] * 6 + [ctypes.POINTER(_i), ctypes.POINTER(_i)], _i),
    "im2win_pack_strided": ([_p, _p] + [_i] * 8 + [_sz, _p], _i),
    "conv2d_im2win_fp32_strided": ([_p, _p, _p, _p, _sz] + [_i] * 9 + [_p], _i),
    "conv2d_im2win_fp16_strided": ([_p, _p, _p, _p, _sz] + [_i] * 9 + [_p], _i),
    "conv2d_im2win_fp16_fused_workspace_bytes": ([_i] * 9, _sz),
    "conv2d_im2win_fp16_fused": ([_p, _p, _p, _p, _sz] + [_i] * 9 + [_p], _i),
    "conv2d_im2win_fp16_fused_noalloc": ([_p, _p, _p] + [_i] * 9 + [_p], _i),
    "im2win_set_knob": ([_i, _i], _i),
    "im2win_get_knob": ([_i], _i),
    "im2win_knob_name": ([_i], ctypes.c_char_p),
    "im2win_conv_kernel_name": ([_i] * 11, ctypes.c_char_p),
    "im2win_status_string": ([_i], ctypes.c_char_p),
    "im2win_last_error": ([], ctypes.c_char_p),
    "conv2d_im2col_workspace_bytes": ([_i] * 9 + [_sz], _sz),
    "im2col_pack": ([_p, _p] + [_i] * 8 + [_sz, _p], _i),
    "conv2d_im2col_fp32": ([_p, _p, _p, _p, _sz] + [_i] * 9 + [_p], _i),
    "conv2d_im2col_fp16": ([_p, _p, _p, _p, _sz] + [_i] * 9 + [_p], _i),
    "conv2d_direct_fp32": ([_p, _p, _p] + [_i] * 9 + [_p], _i),
    "conv2d_direct_fp16": ([_p, _p, _p] + [_i] * 9 + [_p], _i),
    "conv2d_im2win_nhwc_workspace_bytes": ([_i] * 10 + [_sz], _sz),
    "im2win_pack_nhwc": ([_p, _p] + [_i] * 8 + [_sz, _p], _i),
    "conv2d_im2win_nhwc_fp32": ([_p, _p, _p, _p, _sz] + [_i] * 9 + [_p], _i),
    "conv2d_im2win_nhwc_fp16": ([_p, _p, _p, _p, _sz] + [_i] * 9 + [_p], _i),
    "conv2d_im2win_nhwc_fp16_fused_workspace_bytes": ([_i] * 9, _sz),
    "conv2d_im2win_nhwc_fp16_fused": ([_p, _p, _p, _p, _sz] + [_i] * 9 + [_p], _i),
    "im2win_peak_probe": ([_i, _i, _i, _p, _p], _i),
    "im2win_peak_probe_flops": ([_i, _i, _i], ctypes.c_double),
}

_lib = None


class Im2winError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = f"{what}: {status_string(status)} (status {status})"
        if status == IM2WIN_ELAUNCH:
            msg += f": {load().im2win_last_error().decode()}"
        super().__init__(msg)


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()' from the repository root)")
    # torch carries its own HIP runtime, which it loads by the unversioned
    # file name; libim2win.so asks for the versioned soname. Loaded after
    # torch, the library binds to torch's runtime (same soname); loaded
    # first, it would pull in a second runtime that torch then cannot share,
    # and device pointers and streams would not be valid across the two.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in EXPORTS.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().im2win_status_string(status).decode()


def check(status: int, what: str) -> None:
    if status != IM2WIN_OK:
        raise Im2winError(status, what)
