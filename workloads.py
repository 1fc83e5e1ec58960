"""Seeded synthetic inputs and layer shapes for im2win convolution.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark. It holds the layer shapes and the random-number recipe only; it
contains none of the convolution or im2win arithmetic.

Layer shapes follow Table I of "Enabling Memory-efficient Im2win Convolution
with Multi-precision Support on GPU CUDA and Tensor Cores" (input
Ci x Hi x Wi, filter Co x Hf x Wf with stride s, output Co x Ho x Wo; the
input channel count of the filter is the input's). The pages benchmark on
these layer shapes, not on a dataset, so the values are synthetic:

* "uniform" inputs: one ``numpy.random.default_rng(seed)``; x is drawn first,
  then w, each iid U[-1, 1) in float64, then rounded to nearest-even into the
  compute dtype (float32 or float16). Oracle and GPU see the same rounded
  arrays.
* "int" inputs: ``default_rng(seed).integers(-4, 5)`` (x first, then w), so
  every partial sum of a dot product is an exact small integer.
* "bits" inputs (pack only): arbitrary bit patterns of the element width,
  NaN/Inf/subnormal payloads included.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class ConvShape:
    """One forward convolution: NCHW input, Co x Ci x Hf x Wf filters, stride s
    (one int for both axes, or a pair (sh, sw): row stride, column stride)."""

    name: str
    N: int
    Ci: int
    Hi: int
    Wi: int
    Co: int
    Hf: int
    Wf: int
    s: "int | tuple[int, int]"
    dtype: str  # "f32" or "f16" (inputs and filters); output is always f32

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.float16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    # Sizes derived from the shape only (no method arithmetic).
    @property
    def x_shape(self):
        return (self.N, self.Ci, self.Hi, self.Wi)

    @property
    def w_shape(self):
        return (self.Co, self.Ci, self.Hf, self.Wf)

    def with_batch(self, N: int) -> "ConvShape":
        return replace(self, N=N)

    def describe(self) -> str:
        return (f"{self.name}: N={self.N} {self.Ci}x{self.Hi}x{self.Wi} * "
                f"{self.Co}x{self.Ci}x{self.Hf}x{self.Wf} s={self.s} {self.dtype}")


# Table I rows cv1..cv5 (the pages' extracted rows), at the batch sizes and
# precisions the benchmark runs them.
CV5_F32 = ConvShape("cv5", 1, 96, 24, 24, 256, 5, 5, 1, "f32")
CV1_F32 = ConvShape("cv1", 32, 3, 227, 227, 96, 11, 11, 4, "f32")
CV5_F16 = ConvShape("cv5", 128, 96, 24, 24, 256, 5, 5, 1, "f16")
CV3_F16 = ConvShape("cv3", 64, 3, 227, 227, 64, 7, 7, 2, "f16")
CV4_F16 = ConvShape("cv4", 64, 64, 224, 224, 64, 7, 7, 2, "f16")
CV2_F32 = ConvShape("cv2", 32, 3, 231, 231, 96, 11, 11, 4, "f32")

#: The five benchmark workloads, in order: the small fp32 case first, then the
#: fp32 headline layer, then the three fp16 (fp32-accumulate) layers.
CONFIGS = [CV5_F32, CV1_F32, CV5_F16, CV3_F16, CV4_F16]
BY_KEY = {
    "cv5_f32_n1": CV5_F32,
    "cv1_f32_n32": CV1_F32,
    "cv5_f16_n128": CV5_F16,
    "cv3_f16_n64": CV3_F16,
    "cv4_f16_n64": CV4_F16,
    "cv2_f32_n32": CV2_F32,
}


def make_inputs(shape: ConvShape, seed: int = 0, mode: str = "uniform"):
    """Return (x, w) as contiguous numpy arrays in the shape's dtype.

    ``mode`` is "uniform" (iid U[-1,1) rounded to the dtype) or "int"
    (iid integers in [-4, 4]). x is always drawn before w from one generator.
    """
    rng = np.random.default_rng(seed)
    dt = shape.np_dtype
    if mode == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape.x_shape).astype(dt)
        w = rng.uniform(-1.0, 1.0, size=shape.w_shape).astype(dt)
    elif mode == "int":
        x = rng.integers(-4, 5, size=shape.x_shape).astype(dt)
        w = rng.integers(-4, 5, size=shape.w_shape).astype(dt)
    else:
        raise ValueError(f"unknown input mode {mode!r}")
    return np.ascontiguousarray(x), np.ascontiguousarray(w)


def make_bits(shape: ConvShape, seed: int = 0):
    """Random bit patterns with the input's shape and element width (pack tests).

    Returned as an unsigned integer array (uint16 or uint32) so that no value
    is ever interpreted as a float.
    """
    rng = np.random.default_rng(seed)
    ut = np.uint32 if shape.elem_bytes == 4 else np.uint16
    info = np.iinfo(ut)
    return rng.integers(0, int(info.max) + 1, size=shape.x_shape, dtype=ut)


def sample_output_indices(shape: ConvShape, Ho: int, Wo: int, count: int, seed: int = 7):
    """Flat NCHW output indices to check one by one at full size.

    Includes the first and last element of the output and the corners of the
    first and last image, plus ``count`` uniformly random positions.
    """
    total = shape.N * shape.Co * Ho * Wo
    rng = np.random.default_rng(seed)
    fixed = [0, total - 1, Wo - 1, (Ho - 1) * Wo, Ho * Wo - 1,
             (shape.N - 1) * shape.Co * Ho * Wo, total - Ho * Wo]
    rnd = rng.integers(0, total, size=count, dtype=np.int64)
    idx = np.unique(np.concatenate([np.array(fixed, dtype=np.int64), rnd]))
    return idx[(idx >= 0) & (idx < total)]
