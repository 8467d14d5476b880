"""Seeded synthetic inputs for grouped 2-D convolution (NCHW, float32).

This module only draws random numbers. It does no convolution arithmetic, so
the GPU path and the CPU oracle can both be fed from it without sharing any
part of the method. Every tensor comes from ``numpy.random.default_rng``
(PCG64) with seed ``1000*config_index + t``, where t is 0 for x, 1 for w, 2
for bias and 3 for dy.

The workloads below carry the shapes and value distributions the pages
measure or motivate:
  tiny_grouped   the NNlib grouped-conv benchmark shape ("Support groups in
                 DenseConvDims": Float32 input 28x28x100x2, filter 3x3x20x15,
                 groups 5, uniform [0,1) values as rand() draws them).
  dense3x3       the 3x3, 64->64, 56x56 convolution of the DLPrimitives Blog
                 OneDNN comparison ("Attempt to integrate with OneDNN").
  alexnet_conv2  the grouped (G=2) 5x5 layer of the AlexNet family the
                 DLPrimitives Blog validates; post-ReLU input.
  resnext_32x4d  the 32-group 3x3 layer of resnext50_32x4d, which the same
                 blog validates (4 in / 4 out channels per group).
  fc_mode        the kernel==input problem of "SpatialConvolution running in
                 fully-connected mode is very slow, even with R4": 1600 images
                 of 256x6x6 into 4096 planes with a 6x6 kernel.
  mobilenet_dw   a depthwise 3x3 layer (groups = channels = 144, one filter
                 per channel) of the mobilenet family the DLPrimitives Blog
                 validates, at 56x56 with the batch of the ResNeXt shapes;
                 post-ReLU input, no bias.
  resnext_1x1    the 1x1 (pointwise) 256->128 reduction that precedes the
                 grouped 3x3 in a resnext50_32x4d block, at the same 56x56
                 size and batch; post-ReLU input, no bias (the pages treat a
                 1x1 conv as a per-image GEMM unless its input is 1x1, in the
                 cudnn.torch fully-connected-mode issue).
  mobilenet_dw_s2_same
                 the stride-2 depthwise 3x3 of the same mobilenet family
                 (144 channels, 56x56 -> 28x28) with TensorFlow's "same"
                 padding, which puts the one padding row and column at the
                 end only (DLPrimitives Blog, "TensorFlow"): padding given as
                 (top, bottom, left, right) = (0, 1, 0, 1).
  resnext_32x4d_s2
                 the stride-2 grouped 3x3 that opens a later stage of
                 resnext50_32x4d (DLPrimitives Blog validates the network):
                 256 channels in 32 groups of 8, 56x56 -> 28x28, pad 1, no
                 bias (the strided-path "next" row).
  dense3x3_nhwc, resnext_1x1_nhwc, mobilenet_dw_nhwc
                 dense3x3, resnext_1x1 and mobilenet_dw with x, dx, y and dy stored
                 channels-last, the layout the DLPrimitives Blog measures
                 oneDNN fastest in ("Attempt to integrate with OneDNN");
                 make_inputs returns the same NCHW arrays for them and the
                 caller stores them transposed.
No dataset or trained weight is involved; normals use the second parameter
as the standard deviation (He/LeCun scales sqrt(2/fan_in), sqrt(1/fan_in)).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "WORKLOAD_ORDER", "make_inputs", "draw"]


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                      # seeds are 1000*index + t
    x_shape: tuple                  # [N, C, H, W]
    w_shape: tuple                  # [K, C/G, kh, kw]
    dy_shape: tuple                 # [N, K, Ho, Wo] as the workload states it
    groups: int
    stride: int
    padding: int | tuple            # int, or (top, bottom, left, right)
    dilation: int
    x_dist: tuple                   # ("uniform",) | ("normal", std) | ("relu_normal", std)
    w_dist: tuple
    b_dist: tuple | None            # None: the forward pass runs without bias
    dy_dist: tuple = ("normal", 1.0)
    note: str = field(default="", compare=False)
    layout: str = "nchw"            # storage of x, dx, y, dy on the device ("nchw" | "nhwc")


WORKLOADS = {
    "tiny_grouped": Workload(
        "tiny_grouped", 1, (2, 100, 28, 28), (15, 20, 3, 3), (2, 15, 26, 26), 5, 1, 0, 1,
        ("uniform",), ("uniform",), ("normal", 1.0),
        note="G=5: 20 in / 3 out channels per group"),
    "dense3x3": Workload(
        "dense3x3", 2, (32, 64, 56, 56), (64, 64, 3, 3), (32, 64, 56, 56), 1, 1, 1, 1,
        ("normal", 1.0), ("normal", float(np.sqrt(2.0 / 576.0))), ("normal", 0.01)),
    "alexnet_conv2": Workload(
        "alexnet_conv2", 3, (128, 96, 27, 27), (256, 48, 5, 5), (128, 256, 27, 27), 2, 1, 2, 1,
        ("relu_normal", 1.0), ("normal", 0.01), ("normal", 0.01)),
    "resnext_32x4d": Workload(
        "resnext_32x4d", 4, (64, 128, 56, 56), (128, 4, 3, 3), (64, 128, 56, 56), 32, 1, 1, 1,
        ("normal", 1.0), ("normal", float(np.sqrt(2.0 / 36.0))), None),
    "fc_mode": Workload(
        "fc_mode", 5, (1600, 256, 6, 6), (4096, 256, 6, 6), (1600, 4096, 1, 1), 1, 1, 0, 1,
        ("normal", 1.0), ("normal", float(np.sqrt(1.0 / 9216.0))), ("normal", 0.01)),
    "resnext_1x1": Workload(
        "resnext_1x1", 6, (64, 256, 56, 56), (128, 256, 1, 1), (64, 128, 56, 56), 1, 1, 0, 1,
        ("relu_normal", 1.0), ("normal", float(np.sqrt(2.0 / 256.0))), None),
    "mobilenet_dw": Workload(
        "mobilenet_dw", 7, (64, 144, 56, 56), (144, 1, 3, 3), (64, 144, 56, 56), 144, 1, 1, 1,
        ("relu_normal", 1.0), ("normal", float(np.sqrt(2.0 / 9.0))), None),
    "mobilenet_dw_s2_same": Workload(
        "mobilenet_dw_s2_same", 8, (64, 144, 56, 56), (144, 1, 3, 3), (64, 144, 28, 28), 144, 2,
        (0, 1, 0, 1), 1, ("relu_normal", 1.0), ("normal", float(np.sqrt(2.0 / 9.0))), None),
    "resnext_32x4d_s2": Workload(
        "resnext_32x4d_s2", 9, (64, 256, 56, 56), (256, 8, 3, 3), (64, 256, 28, 28), 32, 2, 1, 1,
        ("normal", 1.0), ("normal", float(np.sqrt(2.0 / 72.0))), None),
    # The same tensors as dense3x3, resnext_1x1 and mobilenet_dw (same seeds), stored channels-last.
    "dense3x3_nhwc": Workload(
        "dense3x3_nhwc", 2, (32, 64, 56, 56), (64, 64, 3, 3), (32, 64, 56, 56), 1, 1, 1, 1,
        ("normal", 1.0), ("normal", float(np.sqrt(2.0 / 576.0))), ("normal", 0.01), layout="nhwc"),
    "mobilenet_dw_nhwc": Workload(
        "mobilenet_dw_nhwc", 7, (64, 144, 56, 56), (144, 1, 3, 3), (64, 144, 56, 56), 144, 1, 1, 1,
        ("relu_normal", 1.0), ("normal", float(np.sqrt(2.0 / 9.0))), None, layout="nhwc"),
    "resnext_1x1_nhwc": Workload(
        "resnext_1x1_nhwc", 6, (64, 256, 56, 56), (128, 256, 1, 1), (64, 128, 56, 56), 1, 1, 0, 1,
        ("relu_normal", 1.0), ("normal", float(np.sqrt(2.0 / 256.0))), None, layout="nhwc"),
}
WORKLOAD_ORDER = ["tiny_grouped", "dense3x3", "alexnet_conv2", "resnext_32x4d", "fc_mode", "resnext_1x1",
                  "mobilenet_dw", "mobilenet_dw_s2_same", "resnext_32x4d_s2", "dense3x3_nhwc",
                  "resnext_1x1_nhwc", "mobilenet_dw_nhwc"]


def draw(dist, shape, seed) -> np.ndarray:
    """A float32 array of `shape` from distribution `dist`, seeded by `seed`."""
    rng = np.random.default_rng(seed)
    kind = dist[0]
    if kind == "uniform":
        return rng.random(shape, dtype=np.float32)          # [0, 1), never rounds to 1
    if kind == "normal":
        return (rng.standard_normal(shape, dtype=np.float32) * np.float32(dist[1]))
    if kind == "relu_normal":
        a = rng.standard_normal(shape, dtype=np.float32) * np.float32(dist[1])
        return np.maximum(a, np.float32(0.0))
    if kind == "int":                                         # integers in [lo, hi]
        return rng.integers(dist[1], dist[2] + 1, size=shape).astype(np.float32)
    raise ValueError("unknown distribution %r" % (dist,))


def make_inputs(name: str, batch: int | None = None) -> dict:
    """x, w, b (or None) and dy of workload `name` as float32 numpy arrays.

    With ``batch``, x and dy are cut to their first `batch` images (the same
    values the full workload holds there), for bounded CPU samples."""
    wl = WORKLOADS[name]
    s = 1000 * wl.index
    x = draw(wl.x_dist, wl.x_shape, s + 0)
    w = draw(wl.w_dist, wl.w_shape, s + 1)
    b = None if wl.b_dist is None else draw(wl.b_dist, (wl.w_shape[0],), s + 2)
    dy = draw(wl.dy_dist, wl.dy_shape, s + 3)
    if batch is not None:
        x, dy = x[:batch].copy(), dy[:batch].copy()
    return {"x": x, "w": w, "b": b, "dy": dy}
