"""Descriptor cases shared by the oracle pins and the GPU parity tests.

Only shapes and seeds live here; no convolution arithmetic.
"""
from __future__ import annotations

import numpy as np

from grouped_convolution_amd.workloads import draw


def fits(H, W, kh, kw, sh, sw, ph, pw, dh, dw):
    """True when the dilated kernel fits the padded input on both axes."""
    return H + 2 * ph >= dh * (kh - 1) + 1 and W + 2 * pw >= dw * (kw - 1) + 1


def random_descs(seed, count, max_hw=9, max_k=4, max_cg=3, max_kg=3, max_g=3, max_n=3,
                 strides=(1, 2, 3), pads=(0, 1, 2), dils=(1, 2)):
    """`count` random valid descriptors as dicts (square and non-square)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        G = int(rng.integers(1, max_g + 1))
        d = dict(N=int(rng.integers(1, max_n + 1)),
                 C=G * int(rng.integers(1, max_cg + 1)),
                 K=G * int(rng.integers(1, max_kg + 1)),
                 H=int(rng.integers(1, max_hw + 1)), W=int(rng.integers(1, max_hw + 1)),
                 kh=int(rng.integers(1, max_k + 1)), kw=int(rng.integers(1, max_k + 1)),
                 sh=int(rng.choice(strides)), sw=int(rng.choice(strides)),
                 ph=int(rng.choice(pads)), pw=int(rng.choice(pads)),
                 dh=int(rng.choice(dils)), dw=int(rng.choice(dils)), G=G)
        if fits(d["H"], d["W"], d["kh"], d["kw"], d["sh"], d["sw"], d["ph"], d["pw"],
                d["dh"], d["dw"]):
            out.append(d)
    return out


def asym_descs(seed, count, max_pad=3, **kw):
    """Random descriptors whose end padding (keys pb, pr: rows below, columns right)
    differs from the start padding (ph, pw) on at least one axis."""
    rng = np.random.default_rng(seed)
    out = []
    for d in random_descs(seed, 4 * count, **kw):
        d["pb"], d["pr"] = int(rng.integers(0, max_pad + 1)), int(rng.integers(0, max_pad + 1))
        if (d["pb"], d["pr"]) == (d["ph"], d["pw"]):
            continue
        if (d["H"] + d["ph"] + d["pb"] >= d["dh"] * (d["kh"] - 1) + 1 and
                d["W"] + d["pw"] + d["pr"] >= d["dw"] * (d["kw"] - 1) + 1):
            out.append(d)
        if len(out) == count:
            break
    return out


def conv_kwargs(d):
    """stride/padding/dilation/groups keywords; padding is (top, bottom, left, right)
    when the descriptor carries end padding."""
    pad = (d["ph"], d["pb"], d["pw"], d["pr"]) if "pb" in d else (d["ph"], d["pw"])
    return dict(stride=(d["sh"], d["sw"]), padding=pad,
                dilation=(d["dh"], d["dw"]), groups=d["G"])


def tensors(d, seed, dist=("normal", 1.0), bias=True):
    """x, w, b for descriptor `d` drawn from `dist` (seeds seed+0..2)."""
    x = draw(dist, (d["N"], d["C"], d["H"], d["W"]), seed)
    w = draw(dist, (d["K"], d["C"] // d["G"], d["kh"], d["kw"]), seed + 1)
    b = draw(dist, (d["K"],), seed + 2) if bias else None
    return x, w, b
