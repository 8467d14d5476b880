"""Helpers for the GPU parity tests: upload, run all four ops through the
C-ABI binding, and compare with the oracle under the fp32 tolerance
|gpu - oracle| <= 1e-5 * A_e + 1e-6 (A_e = sum of |products| of the element)."""
from __future__ import annotations

import sys

import numpy as np

RTOL = 1e-5
ATOL = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def gpu_all_ops(x, w, b, dy, stride, padding, dilation, groups, layout="nchw"):
    """Run fwd, bwd_data, bwd_filter, bwd_bias on the GPU; return torch tensors.
    x and dy are NCHW arrays; with layout="nhwc" they are stored channels-last
    for the GPU, and y and dx are returned moved back to NCHW for comparison."""
    import torch
    import grouped_convolution_amd as G
    nhwc = layout == "nhwc"
    store = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 3, 1))) if nhwc else (lambda a: a)
    xd, wd, dyd = dev(store(x)), dev(w), dev(store(dy))
    bd = None if b is None else dev(b)
    kw = dict(stride=stride, padding=padding, dilation=dilation, groups=groups, layout=layout)
    y = G.gconv_fwd(xd, wd, bd, **kw)
    dx = G.gconv_bwd_data(dyd, wd, store(x).shape, **kw)
    dw = G.gconv_bwd_filter(xd, dyd, w.shape, **kw)
    db = G.gconv_bwd_bias(dyd, layout=layout)
    torch.cuda.synchronize()
    if nhwc:
        y, dx = y.permute(0, 3, 1, 2).contiguous(), dx.permute(0, 3, 1, 2).contiguous()
    return y, dx, dw, db


def check(name, got, val, mag, rtol=RTOL, atol=ATOL):
    """Element-wise tolerance check; raises AssertionError naming the worst element."""
    got = np.asarray(got, dtype=np.float64).ravel()
    val = np.asarray(val, dtype=np.float64).ravel()
    mag = np.asarray(mag, dtype=np.float64).ravel()
    assert got.shape == val.shape, (name, got.shape, val.shape)
    if got.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), "%s: non-finite GPU output" % name
    err = np.abs(got - val)
    bound = rtol * mag + atol
    ratio = err / bound
    worst = int(np.argmax(ratio))
    assert ratio[worst] <= 1.0, ("%s: element %d gpu=%r oracle=%r A=%r err=%.3e bound=%.3e"
                                 % (name, worst, got[worst], val[worst], mag[worst], err[worst],
                                    bound[worst]))
    return float(ratio[worst])


def sample_indices(total, count, seed):
    """`count` distinct flat indices in [0, total), always including both ends."""
    rng = np.random.default_rng(seed)
    if total <= count:
        return np.arange(total, dtype=np.int64)
    idx = rng.choice(total, size=count - 2, replace=False)
    return np.unique(np.concatenate([idx, [0, total - 1]]).astype(np.int64))


def gather(t, idx):
    import torch
    return t.reshape(-1)[torch.from_numpy(idx).to(t.device)].cpu().numpy()
