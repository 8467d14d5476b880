"""Randomized parity sweep on the GPU: many seeded descriptors per kernel
family, each op on the dispatcher's choice in NCHW and channels-last, with
normal and small-integer data, then each family forced in turn with the ReLU
epilogue, every element against the CPU oracle.

The families cover the reach of every specialised kernel (small groups with
bands and walks up to 64-wide rows, depthwise layers with multipliers,
MFMA-sized groups, 1x1 layers, kernel == input, tall and wide planes that
span several bands and tiles, and small arbitrary descriptors with stride,
dilation and asymmetric padding). Bar as elsewhere: |gpu - oracle| <=
1e-5 * A_e + 1e-6 per element, bit for bit on integer data (its sums stay
far below 2^24). Failures are collected per family and reported together.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from cases import asym_descs, conv_kwargs, random_descs, tensors
from gpu_util import check, dev, gpu_all_ops, say
from grouped_convolution_amd.workloads import draw

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import grouped_convolution_amd as G  # noqa: E402

OPS = ("fwd", "bwd_data", "bwd_filter", "bwd_bias")
UNSUPPORTED = 6  # GCONV_ERR_UNSUPPORTED: a forced family that does not cover the layer
PER_FAMILY = 24


def _sym_or_end_pad(rng, d, kmax):
    """One layer in four gets end padding of its own (rows below, columns right)."""
    if rng.random() < 0.25:
        d["pb"], d["pr"] = int(rng.integers(0, kmax)), int(rng.integers(0, kmax))
    return d


def _fits_padded(d):
    pb, pr = d.get("pb", d["ph"]), d.get("pr", d["pw"])
    return (d["H"] + d["ph"] + pb >= (d["kh"] - 1) * d["dh"] + 1 and
            d["W"] + d["pw"] + pr >= (d["kw"] - 1) * d["dw"] + 1)


def smallgroup_family(rng):
    G_ = int(rng.integers(1, 17))
    d = dict(N=int(rng.integers(1, 4)), C=G_ * int(rng.choice([1, 2, 3, 4, 4, 8])),
             K=G_ * int(rng.integers(1, 9)), H=int(rng.integers(3, 61)), W=int(rng.integers(3, 65)),
             kh=3, kw=3, sh=int(rng.choice([1, 1, 2])), ph=int(rng.integers(0, 3)),
             pw=int(rng.integers(0, 3)), dh=int(rng.choice([1, 1, 1, 2])), G=G_)
    d["sw"] = d["sh"] if rng.random() < 0.8 else int(rng.choice([1, 2]))
    d["dw"] = d["dh"] if rng.random() < 0.8 else int(rng.choice([1, 2]))
    return _sym_or_end_pad(rng, d, 3)


def depthwise_family(rng):
    k = int(rng.choice([3, 3, 3, 5]))
    C = int(rng.integers(1, 25))
    d = dict(N=int(rng.integers(1, 4)), C=C, K=C * int(rng.choice([1, 1, 2, 3])),
             H=int(rng.integers(k, 65)), W=int(rng.integers(k, 65)), kh=k, kw=k,
             sh=int(rng.choice([1, 1, 2])), ph=int(rng.integers(0, k)), pw=int(rng.integers(0, k)),
             dh=int(rng.choice([1, 1, 1, 2])), G=C)
    d["sw"], d["dw"] = d["sh"], d["dh"]
    return _sym_or_end_pad(rng, d, k)


def mfma_family(rng):
    k = int(rng.choice([3, 5]))
    G_ = int(rng.choice([1, 2, 3]))
    return dict(N=int(rng.integers(1, 4)), C=G_ * int(rng.integers(1, 70)), K=G_ * int(rng.integers(1, 100)),
                H=int(rng.integers(k, 34)), W=int(rng.integers(k, 34)), kh=k, kw=k,
                sh=int(rng.choice([1, 1, 2])), sw=int(rng.choice([1, 1, 2])), ph=int(rng.integers(0, k)),
                pw=int(rng.integers(0, k)), dh=int(rng.choice([1, 1, 2])), dw=int(rng.choice([1, 1, 2])), G=G_)


def pointwise_family(rng):
    G_ = int(rng.choice([1, 1, 2, 4]))
    return dict(N=int(rng.integers(1, 4)), C=G_ * int(rng.integers(1, 150)), K=G_ * int(rng.integers(1, 150)),
                H=int(rng.integers(1, 40)), W=int(rng.integers(1, 40)), kh=1, kw=1, sh=1, sw=1, ph=0, pw=0,
                dh=1, dw=1, G=G_)


def fc_family(rng):
    G_ = int(rng.choice([1, 1, 2, 4]))
    H, W = int(rng.integers(1, 9)), int(rng.integers(1, 9))
    return dict(N=int(rng.integers(1, 70)), C=G_ * int(rng.integers(1, 40)), K=G_ * int(rng.integers(1, 150)),
                H=H, W=W, kh=H, kw=W, sh=int(rng.choice([1, 2])), sw=int(rng.choice([1, 2])), ph=0, pw=0,
                dh=1, dw=1, G=G_)


def tall_wide_family(rng):
    k = int(rng.choice([1, 3, 3, 5]))
    G_ = int(rng.choice([1, 2, 4, 8, 16, 32]))
    d = dict(N=int(rng.integers(1, 3)), C=G_ * int(rng.choice([1, 2, 4, 8, 16])),
             K=G_ * int(rng.choice([1, 2, 4, 8, 16])), H=int(rng.integers(k, 121)), W=int(rng.integers(k, 121)),
             kh=k, kw=k, sh=int(rng.choice([1, 1, 2])), ph=int(rng.integers(0, k)), pw=int(rng.integers(0, k)),
             dh=1, dw=1, G=G_)
    d["sw"] = d["sh"]
    return d if d["N"] * d["C"] * d["H"] * d["W"] <= 3_000_000 else None


FAMILIES = {
    "smallgroup": smallgroup_family, "depthwise": depthwise_family, "mfma": mfma_family,
    "pointwise": pointwise_family, "fc": fc_family, "tall_wide": tall_wide_family,
}


def family_descs(name, seed, count):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        d = FAMILIES[name](rng)
        if d is not None and _fits_padded(d):
            out.append(d)
    return out


def _oracle(x, w, b, dy, kw, relu=False):
    return (oracle.fwd(x, w, b, relu=relu, **kw), oracle.bwd_data(dy, w, x.shape, **kw),
            oracle.bwd_filter(x, dy, w.shape, **kw), oracle.bwd_bias(dy))


def _sweep(descs, seed0):
    """All checks over `descs`; returns the list of failure messages."""
    fails = []
    for i, d in enumerate(descs):
        kw = conv_kwargs(d)
        say("soak %d %s" % (i, d))
        for layout in ("nchw", "nhwc"):
            for dist in (("normal", 1.0), ("int", -3, 3)):
                x, w, b = tensors(d, seed0 + 10 * i, dist=dist)
                y_ref, _ = oracle.fwd(x, w, b, **kw)
                dy = draw(dist, y_ref.shape, seed0 + 10 * i + 5)
                ref = _oracle(x, w, b, dy, kw)
                got = gpu_all_ops(x, w, b, dy, kw["stride"], kw["padding"], kw["dilation"], kw["groups"],
                                  layout=layout)
                for op, g, (val, mag) in zip(OPS, got, ref):
                    g = g.cpu().numpy()
                    try:
                        assert g.shape == val.shape, (g.shape, val.shape)
                        if dist[0] == "int":
                            assert np.array_equal(g.astype(np.float64), val), "integer data not exact"
                        else:
                            check(op, g, val, mag)
                    except AssertionError as e:
                        fails.append("%s %s %s %s: %s" % (layout, dist[0], op, d, str(e)[:300]))
        # every family forced in turn, NCHW, normal data, ReLU on the forward
        x, w, b = tensors(d, seed0 + 10 * i + 7)
        y_ref, _ = oracle.fwd(x, w, b, **kw)
        dy = draw(("normal", 1.0), y_ref.shape, seed0 + 10 * i + 8)
        ref = _oracle(x, w, b, dy, kw, relu=True)
        xd, wd, dyd, bd = dev(x), dev(w), dev(dy), dev(b)
        calls = {"fwd": lambda: G.gconv_fwd(xd, wd, bd, relu=True, **kw),
                 "bwd_data": lambda: G.gconv_bwd_data(dyd, wd, x.shape, **kw),
                 "bwd_filter": lambda: G.gconv_bwd_filter(xd, dyd, w.shape, **kw),
                 "bwd_bias": lambda: G.gconv_bwd_bias(dyd)}
        for path in (G.PATH_DIRECT, G.PATH_SMALLGROUP, G.PATH_IGEMM, G.PATH_FC, G.PATH_POINTWISE):
            G.gconv_set_path_override(path)
            try:
                for op, (val, mag) in zip(OPS, ref):
                    try:
                        g = calls[op]()
                    except G.GconvError as e:
                        if e.status == UNSUPPORTED:
                            continue
                        raise
                    torch.cuda.synchronize()
                    try:
                        check(op, g.cpu().numpy(), val, mag)
                    except AssertionError as e:
                        fails.append("forced %s %s %s: %s" % (G.PATH_NAMES[path], op, d, str(e)[:300]))
            finally:
                G.gconv_set_path_override(G.PATH_AUTO)
    return fails


@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_randomized_sweep(family):
    seed = 20000 + 1000 * sorted(FAMILIES).index(family)
    descs = family_descs(family, seed, PER_FAMILY)
    fails = _sweep(descs, seed)
    assert not fails, "%d failures, first: %s" % (len(fails), "\n".join(fails[:5]))


def test_randomized_sweep_small_arbitrary():
    """Small descriptors of any shape (non-square kernels, strides up to 3,
    dilation, end padding of their own)."""
    descs = (random_descs(27000, PER_FAMILY, max_hw=20, max_k=5, max_cg=8, max_kg=8, max_g=4) +
             asym_descs(27001, PER_FAMILY // 4, max_hw=16, max_k=5, max_cg=6, max_kg=6, max_g=4))
    fails = _sweep(descs, 27000)
    assert not fails, "%d failures, first: %s" % (len(fails), "\n".join(fails[:5]))
