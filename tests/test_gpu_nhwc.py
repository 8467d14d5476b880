"""GPU parity of the channels-last (NHWC) layout against the CPU oracle.

The oracle computes in NCHW; here the NHWC activations are the same values
with the channel axis last, so the reference is the oracle's result moved to
that layout (a numpy transpose of test data, no arithmetic). Bar as for NCHW:
|gpu - oracle| <= 1e-5 * A_e + 1e-6 per element, exact for integer data.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from cases import asym_descs, conv_kwargs, random_descs, tensors
from gpu_util import check, dev, say
from grouped_convolution_amd.workloads import draw

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import grouped_convolution_amd as G  # noqa: E402

OPS = ("fwd", "bwd_data", "bwd_filter", "bwd_bias")


def to_nhwc(a):
    return np.ascontiguousarray(a.transpose(0, 2, 3, 1))


@pytest.fixture(autouse=True)
def _auto_path():
    G.gconv_set_path_override(G.PATH_AUTO)
    yield
    G.gconv_set_path_override(G.PATH_AUTO)


def refs(x, w, b, dy, kw):
    """Oracle (value, A_e) per op, with activations moved to NHWC."""
    y, ya = oracle.fwd(x, w, b, **kw)
    dx, dxa = oracle.bwd_data(dy, w, x.shape, **kw)
    return {"fwd": (to_nhwc(y), to_nhwc(ya)), "bwd_data": (to_nhwc(dx), to_nhwc(dxa)),
            "bwd_filter": oracle.bwd_filter(x, dy, w.shape, **kw), "bwd_bias": oracle.bwd_bias(dy)}


def gpu_nhwc(x, w, b, dy, kw):
    """The four ops on NHWC copies of x and dy (NCHW numpy inputs)."""
    xd, wd, dyd = dev(to_nhwc(x)), dev(w), dev(to_nhwc(dy))
    bd = None if b is None else dev(b)
    out = {}
    for op, fn in (("fwd", lambda: G.gconv_fwd(xd, wd, bd, layout="nhwc", **kw)),
                   ("bwd_data", lambda: G.gconv_bwd_data(dyd, wd, to_nhwc(x).shape, layout="nhwc", **kw)),
                   ("bwd_filter", lambda: G.gconv_bwd_filter(xd, dyd, w.shape, layout="nhwc", **kw)),
                   ("bwd_bias", lambda: G.gconv_bwd_bias(dyd, layout="nhwc"))):
        try:
            out[op] = fn()
        except G.GconvError as e:
            if "GCONV_ERR_UNSUPPORTED" not in str(e):
                raise
            out[op] = None
    torch.cuda.synchronize()
    return out


def compare(tag, got, ref):
    done = []
    for op in OPS:
        if got[op] is None:
            continue
        val, mag = ref[op]
        assert tuple(got[op].shape) == val.shape, (tag, op, tuple(got[op].shape), val.shape)
        check("%s %s" % (tag, op), got[op].cpu().numpy(), val, mag)
        done.append(op)
    return done


@pytest.mark.parametrize("seed", range(2))
def test_nhwc_random_descriptors_every_family(seed):
    """Random descriptors (strides, pads, dilation, groups) in NHWC on the
    dispatcher's choice and on each forced family."""
    for d in random_descs(3100 + seed, 12, max_hw=12, max_k=5, max_cg=6, max_kg=6, max_g=4):
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 3200 + seed)
        y_ref, _ = oracle.fwd(x, w, b, **kw)
        dy = draw(("normal", 1.0), y_ref.shape, 3300 + seed)
        ref = refs(x, w, b, dy, kw)
        covered = set()
        for path in (G.PATH_AUTO, G.PATH_DIRECT, G.PATH_SMALLGROUP, G.PATH_IGEMM):
            say("nhwc desc %s path %s" % (d, G.PATH_NAMES[path]))
            G.gconv_set_path_override(path)
            try:
                covered |= set(compare("nhwc %s %s" % (G.PATH_NAMES[path], d), gpu_nhwc(x, w, b, dy, kw), ref))
            finally:
                G.gconv_set_path_override(G.PATH_AUTO)
        assert covered == set(OPS)


def test_nhwc_asymmetric_padding():
    """End padding that differs from the start padding, in NHWC, on the
    dispatcher's choice, with ReLU fused into the forward pass."""
    for d in asym_descs(3700, 10, max_hw=12, max_k=5, max_cg=6, max_kg=6, max_g=4):
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 3710)
        y_ref, ya = oracle.fwd(x, w, b, relu=True, **kw)
        dy = draw(("normal", 1.0), y_ref.shape, 3720)
        say("nhwc asym %s" % d)
        ref = refs(x, w, b, dy, kw)
        ref["fwd"] = (to_nhwc(y_ref), to_nhwc(ya))
        got = gpu_nhwc(x, w, b, dy, kw)
        got["fwd"] = G.gconv_fwd(dev(to_nhwc(x)), dev(w), dev(b), layout="nhwc", relu=True, **kw)
        assert compare("nhwc asym %s" % d, got, ref) == list(OPS)


NHWC_CASES = [
    # dense 3x3 (MFMA implicit GEMM between the reorderings), several 64-wide tiles
    # of pixels and channels with ragged tails
    (dict(N=3, C=70, K=66, H=13, W=11, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=1),
     {"fwd": "igemm", "bwd_data": "igemm", "bwd_filter": "igemm", "bwd_bias": "direct"}),
    # channel counts in whole quads: the flat MFMA kernel reads the NHWC input itself
    # (16-byte DMA per pixel) and stores NHWC; two groups at stride 2 (gradInput reads
    # dy as if upsampled) ...
    (dict(N=2, C=64, K=96, H=15, W=17, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=2),
     {"fwd": "igemm", "bwd_data": "igemm"}),
    # ... and 5x5 with tiles spanning two images
    (dict(N=3, C=16, K=32, H=9, W=11, kh=5, kw=5, sh=1, sw=1, ph=2, pw=2, dh=1, dw=1, G=1),
     {"fwd": "igemm", "bwd_data": "igemm", "bwd_filter": "igemm"}),
    # ResNeXt-style 4 per group and depthwise stride 2 (small-group family)
    (dict(N=2, C=32, K=32, H=14, W=15, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=8),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    (dict(N=2, C=12, K=12, H=17, W=16, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=12),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # depthwise forward and gradInput on the native NHWC kernel (no reordering):
    # 10 channels (one per thread, no 16-byte loads), 3x3 ...
    (dict(N=2, C=10, K=10, H=13, W=11, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=10),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # ... four channels per thread at unit stride: each thread slides a window along four
    # outputs of a row (13 columns: the last block holds one), 3x3 and 5x5 ...
    (dict(N=2, C=12, K=12, H=9, W=13, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=12),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    (dict(N=3, C=8, K=8, H=11, W=10, kh=5, kw=5, sh=1, sw=1, ph=2, pw=0, dh=1, dw=1, G=8),
     {"fwd": "smallgroup", "bwd_data": "smallgroup"}),
    # ... 16 channels (four per thread) 5x5 at stride 2 (gradInput keeps only the exact quotients) ...
    (dict(N=2, C=16, K=16, H=17, W=16, kh=5, kw=5, sh=2, sw=2, ph=2, pw=2, dh=1, dw=1, G=16),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "direct"}),
    # ... dilation 2 ...
    (dict(N=1, C=8, K=8, H=15, W=14, kh=3, kw=3, sh=1, sw=1, ph=2, pw=2, dh=2, dw=2, G=8),
     {"fwd": "smallgroup", "bwd_data": "smallgroup"}),
    # ... and one more zero row and column at the end than at the start, at stride 2
    (dict(N=2, C=24, K=24, H=16, W=15, kh=3, kw=3, sh=2, sw=2, dh=1, dw=1, G=24, ph=0, pb=1, pw=0, pr=1),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # 1x1, one group: one GEMM over the N*H*W pixel rows (fully-connected path)
    (dict(N=3, C=40, K=72, H=9, W=10, kh=1, kw=1, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1),
     {"fwd": "fc", "bwd_data": "fc", "bwd_filter": "fc"}),
    # 1x1 with two groups: reordered around the pointwise GEMMs
    (dict(N=2, C=32, K=48, H=7, W=9, kh=1, kw=1, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=2),
     {"fwd": "pointwise", "bwd_data": "pointwise", "bwd_filter": "pointwise"}),
    # kernel == input (fully-connected mode) in NHWC
    (dict(N=5, C=8, K=20, H=4, W=3, kh=4, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1),
     {"fwd": "fc", "bwd_data": "fc", "bwd_filter": "fc"}),
]


@pytest.mark.parametrize("case", range(len(NHWC_CASES)))
def test_nhwc_cases(case):
    """NHWC on the dispatcher's own family (asserted): normal data to the
    tolerance, integer data bit for bit."""
    d, paths = NHWC_CASES[case]
    kw = conv_kwargs(d)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], layout="nhwc", **kw)
    for op, name in paths.items():
        chosen = G.gconv_select_path(desc, getattr(G, "OP_" + op.upper()))
        assert G.PATH_NAMES[chosen] == name, (d, op, G.PATH_NAMES[chosen])
    if d["G"] == d["C"] == d["K"] and d["kh"] in (3, 5):
        # the native depthwise kernel: no reordering, no workspace
        assert G.gconv_workspace_size(desc, G.OP_FWD) == 0 and G.gconv_workspace_size(desc, G.OP_BWD_DATA) == 0
    say("nhwc case %s" % d)
    x, w, b = tensors(d, 3400 + case)
    y_ref, _ = oracle.fwd(x, w, b, **kw)
    dy = draw(("normal", 1.0), y_ref.shape, 3410 + case)
    assert compare("nhwc %s" % d, gpu_nhwc(x, w, b, dy, kw), refs(x, w, b, dy, kw)) == list(OPS)
    xi, wi, bi = tensors(d, 3500 + case, dist=("int", -3, 3))
    dyi = draw(("int", -3, 3), y_ref.shape, 3510 + case)
    got = gpu_nhwc(xi, wi, bi, dyi, kw)
    ref = refs(xi, wi, bi, dyi, kw)
    for op in OPS:
        assert np.array_equal(got[op].cpu().numpy().astype(np.float64), ref[op][0]), (d, op)


# Depthwise 3x3 at unit stride, four channels a lane, on the row-walking kernel:
# a wave owns 64 (channel quad, four-column run) units of a row and walks a band
# of rows. The band height follows from the problem size (about 2048 waves in
# all), so these shapes are large enough for bands of several rows, a ragged
# last band and a ragged last strip of units.
WALK_CASES = [
    # 62 quads x 14 runs = 868 units (14 strips, the last 36 lanes); bands of 3
    # rows, the last of 1; bias and ReLU
    (dict(N=8, C=248, K=248, H=40, W=54, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=248), True),
    # no padding: 70 columns (the last run of 2), 288 units in 5 strips, bands of 2 rows
    (dict(N=16, C=64, K=64, H=30, W=72, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=64), False),
    # two zero rows at the end and none at the start, two zero columns at the
    # start and none at the end; bands of 3 rows
    (dict(N=32, C=128, K=128, H=33, W=40, kh=3, kw=3, sh=1, sw=1, dh=1, dw=1, G=128,
          ph=0, pb=2, pw=2, pr=0), True),
]


@pytest.mark.parametrize("case", range(len(WALK_CASES)))
def test_nhwc_depthwise_walk(case):
    """Channels-last depthwise forward (bias, optional ReLU), gradInput and
    gradWeight on the row-walking kernels against the oracle; integer data bit
    for bit."""
    d, relu = WALK_CASES[case]
    kw = conv_kwargs(d)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], layout="nhwc", **kw)
    for op in ("fwd", "bwd_data"):
        assert G.PATH_NAMES[G.gconv_select_path(desc, getattr(G, "OP_" + op.upper()))] == "smallgroup"
        assert G.gconv_workspace_size(desc, getattr(G, "OP_" + op.upper())) == 0
    for dist, seed in ((("normal", 1.0), 3800), (("int", -3, 3), 3850)):
        say("nhwc depthwise walk %s relu %s %s" % (d, relu, dist[0]))
        x, w, b = tensors(d, seed + 10 * case, dist=dist)
        y_ref, ya = oracle.fwd(x, w, b, relu=relu, **kw)
        dy = draw(dist, y_ref.shape, seed + 10 * case + 5)
        dx_ref, dxa = oracle.bwd_data(dy, w, x.shape, **kw)
        dw_ref, dwa = oracle.bwd_filter(x, dy, w.shape, **kw)
        y = G.gconv_fwd(dev(to_nhwc(x)), dev(w), dev(b), layout="nhwc", relu=relu, **kw)
        dx = G.gconv_bwd_data(dev(to_nhwc(dy)), dev(w), to_nhwc(x).shape, layout="nhwc", **kw)
        dwg = G.gconv_bwd_filter(dev(to_nhwc(x)), dev(to_nhwc(dy)), w.shape, layout="nhwc", **kw)
        torch.cuda.synchronize()
        for tag, got, val, mag in (("fwd", y, to_nhwc(y_ref), to_nhwc(ya)), ("bwd_data", dx, to_nhwc(dx_ref), to_nhwc(dxa)),
                                   ("bwd_filter", dwg, dw_ref, dwa)):
            g = got.cpu().numpy()
            assert g.shape == val.shape, (d, tag)
            if dist[0] == "int":
                assert np.array_equal(g.astype(np.float64), val), (d, tag)
            else:
                check("walk %s %s" % (tag, d), g, val, mag)


def test_nhwc_workspace_guard_bands():
    """The staged ops write only their outputs and their workspace: guard
    floats around every output and around the workspace stay untouched."""
    d = dict(N=2, C=24, K=40, H=9, W=8, kh=3, kw=3, sh=2, sw=1, ph=1, pw=0, dh=1, dw=2, G=2)
    kw = conv_kwargs(d)
    x, w, b = tensors(d, 3600)
    y_ref, _ = oracle.fwd(x, w, b, **kw)
    dy = draw(("normal", 1.0), y_ref.shape, 3610)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], layout="nhwc", **kw)
    sentinel = 12345.0
    for op, name in ((G.OP_FWD, "fwd"), (G.OP_BWD_DATA, "bwd_data"), (G.OP_BWD_FILTER, "bwd_filter")):
        nws = G.gconv_workspace_size(desc, op)
        assert nws > 0
        pad = 64
        buf = torch.full((pad + nws // 4 + pad,), sentinel, device="cuda")
        ws = buf[pad:pad + nws // 4]
        ref = refs(x, w, b, dy, kw)[name]
        shape = ref[0].shape
        obuf = torch.full((pad + int(np.prod(shape)) + pad,), sentinel, device="cuda")
        out = obuf[pad:pad + int(np.prod(shape))].view(*shape)
        xd, wd, dyd = dev(to_nhwc(x)), dev(w), dev(to_nhwc(dy))
        if name == "fwd":
            G.gconv_fwd(xd, wd, dev(b), layout="nhwc", out=out, workspace=ws, **kw)
        elif name == "bwd_data":
            G.gconv_bwd_data(dyd, wd, to_nhwc(x).shape, layout="nhwc", out=out, workspace=ws, **kw)
        else:
            G.gconv_bwd_filter(xd, dyd, w.shape, layout="nhwc", out=out, workspace=ws, **kw)
        torch.cuda.synchronize()
        check("guarded nhwc %s" % name, out.cpu().numpy(), ref[0], ref[1])
        for t in (buf, obuf):
            h = t.cpu().numpy()
            assert np.all(h[:pad] == sentinel) and np.all(h[-pad:] == sentinel), name


@pytest.mark.parametrize("stride", [1, 2])
def test_nhwc_depthwise_wgrad_misaligned(stride):
    """Channels-last depthwise gradWeight on x and dy that start one float into
    their allocations (not 16-byte aligned): the native kernel takes 4-byte
    loads and agrees with the oracle, with normal data to the tolerance and
    integer data bit for bit; the workspace is the aligned call's."""
    d = dict(N=3, C=12, K=12, H=11, W=13, kh=3, kw=3, sh=stride, sw=stride, ph=1, pw=1, dh=1, dw=1, G=12)
    kw = conv_kwargs(d)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], 3, 3, layout="nhwc", **kw)
    nws = G.gconv_workspace_size(desc, G.OP_BWD_FILTER)
    for dist, seed in ((("normal", 1.0), 3700), (("int", -3, 3), 3800)):
        x, w, _ = tensors(d, seed + stride, dist=dist, bias=False)
        y_ref, _ = oracle.fwd(x, w, None, **kw)
        dy = draw(dist, y_ref.shape, seed + 10 + stride)
        say("misaligned nhwc depthwise gradWeight stride %d %s" % (stride, dist[0]))

        def offset_view(a):
            flat = torch.zeros(a.size + 1, device="cuda")
            v = flat[1:].view(*a.shape)
            v.copy_(torch.from_numpy(np.ascontiguousarray(a)))
            assert v.data_ptr() % 16 != 0
            return v

        xd, dyd = offset_view(to_nhwc(x)), offset_view(to_nhwc(dy))
        ws = torch.empty(max(nws // 4, 1), device="cuda")
        dw = G.gconv_bwd_filter(xd, dyd, w.shape, layout="nhwc", workspace=ws, **kw)
        torch.cuda.synchronize()
        val, mag = oracle.bwd_filter(x, dy, w.shape, **kw)
        if dist[0] == "int":
            assert np.array_equal(dw.cpu().numpy().astype(np.float64), val)
        else:
            check("misaligned dw", dw.cpu().numpy(), val, mag)


NHWC_WGRAD_CASES = [
    dict(N=3, C=64, K=64, H=20, W=22, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=1),    # 32 x 64 tiles, 8 waves
    dict(N=2, C=32, K=48, H=17, W=31, kh=3, kw=3, sh=1, sw=1, ph=0, pw=1, dh=1, dw=1, G=2),    # 16 x 24 per group
    dict(N=2, C=32, K=32, H=19, W=21, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=1),    # stride 2
    dict(N=2, C=16, K=32, H=18, W=18, kh=3, kw=3, sh=1, sw=1, ph=2, pw=2, dh=2, dw=2, G=1),    # dilation 2
    dict(N=2, C=48, K=128, H=13, W=15, kh=5, kw=5, sh=1, sw=1, ph=2, pw=2, dh=1, dw=1, G=1),   # 5x5
    dict(N=2, C=32, K=32, H=15, W=63, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=1),    # wide rows
    dict(N=2, C=64, K=64, H=16, W=16, kh=3, kw=3, sh=1, sw=1, ph=0, pb=1, pw=1, pr=2, dh=1, dw=1, G=2),  # asym pads
]


@pytest.mark.parametrize("case", range(len(NHWC_WGRAD_CASES)))
def test_nhwc_mfma_gradweight(case):
    """gradWeight of channels-last x and dy on the MFMA path, read in place (quad
    planes filled by 16-byte DMA): normal data to the tolerance, integer data bit
    for bit; and the same call on tensors one float off 16-byte alignment (the
    reordering route) gives the same bits."""
    d = NHWC_WGRAD_CASES[case]
    kw = conv_kwargs(d)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], layout="nhwc", **kw)
    assert G.PATH_NAMES[G.gconv_select_path(desc, G.OP_BWD_FILTER)] == "igemm", d
    Ho, Wo = G.gconv_output_dims(desc)
    wshape = (d["K"], d["C"] // d["G"], d["kh"], d["kw"])
    for dist, seed in ((("normal", 1.0), 3950), (("int", -3, 3), 3970)):
        x = draw(dist, (d["N"], d["C"], d["H"], d["W"]), seed + case)
        dy = draw(dist, (d["N"], d["K"], Ho, Wo), seed + 10 + case)
        say("nhwc mfma gradWeight %s %s" % (d, dist[0]))
        got = G.gconv_bwd_filter(dev(to_nhwc(x)), dev(to_nhwc(dy)), wshape, layout="nhwc", **kw)

        def offset_view(a):
            flat = torch.zeros(a.size + 1, device="cuda")
            v = flat[1:].view(*a.shape)
            v.copy_(torch.from_numpy(np.ascontiguousarray(a)))
            return v

        staged = G.gconv_bwd_filter(offset_view(to_nhwc(x)), offset_view(to_nhwc(dy)), wshape, layout="nhwc", **kw)
        torch.cuda.synchronize()
        val, mag = oracle.bwd_filter(x, dy, wshape, **kw)
        g = got.cpu().numpy()
        if dist[0] == "int":
            assert np.array_equal(g.astype(np.float64), val), d
        else:
            check("nhwc mfma dw %s" % d, g, val, mag)
        check("nhwc staged dw %s" % d, staged.cpu().numpy(), val, mag)
