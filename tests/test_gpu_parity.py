"""GPU parity: the HIP path (through the C-ABI binding) against the CPU oracle.

Bar: per element |gpu - oracle| <= 1e-5 * A_e + 1e-6, where A_e is the sum of
|products| over that element's reduction (from the oracle); exact equality
for integer-valued data (all partial sums exact in fp32) and for output
shapes. Every kernel family is cross-checked by forcing it in turn.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from cases import asym_descs, conv_kwargs, fits, random_descs, tensors
from gpu_util import check, dev, gather, gpu_all_ops, sample_indices, say
from grouped_convolution_amd.workloads import WORKLOAD_ORDER, WORKLOADS, draw, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import grouped_convolution_amd as G  # noqa: E402

ALL_PATHS = [G.PATH_DIRECT, G.PATH_SMALLGROUP, G.PATH_IGEMM, G.PATH_FC, G.PATH_POINTWISE]


@pytest.fixture(autouse=True)
def _auto_path():
    G.gconv_set_path_override(G.PATH_AUTO)
    yield
    G.gconv_set_path_override(G.PATH_AUTO)


def oracle_all(x, w, b, dy, kw):
    return (oracle.fwd(x, w, b, **kw), oracle.bwd_data(dy, w, x.shape, **kw),
            oracle.bwd_filter(x, dy, w.shape, **kw), oracle.bwd_bias(dy))


OPS = ("fwd", "bwd_data", "bwd_filter", "bwd_bias")


def run_path(path, x, w, b, dy, kw):
    """Each op on one forced path: a dict op -> result tensor, or None for the
    ops that path does not cover (GCONV_ERR_UNSUPPORTED)."""
    xd, wd, dyd = dev(x), dev(w), dev(dy)
    bd = None if b is None else dev(b)
    calls = {
        "fwd": lambda: G.gconv_fwd(xd, wd, bd, **kw),
        "bwd_data": lambda: G.gconv_bwd_data(dyd, wd, x.shape, **kw),
        "bwd_filter": lambda: G.gconv_bwd_filter(xd, dyd, w.shape, **kw),
        "bwd_bias": lambda: G.gconv_bwd_bias(dyd),
    }
    out = {}
    G.gconv_set_path_override(path)
    try:
        for op in OPS:
            try:
                out[op] = calls[op]()
            except G.GconvError as e:
                if e.status != 6:  # GCONV_ERR_UNSUPPORTED: the family does not cover it
                    raise
                out[op] = None
        torch.cuda.synchronize()
    finally:
        G.gconv_set_path_override(G.PATH_AUTO)
    return out


def compare_full(tag, gpu, ref):
    """gpu: tuple of 4 tensors, or dict op -> tensor/None. Returns ops compared."""
    if not isinstance(gpu, dict):
        gpu = dict(zip(OPS, gpu))
    done = []
    for name, (val, mag) in zip(OPS, ref):
        g = gpu[name]
        if g is None:
            continue
        assert tuple(g.shape) == val.shape, (tag, name, tuple(g.shape), val.shape)
        check("%s %s" % (tag, name), g.cpu().numpy(), val, mag)
        done.append(name)
    return done


# ----------------------------------------------------------------- random descriptors

@pytest.mark.parametrize("seed", range(3))
def test_random_descriptors_every_path(seed):
    descs = random_descs(40 + seed, 24, max_hw=12, max_k=5, max_cg=6, max_kg=6, max_g=4)
    for d in descs:
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 500 + seed)
        y_ref, _ = oracle.fwd(x, w, b, **kw)
        dy = draw(("normal", 1.0), y_ref.shape, 600 + seed)
        ref = oracle_all(x, w, b, dy, kw)
        covered = set()
        for path in ALL_PATHS:
            say("desc %s path %s" % (d, G.PATH_NAMES[path]))
            covered |= set(compare_full("%s %s" % (G.PATH_NAMES[path], d),
                                        run_path(path, x, w, b, dy, kw), ref))
        assert covered == set(OPS)


def mfma_family_descs(seed, count):
    """Random descriptors inside the MFMA family's reach: 3x3 / 5x5 filters,
    channel counts that span several reduction chunks and output tiles (with
    ragged tails), stride on the forward pass, dilation, groups."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        k = int(rng.choice([3, 5]))
        G_ = int(rng.choice([1, 2, 3]))
        d = dict(N=int(rng.integers(1, 4)), C=G_ * int(rng.integers(1, 40)),
                 K=G_ * int(rng.integers(1, 80)), H=int(rng.integers(k, 30)),
                 W=int(rng.integers(k, 30)), kh=k, kw=k,
                 sh=int(rng.choice([1, 1, 2])), sw=int(rng.choice([1, 1, 2])),
                 ph=int(rng.integers(0, k)), pw=int(rng.integers(0, k)),
                 dh=int(rng.choice([1, 1, 2])), dw=int(rng.choice([1, 1, 2])), G=G_)
        if fits(d["H"], d["W"], d["kh"], d["kw"], d["sh"], d["sw"], d["ph"], d["pw"], d["dh"],
                d["dw"]):
            out.append(d)
    return out


@pytest.mark.parametrize("seed", range(3))
def test_random_descriptors_mfma_family(seed):
    covered = {op: 0 for op in OPS}
    for d in mfma_family_descs(70 + seed, 16):
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 700 + seed)
        y_ref, _ = oracle.fwd(x, w, b, **kw)
        dy = draw(("normal", 1.0), y_ref.shape, 710 + seed)
        ref = oracle_all(x, w, b, dy, kw)
        for path in [G.PATH_AUTO] + ALL_PATHS:
            say("mfma-family desc %s path %s" % (d, G.PATH_NAMES[path]))
            for op in compare_full("%s %s" % (G.PATH_NAMES[path], d),
                                   run_path(path, x, w, b, dy, kw), ref):
                if path == G.PATH_IGEMM:
                    covered[op] += 1
    # the MFMA family must actually have run forward and gradInput here
    assert covered["fwd"] >= 8 and covered["bwd_data"] >= 4, covered


@pytest.mark.parametrize("seed", range(2))
def test_random_descriptors_smallgroup_family(seed):
    """3x3 filters with a few channels per group (up to 4 in, 8 out), the reach
    of the small-group kernels: strides, dilation, padding, ragged widths."""
    rng = np.random.default_rng(120 + seed)
    covered = {op: 0 for op in OPS}
    n_done = 0
    while n_done < 12:
        G_ = int(rng.integers(1, 9))
        d = dict(N=int(rng.integers(1, 4)), C=G_ * int(rng.integers(1, 5)),
                 K=G_ * int(rng.integers(1, 9)), H=int(rng.integers(3, 40)),
                 W=int(rng.integers(3, 70)), kh=3, kw=3,
                 sh=int(rng.choice([1, 1, 2])), sw=int(rng.choice([1, 1, 2])),
                 ph=int(rng.integers(0, 3)), pw=int(rng.integers(0, 3)),
                 dh=int(rng.choice([1, 1, 2])), dw=int(rng.choice([1, 1, 2])), G=G_)
        if not fits(d["H"], d["W"], 3, 3, d["sh"], d["sw"], d["ph"], d["pw"], d["dh"], d["dw"]):
            continue
        n_done += 1
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 1200 + seed)
        y_ref, _ = oracle.fwd(x, w, b, **kw)
        dy = draw(("normal", 1.0), y_ref.shape, 1210 + seed)
        ref = oracle_all(x, w, b, dy, kw)
        for path in [G.PATH_AUTO, G.PATH_SMALLGROUP]:
            say("small-group desc %s path %s" % (d, G.PATH_NAMES[path]))
            for op in compare_full("%s %s" % (G.PATH_NAMES[path], d),
                                   run_path(path, x, w, b, dy, kw), ref):
                if path == G.PATH_SMALLGROUP:
                    covered[op] += 1
    assert covered["fwd"] >= 10 and covered["bwd_data"] >= 3 and covered["bwd_filter"] >= 3, \
        covered


@pytest.mark.parametrize("seed", range(2))
def test_fc_mode_random(seed):
    """Kernel == input (fully-connected mode), with groups and ragged M / N / R,
    through the GEMM path and every other path that covers it."""
    rng = np.random.default_rng(90 + seed)
    fc_ran = 0
    for _ in range(8):
        G_ = int(rng.choice([1, 1, 2, 3]))
        H, W = int(rng.integers(1, 7)), int(rng.integers(1, 7))
        d = dict(N=int(rng.integers(1, 300)), C=G_ * int(rng.integers(1, 40)),
                 K=G_ * int(rng.integers(1, 150)), H=H, W=W, kh=H, kw=W, sh=1, sw=1,
                 ph=0, pw=0, dh=1, dw=1, G=G_)
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 900 + seed)
        dy = draw(("normal", 1.0), (d["N"], d["K"], 1, 1), 910 + seed)
        ref = oracle_all(x, w, b, dy, kw)
        for path in [G.PATH_AUTO, G.PATH_FC, G.PATH_DIRECT]:
            say("fc desc %s path %s" % (d, G.PATH_NAMES[path]))
            done = compare_full("%s %s" % (G.PATH_NAMES[path], d), run_path(path, x, w, b, dy, kw),
                                ref)
            if path == G.PATH_FC:
                fc_ran += len(done) >= 3
    assert fc_ran == 8


@pytest.mark.parametrize("seed", range(2))
def test_random_descriptors_depthwise_family(seed):
    """Depthwise layers (groups = input channels, channel multiplier 1-3): 3x3
    and 5x5 filters, strides 1 and 2, dilation, padding, ragged sizes, on the
    dispatcher's choice and on the small-group and direct families."""
    rng = np.random.default_rng(170 + seed)
    covered = {op: 0 for op in OPS}
    n_done = 0
    while n_done < 8:
        k = int(rng.choice([3, 3, 5]))
        C = int(rng.integers(1, 10))
        d = dict(N=int(rng.integers(1, 4)), C=C, K=C * int(rng.integers(1, 4)),
                 H=int(rng.integers(k, 40)), W=int(rng.integers(k, 62)), kh=k, kw=k,
                 sh=int(rng.choice([1, 1, 2])), sw=int(rng.choice([1, 1, 2])),
                 ph=int(rng.integers(0, k)), pw=int(rng.integers(0, k // 2 + 1)),
                 dh=int(rng.choice([1, 1, 2])), dw=int(rng.choice([1, 1, 2])), G=C)
        if not fits(d["H"], d["W"], k, k, d["sh"], d["sw"], d["ph"], d["pw"], d["dh"], d["dw"]):
            continue
        n_done += 1
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 1700 + 10 * seed + n_done)
        y_ref, _ = oracle.fwd(x, w, b, **kw)
        dy = draw(("normal", 1.0), y_ref.shape, 1750 + 10 * seed + n_done)
        ref = oracle_all(x, w, b, dy, kw)
        for path in [G.PATH_AUTO, G.PATH_SMALLGROUP, G.PATH_DIRECT]:
            say("depthwise desc %s path %s" % (d, G.PATH_NAMES[path]))
            for op in compare_full("%s %s" % (G.PATH_NAMES[path], d),
                                   run_path(path, x, w, b, dy, kw), ref):
                if path == G.PATH_SMALLGROUP:
                    covered[op] += 1
    assert covered["fwd"] >= 6, covered


@pytest.mark.parametrize("seed", range(2))
def test_random_descriptors_pointwise_family(seed):
    """1x1 filters at stride 1 without padding, the pointwise GEMM path: planes
    of any size (not a multiple of 4 or of the 128-wide tile), channel counts
    on both sides of the tile edges, groups, and gradWeight reductions split
    over several slices or not at all."""
    rng = np.random.default_rng(160 + seed)
    pw_ran = 0
    for _ in range(6):
        G_ = int(rng.choice([1, 1, 2, 3]))
        d = dict(N=int(rng.integers(1, 5)), C=G_ * int(rng.integers(1, 150)),
                 K=G_ * int(rng.integers(1, 150)), H=int(rng.integers(2, 24)),
                 W=int(rng.integers(1, 24)), kh=1, kw=1, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1,
                 G=G_)
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 1600 + seed)
        dy = draw(("normal", 1.0), (d["N"], d["K"], d["H"], d["W"]), 1610 + seed)
        ref = oracle_all(x, w, b, dy, kw)
        desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], 1, 1, groups=G_)
        assert G.gconv_select_path(desc, G.OP_FWD) == G.PATH_POINTWISE, d
        for path in [G.PATH_AUTO, G.PATH_POINTWISE]:
            say("pointwise desc %s path %s" % (d, G.PATH_NAMES[path]))
            done = compare_full("%s %s" % (G.PATH_NAMES[path], d), run_path(path, x, w, b, dy, kw),
                                ref)
            pw_ran += path == G.PATH_POINTWISE and len(done) == 4
    assert pw_ran == 6


@pytest.mark.parametrize("groups", [1, 2])
def test_pointwise_integer_probe_exact(groups):
    """Integer data in [-3, 3] on a ResNeXt-sized 1x1 layer (256 -> 128 channels,
    56x56, 4 images): every partial sum is an exact fp32 integer, so the
    pointwise path equals the oracle bit for bit, split reduction included."""
    d = dict(N=4, C=256, K=128, H=56, W=56, kh=1, kw=1, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1,
             G=groups)
    kw = conv_kwargs(d)
    x = draw(("int", -3, 3), (4, 256, 56, 56), 21)
    w = draw(("int", -3, 3), (128, 256 // groups, 1, 1), 22)
    b = draw(("int", -3, 3), (128,), 23)
    dy = draw(("int", -3, 3), (4, 128, 56, 56), 24)
    desc = G.make_desc(4, 256, 56, 56, 128, 1, 1, groups=groups)
    for op in (G.OP_FWD, G.OP_BWD_DATA, G.OP_BWD_FILTER):
        assert G.gconv_select_path(desc, op) == G.PATH_POINTWISE
    assert G.gconv_workspace_size(desc, G.OP_BWD_FILTER) > 0   # split reduction
    say("pointwise integer probe groups %d" % groups)
    y, dx, dw, db = gpu_all_ops(x, w, b, dy, **kw)
    iy = sample_indices(y.numel(), 256, 31)
    ix = sample_indices(dx.numel(), 256, 32)
    assert np.array_equal(gather(y, iy), oracle.fwd(x, w, b, idx=iy, **kw)[0])
    assert np.array_equal(gather(dx, ix), oracle.bwd_data(dy, w, x.shape, idx=ix, **kw)[0])
    assert np.array_equal(dw.cpu().numpy().astype(np.float64),
                          oracle.bwd_filter(x, dy, w.shape, **kw)[0])


RELU_CASES = [
    # (descriptor, path the dispatcher takes for the forward pass)
    (dict(N=2, C=32, K=32, H=20, W=20, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=1), "igemm"),
    (dict(N=2, C=32, K=32, H=8, W=8, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=1), "igemm"),
    (dict(N=2, C=16, K=16, H=14, W=14, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=4),
     "smallgroup"),
    (dict(N=2, C=8, K=8, H=15, W=13, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=2),
     "smallgroup"),
    (dict(N=2, C=8, K=16, H=12, W=20, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=8),
     "smallgroup"),
    (dict(N=2, C=20, K=6, H=10, W=10, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=2), "direct"),
    (dict(N=1, C=4, K=4, H=12, W=12, kh=7, kw=7, sh=1, sw=1, ph=3, pw=3, dh=1, dw=1, G=1), "direct"),
    (dict(N=5, C=8, K=6, H=3, W=3, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1), "fc"),
    (dict(N=2, C=16, K=24, H=10, W=9, kh=1, kw=1, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1),
     "pointwise"),
]


@pytest.mark.parametrize("case", range(len(RELU_CASES)))
def test_relu_epilogue(case):
    """gconv_fwd_ex with the ReLU epilogue on every forward kernel family: max(y, 0)
    after the bias, element by element against the oracle; the plain forward
    pass of the same call sequence is unaffected."""
    d, path = RELU_CASES[case]
    kw = conv_kwargs(d)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], **kw)
    assert G.PATH_NAMES[G.gconv_select_path(desc, G.OP_FWD)] == path, d
    x, w, b = tensors(d, 1900 + case)
    say("relu epilogue %s" % d)
    xd, wd, bd = dev(x), dev(w), dev(b)
    y_relu = G.gconv_fwd(xd, wd, bd, relu=True, **kw)
    y_plain = G.gconv_fwd(xd, wd, bd, **kw)
    val, mag = oracle.fwd(x, w, b, relu=True, **kw)
    check("relu %s" % d, y_relu.cpu().numpy(), val, mag)
    val0, mag0 = oracle.fwd(x, w, b, **kw)
    check("plain %s" % d, y_plain.cpu().numpy(), val0, mag0)
    assert (y_relu >= 0).all()


# ----------------------------------------------------------------- asymmetric padding

@pytest.mark.parametrize("seed", range(2))
def test_asymmetric_padding_every_path(seed):
    """End padding that differs from the start padding (DLPrimitives Blog,
    "TensorFlow"), random descriptors, every kernel family that takes them."""
    descs = asym_descs(70 + seed, 16, max_hw=12, max_k=5, max_cg=6, max_kg=6, max_g=4)
    for d in descs:
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 700 + seed)
        y_ref, _ = oracle.fwd(x, w, b, **kw)
        dy = draw(("normal", 1.0), y_ref.shape, 710 + seed)
        ref = oracle_all(x, w, b, dy, kw)
        covered = set()
        for path in ALL_PATHS:
            say("asym desc %s path %s" % (d, G.PATH_NAMES[path]))
            covered |= set(compare_full("%s %s" % (G.PATH_NAMES[path], d),
                                        run_path(path, x, w, b, dy, kw), ref))
        assert covered == set(OPS)


def _same(H, W, k, s):
    t, b, l, r = G.same_padding(H, W, k, k, s)
    return dict(ph=t, pb=b, pw=l, pr=r)


ASYM_CASES = [
    # TensorFlow "same" padding at stride 2 (one more zero row and column at the end) on the
    # MFMA kernels, 3x3 and 5x5 ...
    (dict(N=2, C=32, K=32, H=20, W=20, kh=3, kw=3, sh=2, sw=2, dh=1, dw=1, G=1, **_same(20, 20, 3, 2)),
     {"fwd": "igemm", "bwd_data": "igemm", "bwd_filter": "igemm"}),
    (dict(N=2, C=32, K=32, H=21, W=20, kh=5, kw=5, sh=2, sw=2, dh=1, dw=1, G=1, **_same(21, 20, 5, 2)),
     {"fwd": "igemm", "bwd_data": "igemm", "bwd_filter": "igemm"}),
    # ... unequal start and end pads at stride 1, two groups
    (dict(N=2, C=32, K=48, H=13, W=17, kh=3, kw=3, sh=1, sw=1, ph=0, pb=2, pw=1, pr=0, dh=1, dw=1,
          G=2), {"fwd": "igemm", "bwd_data": "igemm", "bwd_filter": "igemm"}),
    # small-group row tile: no top pad, two right; and the widest row (62 + 0 + 2 columns)
    (dict(N=3, C=16, K=16, H=14, W=20, kh=3, kw=3, sh=1, sw=1, ph=1, pb=0, pw=0, pr=2, dh=1, dw=1,
          G=4), {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    (dict(N=2, C=8, K=8, H=5, W=62, kh=3, kw=3, sh=1, sw=1, ph=0, pb=1, pw=0, pr=2, dh=1, dw=1,
          G=2), {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # small-group general kernels at stride 2 with "same" padding
    (dict(N=2, C=32, K=32, H=15, W=14, kh=3, kw=3, sh=2, sw=2, dh=1, dw=1, G=8, **_same(15, 14, 3, 2)),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # depthwise row kernels (forward, gradInput, gradWeight) and depthwise "same" at stride 2
    (dict(N=3, C=8, K=8, H=17, W=30, kh=3, kw=3, sh=1, sw=1, ph=0, pb=1, pw=2, pr=0, dh=1, dw=1,
          G=8), {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    (dict(N=2, C=8, K=16, H=16, W=18, kh=3, kw=3, sh=2, sw=2, dh=1, dw=1, G=8, **_same(16, 18, 3, 2)),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # ... at the widest stride-2 row (31 outputs read input columns 0..62 of the LDS row;
    # gradInput's virtual input is read with pad 2 at the start), multiplier 1, nine groups
    # (the last block of four holds one)
    (dict(N=3, C=9, K=9, H=62, W=62, kh=3, kw=3, sh=2, sw=2, dh=1, dw=1, G=9, **_same(62, 62, 3, 2)),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # LDS-tiled direct kernels (20 in / 3 out per group)
    (dict(N=2, C=20, K=6, H=10, W=11, kh=3, kw=3, sh=1, sw=1, ph=2, pb=0, pw=0, pr=1, dh=1, dw=1,
          G=2), {"fwd": "direct", "bwd_data": "direct", "bwd_filter": "direct"}),
    # an even kernel, whose "same" padding is always asymmetric
    (dict(N=2, C=8, K=8, H=9, W=10, kh=4, kw=4, sh=1, sw=1, dh=1, dw=1, G=1, **_same(9, 10, 4, 1)),
     {"fwd": "direct", "bwd_data": "direct", "bwd_filter": "direct"}),
    # 1x1 with end padding: the extra output rows and columns hold the bias only, so it
    # leaves the pointwise GEMM (whose output planes are H x W)
    (dict(N=2, C=16, K=24, H=10, W=9, kh=1, kw=1, sh=1, sw=1, ph=0, pb=1, pw=0, pr=2, dh=1, dw=1,
          G=1), {"fwd": "direct", "bwd_data": "direct", "bwd_filter": "direct"}),
    # kernel == input with end padding below the stride: still one output, FC mode
    (dict(N=5, C=8, K=6, H=3, W=3, kh=3, kw=3, sh=2, sw=2, ph=0, pb=1, pw=0, pr=1, dh=1, dw=1,
          G=1), {"fwd": "fc", "bwd_data": "fc", "bwd_filter": "fc"}),
    # a dilated kernel the size of the input with end padding: one output, but its taps past
    # (0, 0) fall in the padding, so it is not a Linear layer and leaves the FC path
    (dict(N=3, C=4, K=5, H=2, W=2, kh=2, kw=2, sh=1, sw=1, ph=0, pb=1, pw=0, pr=1, dh=2, dw=2,
          G=1), {"fwd": "direct", "bwd_data": "direct", "bwd_filter": "direct"}),
]


# Strided gradInput on the MFMA path, in sub-pixel form: the dx pixels in
# blocks of sh x sw, each block a unit-stride correlation of the stored dy
# with an E x E super-filter (its taps that match no stored tap zero) and
# Cg*sh*sw output channels, one per (channel, sub-pixel). Cases span E = 1, 2
# and 3, 1 to 9 sub-pixels, the 16-byte stores (2x2 sub-pixels, dx width a
# multiple of 8) and the per-element ones, and 1 to 16 output fragments.
SUBPIXEL_CASES = [
    dict(N=2, C=64, K=64, H=40, W=40, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=8),    # 8 per group, 16-byte stores
    dict(N=2, C=32, K=48, H=35, W=41, kh=3, kw=3, sh=2, sw=2, ph=1, pw=0, dh=1, dw=1, G=1),    # odd sizes
    dict(N=3, C=128, K=64, H=34, W=34, kh=3, kw=3, sh=2, sw=2, ph=0, pw=0, dh=1, dw=1, G=2),   # pad 0: offsets -1, 0
    dict(N=1, C=256, K=32, H=36, W=38, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=1),   # 1024 super-channels
    dict(N=2, C=32, K=32, H=48, W=47, kh=3, kw=3, sh=3, sw=3, ph=1, pw=1, dh=1, dw=1, G=2),    # stride 3: 9 sub-pixels
    dict(N=2, C=48, K=32, H=40, W=40, kh=4, kw=4, sh=2, sw=2, ph=1, pw=2, dh=1, dw=1, G=1),    # 4x4: E = 3
    dict(N=2, C=32, K=32, H=40, W=36, kh=2, kw=2, sh=2, sw=2, ph=0, pw=0, dh=1, dw=1, G=2),    # 2x2: E = 1
    dict(N=2, C=64, K=64, H=40, W=40, kh=3, kw=3, sh=2, sw=2, ph=0, pb=1, pw=0, pr=1, dh=1, dw=1, G=8),  # "same"
    dict(N=2, C=48, K=48, H=33, W=32, kh=5, kw=5, sh=2, sw=2, ph=2, pw=2, dh=1, dw=1, G=2),    # 5x5: E = 3
    dict(N=2, C=24, K=32, H=30, W=29, kh=3, kw=3, sh=2, sw=1, ph=1, pw=1, dh=1, dw=1, G=2),    # strides (2, 1)
    dict(N=2, C=48, K=64, H=32, W=32, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=4),    # 3 output fragments
    dict(N=2, C=32, K=32, H=20, W=24, kh=3, kw=3, sh=2, sw=2, ph=2, pw=2, dh=1, dw=1, G=4),    # pad 2: offsets 0, 1
    dict(N=2, C=16, K=64, H=20, W=20, kh=1, kw=1, sh=2, sw=2, ph=0, pw=0, dh=1, dw=1, G=1),    # 1x1: zero sub-pixels
    dict(N=2, C=32, K=32, H=40, W=40, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=8),    # 4 per group
    dict(N=2, C=24, K=16, H=21, W=26, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=4),    # 6 dx, 4 dy per group
]


# Larger shapes (many workgroups, images spanning tiles), checked on sampled outputs.
SUBPIXEL_LARGE = [
    dict(N=16, C=64, K=64, H=64, W=64, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=8),
    dict(N=18, C=64, K=64, H=65, W=63, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=8),   # ragged blocks
    dict(N=8, C=32, K=48, H=128, W=128, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=1),
    dict(N=16, C=64, K=64, H=96, W=96, kh=3, kw=3, sh=3, sw=3, ph=1, pw=1, dh=1, dw=1, G=8),   # 9 sub-pixels
    dict(N=16, C=64, K=64, H=64, W=64, kh=4, kw=4, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=8),   # E = 3
    dict(N=8, C=128, K=128, H=64, W=64, kh=2, kw=2, sh=2, sw=2, ph=0, pw=0, dh=1, dw=1, G=8),  # E = 1
    dict(N=16, C=64, K=64, H=64, W=64, kh=3, kw=3, sh=2, sw=2, ph=0, pb=1, pw=0, pr=1, dh=1, dw=1, G=8),  # "same"
    dict(N=8, C=256, K=256, H=56, W=56, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=1),  # 16 fragments
    dict(N=16, C=128, K=128, H=64, W=64, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=32),  # 4 per group
]


@pytest.mark.parametrize("case", range(len(SUBPIXEL_LARGE)))
@pytest.mark.parametrize("layout", ["nchw", "nhwc"])
def test_strided_gradinput_subpixel_sampled(case, layout):
    """Strided gradInput in sub-pixel form at sizes of many workgroups, against
    the oracle on 4000 sampled outputs: normal data to the tolerance, integer
    data bit for bit."""
    d = SUBPIXEL_LARGE[case]
    kw = conv_kwargs(d)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], layout=layout, **kw)
    assert G.PATH_NAMES[G.gconv_select_path(desc, G.OP_BWD_DATA)] == "igemm", d
    nhwc = layout == "nhwc"
    to = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 3, 1))) if nhwc else (lambda a: a)
    Ho, Wo = G.gconv_output_dims(desc)
    ws = G.gconv_workspace_size(desc, G.OP_BWD_DATA)
    for dist, seed in ((("normal", 1.0), 2900), (("int", -3, 3), 2950)):
        w = draw(dist, (d["K"], d["C"] // d["G"], d["kh"], d["kw"]), seed + case)
        dy = draw(dist, (d["N"], d["K"], Ho, Wo), seed + 20 + case)
        say("subpixel sampled %s %s %s" % (layout, d, dist[0]))
        got = G.gconv_bwd_data(dev(to(dy)), dev(w), to(np.empty((d["N"], d["C"], d["H"], d["W"]), np.float32)).shape,
                               layout=layout, workspace=torch.empty(max(ws // 4, 1), device="cuda"), **kw)
        if nhwc:
            got = got.permute(0, 3, 1, 2).contiguous()
        idx = sample_indices(d["N"] * d["C"] * d["H"] * d["W"], 4000, seed + case)
        g = gather(got, idx)
        val, mag = oracle.bwd_data(dy, w, (d["N"], d["C"], d["H"], d["W"]), idx=idx, **kw)
        if dist[0] == "int":
            assert np.array_equal(g.astype(np.float64), val), d
        else:
            check("subpixel sampled %s" % d, g, val, mag)


@pytest.mark.parametrize("case", range(len(SUBPIXEL_CASES)))
@pytest.mark.parametrize("layout", ["nchw", "nhwc"])
def test_strided_gradinput_subpixel(case, layout):
    """Strided gradInput in sub-pixel form (the family asserted) against the
    oracle on every output: normal data to the tolerance, integer data bit for
    bit."""
    d = SUBPIXEL_CASES[case]
    kw = conv_kwargs(d)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], layout=layout, **kw)
    assert G.PATH_NAMES[G.gconv_select_path(desc, G.OP_BWD_DATA)] == "igemm", d
    nhwc = layout == "nhwc"
    to = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 3, 1))) if nhwc else (lambda a: a)
    for dist, seed in ((("normal", 1.0), 2700), (("int", -3, 3), 2800)):
        x, w, _ = tensors(d, seed + case, dist=dist, bias=False)
        Ho, Wo = G.gconv_output_dims(desc)
        dy = draw(dist, (d["N"], d["K"], Ho, Wo), seed + 50 + case)
        say("subpixel %s %s %s" % (layout, d, dist[0]))
        ws = G.gconv_workspace_size(desc, G.OP_BWD_DATA)
        got = G.gconv_bwd_data(dev(to(dy)), dev(w), to(x).shape, layout=layout,
                               workspace=torch.empty(max(ws // 4, 1), device="cuda"), **kw)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        if nhwc:
            got = got.transpose(0, 3, 1, 2)
        val, mag = oracle.bwd_data(dy, w, x.shape, **kw)
        if dist[0] == "int":
            assert np.array_equal(got.astype(np.float64), val), d
        else:
            check("subpixel %s" % d, got, val, mag)


# Depthwise 3x3 at unit stride (forward and gradInput) on the row-walking
# kernel: lanes = output columns of one, two or four planes (rows of up to 62,
# 30 or 14 outputs), bands of 14 output rows streamed one input row at a time.
DW_WALK_CASES = [
    # 62 outputs a row (the widest: lanes 62 and 63 only feed tap columns), three
    # bands (14, 14, 2 rows), 3 planes (one a wave), bias and ReLU
    (dict(N=1, C=3, K=3, H=30, W=62, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=3), True),
    # two planes a wave (30 outputs), an odd plane count (the last wave half
    # idle), no padding: 28 x 28 outputs in two bands
    (dict(N=3, C=5, K=5, H=30, W=30, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=5), False),
    # four planes a wave (14 outputs), 7 planes (the second wave's last slot
    # idle), two bands
    (dict(N=1, C=7, K=7, H=20, W=14, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=7), True),
    # padding 2: 18 x 14 outputs, four planes a wave
    (dict(N=2, C=4, K=4, H=16, W=12, kh=3, kw=3, sh=1, sw=1, ph=2, pw=2, dh=1, dw=1, G=4), False),
    # 60 rows of 10: two gradWeight bands (56, 4), four planes a wave, 6 planes
    (dict(N=1, C=6, K=6, H=60, W=10, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=6), False),
    # asymmetric padding: one row on top, none below, none left, two right
    (dict(N=2, C=6, K=6, H=29, W=20, kh=3, kw=3, sh=1, sw=1, dh=1, dw=1, G=6, ph=1, pb=0, pw=0, pr=2), False),
]


# ... and at stride 2: the forward puts output wo on lane 2 wo of its plane
# (planes of up to 31, 15 or 7 outputs a row: one, two or four a wave), the
# gradInput walks dy rows with dx column w on lane w + 2 (rows of up to 62, 30
# or 14 dx columns); bands of 7 output rows or 7 dy-row steps.
DW_WALK_CASES += [
    # 56 -> 28 "same" (no start padding, one zero row and column at the end):
    # four bands, one plane a wave
    (dict(N=2, C=3, K=3, H=56, W=56, kh=3, kw=3, sh=2, sw=2, dh=1, dw=1, G=3, ph=0, pb=1, pw=0, pr=1), True),
    # padding 1, odd sizes: 30 x 29 -> 15 x 15, two planes a wave (forward), two
    # dx planes a wave (gradInput, 29 columns), five planes
    (dict(N=1, C=5, K=5, H=30, W=29, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=5), False),
    # padding 2 on 13 x 14: 8 x 8 outputs (forward: two planes a wave), four dx
    # planes a wave
    (dict(N=3, C=2, K=2, H=13, W=14, kh=3, kw=3, sh=2, sw=2, ph=2, pw=2, dh=1, dw=1, G=2), True),
    # 7-column outputs (four forward planes a wave); two zero rows on top and
    # none below, one zero column each side
    (dict(N=2, C=9, K=9, H=33, W=13, kh=3, kw=3, sh=2, sw=2, dh=1, dw=1, G=9, ph=2, pb=0, pw=1, pr=1), False),
    # the widest rows of the stride-2 walks: 31 outputs on lanes 0 .. 62 (forward and
    # gradWeight), 62 dx columns on lanes 2 .. 63 (gradInput)
    (dict(N=1, C=3, K=3, H=12, W=62, kh=3, kw=3, sh=2, sw=2, dh=1, dw=1, G=3, ph=0, pb=1, pw=0, pr=1), True),
    # 30 outputs a row at unit stride: two planes a wave, each its 32 lanes exactly
    (dict(N=1, C=3, K=3, H=9, W=30, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=3), True),
    # 120 x 20 -> 60 x 10 at stride 2: three gradWeight bands (28, 28, 4), two
    # planes a wave
    (dict(N=1, C=4, K=4, H=120, W=20, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=4), False),
]


# Groups of two to four input and up to four output channels, 3x3 at unit
# stride (forward, and gradInput as the forward of dy with reversed taps), on
# the banded row kernel (one 64-float LDS row per input row, bands of up to
# 16 output rows).
SG_ROW_CASES = [
    # 4 in / 4 out, 62 outputs a row (the widest tile row: 64 floats), 30 rows
    # in two bands of 15, bias and ReLU
    (dict(N=2, C=16, K=16, H=30, W=62, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=4), True),
    # 3 in / 2 out, no padding: 15 x 19 outputs in one band
    (dict(N=1, C=12, K=8, H=17, W=21, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=4), False),
    # 2 in / 4 out with padding 2: 11 x 42 outputs
    (dict(N=3, C=6, K=12, H=9, W=40, kh=3, kw=3, sh=1, sw=1, ph=2, pw=2, dh=1, dw=1, G=3), True),
    # 1 in / 4 out (channel multiplier 4): the forward takes the depthwise
    # kernel, gradInput (4 in / 1 out) the row kernel
    (dict(N=1, C=5, K=20, H=28, W=28, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=5), False),
    # asymmetric padding: one row on top, none below, none left, two right
    (dict(N=2, C=8, K=8, H=29, W=20, kh=3, kw=3, sh=1, sw=1, dh=1, dw=1, G=2, ph=1, pb=0, pw=0, pr=2), False),
    # 4 in / 3 out at 56 x 56: four bands of 14
    (dict(N=2, C=8, K=6, H=56, W=56, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=2), True),
]


@pytest.mark.parametrize("case", range(len(SG_ROW_CASES)))
def test_smallgroup_rows(case):
    """Small groups at unit stride on the banded row kernel: forward (bias,
    optional ReLU) and gradInput against the oracle on every output, gradWeight
    alongside; integer data bit for bit."""
    d, relu = SG_ROW_CASES[case]
    kw = conv_kwargs(d)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], **kw)
    for op in (G.OP_FWD, G.OP_BWD_DATA):
        assert G.PATH_NAMES[G.gconv_select_path(desc, op)] == "smallgroup", d
    for dist, seed in ((("normal", 1.0), 3100), (("int", -3, 3), 3150)):
        say("small-group rows %s relu %s %s" % (d, relu, dist[0]))
        x, w, b = tensors(d, seed + 10 * case, dist=dist)
        y_ref, ya = oracle.fwd(x, w, b, relu=relu, **kw)
        dy = draw(dist, y_ref.shape, seed + 10 * case + 5)
        dx_ref, dxa = oracle.bwd_data(dy, w, x.shape, **kw)
        dw_ref, dwa = oracle.bwd_filter(x, dy, w.shape, **kw)
        y = G.gconv_fwd(dev(x), dev(w), dev(b), relu=relu, **kw)
        dx = G.gconv_bwd_data(dev(dy), dev(w), x.shape, **kw)
        dwg = G.gconv_bwd_filter(dev(x), dev(dy), w.shape, **kw)
        torch.cuda.synchronize()
        for tag, got, val, mag in (("fwd", y, y_ref, ya), ("bwd_data", dx, dx_ref, dxa),
                                   ("bwd_filter", dwg, dw_ref, dwa)):
            g = got.cpu().numpy()
            assert g.shape == val.shape, (d, tag)
            if dist[0] == "int":
                assert np.array_equal(g.astype(np.float64), val), (d, tag)
            else:
                check("sg rows %s %s" % (tag, d), g, val, mag)


@pytest.mark.parametrize("case", range(len(DW_WALK_CASES)))
def test_depthwise_walk(case):
    """Depthwise forward (bias, optional ReLU), gradInput and gradWeight at
    stride 1 and 2 on the row-walking kernels against the oracle on every
    output; integer data bit for bit."""
    d, relu = DW_WALK_CASES[case]
    kw = conv_kwargs(d)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], **kw)
    for op in (G.OP_FWD, G.OP_BWD_DATA, G.OP_BWD_FILTER):
        assert G.PATH_NAMES[G.gconv_select_path(desc, op)] == "smallgroup", d
    for dist, seed in ((("normal", 1.0), 2900), (("int", -3, 3), 2950)):
        say("depthwise walk %s relu %s %s" % (d, relu, dist[0]))
        x, w, b = tensors(d, seed + 10 * case, dist=dist)
        y_ref, ya = oracle.fwd(x, w, b, relu=relu, **kw)
        dy = draw(dist, y_ref.shape, seed + 10 * case + 5)
        dx_ref, dxa = oracle.bwd_data(dy, w, x.shape, **kw)
        dw_ref, dwa = oracle.bwd_filter(x, dy, w.shape, **kw)
        y = G.gconv_fwd(dev(x), dev(w), dev(b), relu=relu, **kw)
        dx = G.gconv_bwd_data(dev(dy), dev(w), x.shape, **kw)
        dwg = G.gconv_bwd_filter(dev(x), dev(dy), w.shape, **kw)
        torch.cuda.synchronize()
        for tag, got, val, mag in (("fwd", y, y_ref, ya), ("bwd_data", dx, dx_ref, dxa),
                                   ("bwd_filter", dwg, dw_ref, dwa)):
            g = got.cpu().numpy()
            assert g.shape == val.shape, (d, tag)
            if dist[0] == "int":
                assert np.array_equal(g.astype(np.float64), val), (d, tag)
            else:
                check("dw walk %s %s" % (tag, d), g, val, mag)


@pytest.mark.parametrize("case", range(len(ASYM_CASES)))
def test_asymmetric_padding_cases(case):
    """Asymmetric padding on the dispatcher's own choice of family (asserted):
    normal data to the tolerance, then integer data bit for bit."""
    d, paths = ASYM_CASES[case]
    kw = conv_kwargs(d)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], **kw)
    for op, name in paths.items():
        chosen = G.gconv_select_path(desc, getattr(G, "OP_" + op.upper()))
        assert G.PATH_NAMES[chosen] == name, (d, op, G.PATH_NAMES[chosen])
    say("asym case %s" % d)
    x, w, b = tensors(d, 2100 + case)
    y_ref, _ = oracle.fwd(x, w, b, **kw)
    dy = draw(("normal", 1.0), y_ref.shape, 2110 + case)
    compare_full("asym %s" % d, gpu_all_ops(x, w, b, dy, **kw), oracle_all(x, w, b, dy, kw))
    xi, wi, bi = tensors(d, 2200 + case, dist=("int", -3, 3))
    dyi = draw(("int", -3, 3), y_ref.shape, 2210 + case)
    got = gpu_all_ops(xi, wi, bi, dyi, **kw)
    for g, (val, _) in zip(got, oracle_all(xi, wi, bi, dyi, kw)):
        assert np.array_equal(g.cpu().numpy().astype(np.float64), val), d


@pytest.mark.parametrize("shape", [
    (3, 6, 13, 13),     # one pass, odd plane length (scalar loads)
    (5, 70, 28, 28),    # one pass, 16-byte loads, 70 channels
    (70, 2, 64, 64),    # split partials: more than 1 MiB per channel
    (700, 40, 1, 1),    # split partials over the rows of a [N, K] gradient (several rows per wave)
    (5000, 64, 1, 1),   # ... 64 columns: four rows per wave instruction
    (300, 1000, 1, 1),  # ... 250 column quads over four column blocks
    (40, 4100, 1, 1),   # ... wide rows: one thread per column quad
])
def test_bias_reduction_forms(shape):
    """gradBias in each of its forms (one workgroup per channel, or split
    partials plus an ordered finalize) against the oracle; integer-valued dy
    bit for bit."""
    say("bias %s" % (shape,))
    dy = draw(("normal", 1.0), shape, 2300 + shape[1])
    val, mag = oracle.bwd_bias(dy)
    check("bias %s" % (shape,), G.gconv_bwd_bias(dev(dy)).cpu().numpy(), val, mag)
    dyi = draw(("int", -3, 3), shape, 2400 + shape[1])
    vali, _ = oracle.bwd_bias(dyi)
    assert np.array_equal(G.gconv_bwd_bias(dev(dyi)).cpu().numpy().astype(np.float64), vali)


@pytest.mark.parametrize("shape,layout", [
    ((32, 64, 56, 56), "nchw"),     # planes split over 8 workgroups per channel
    ((160, 6, 25, 25), "nchw"),     # planes of 625 floats (scalar loads), 12 slices per channel
    ((1600, 4096, 1, 1), "nchw"),   # [N, K] rows, 4 column blocks x 124 row slices
    ((3000, 1002, 1, 1), "nchw"),   # [N, K] rows, K not a multiple of 4 (one column per thread)
    ((8, 64, 28, 28), "nhwc"),      # NHWC: [N*Ho*Wo, 64] narrow rows
])
def test_bias_split_slices(shape, layout):
    """gradBias whose reduction groups are split over workgroups, with the
    slices' partials in the workspace and added in order by a second kernel.
    Whatever the workspace holds beforehand (random bits), and on a second call
    with the same workspace, the result matches the oracle, and integer data
    bit for bit."""
    N, K, Ho, Wo = shape
    nhwc = layout == "nhwc"
    desc = G.make_desc(N, K, Ho, Wo, K, 1, 1, layout=layout)
    nws = G.gconv_workspace_size(desc, G.OP_BWD_BIAS)
    assert nws > 0, shape
    gen = torch.Generator(device="cuda").manual_seed(shape[1])
    ws = torch.randint(-2**31, 2**31 - 1, (nws // 4,), dtype=torch.int32, device="cuda",
                       generator=gen).view(torch.float32)
    for dist, seed in ((("normal", 1.0), 2500), (("int", -3, 3), 2600)):
        dy = draw(dist, shape, seed + K)
        val, mag = oracle.bwd_bias(dy)
        dyd = dev(np.ascontiguousarray(dy.transpose(0, 2, 3, 1)) if nhwc else dy)
        for call in range(2):
            say("bias slices %s %s %s call %d" % (shape, layout, dist[0], call))
            got = G.gconv_bwd_bias(dyd, workspace=ws, layout=layout).cpu().numpy()
            if dist[0] == "int":
                assert np.array_equal(got.astype(np.float64), val), (shape, call)
            else:
                check("bias %s call %d" % (shape, call), got, val, mag)


def test_fc_1x1_on_1x1_is_linear():
    """A 1x1 convolution of a 1x1 input (the Linear(128, 32) case of the
    cudnn.torch issue) runs the GEMM path and matches the oracle."""
    d = dict(N=16, C=128, H=1, W=1, K=32, kh=1, kw=1, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1)
    kw = conv_kwargs(d)
    x, w, b = tensors(d, 950)
    dy = draw(("normal", 1.0), (16, 32, 1, 1), 951)
    desc = G.make_desc(16, 128, 1, 1, 32, 1, 1)
    assert G.gconv_select_path(desc, G.OP_FWD) == G.PATH_FC
    compare_full("linear", run_path(G.PATH_AUTO, x, w, b, dy, kw), oracle_all(x, w, b, dy, kw))


def test_ragged_shapes_span_several_tiles():
    """Shapes whose extents are not multiples of any tile (tails in every dim)."""
    cases = [
        dict(N=3, C=70, H=19, W=23, K=66, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=1),
        dict(N=2, C=96, H=13, W=29, K=132, kh=5, kw=5, sh=1, sw=1, ph=2, pw=2, dh=1, dw=1, G=2),
        dict(N=5, C=36, H=17, W=11, K=36, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=9),
        dict(N=33, C=20, H=5, W=7, K=70, kh=5, kw=7, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1),
        dict(N=4, C=48, H=15, W=15, K=64, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=4),
        dict(N=2, C=32, H=21, W=20, K=32, kh=3, kw=3, sh=1, sw=1, ph=2, pw=2, dh=2, dw=2, G=32),
    ]
    for i, d in enumerate(cases):
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 800 + i)
        y, _ = oracle.fwd(x, w, b, **kw)
        dy = draw(("normal", 1.0), y.shape, 900 + i)
        ref = oracle_all(x, w, b, dy, kw)
        for path in [G.PATH_AUTO] + ALL_PATHS:
            say("ragged %s path %s" % (d, G.PATH_NAMES[path]))
            compare_full("ragged%d %s" % (i, G.PATH_NAMES[path]),
                         run_path(path, x, w, b, dy, kw), ref)


# ----------------------------------------------------------------- the five workloads

REDUCED_BATCH = {"tiny_grouped": 2, "dense3x3": 2, "alexnet_conv2": 2, "resnext_32x4d": 3,
                 "fc_mode": 24, "resnext_1x1": 2, "mobilenet_dw": 2, "mobilenet_dw_s2_same": 2,
                 "resnext_32x4d_s2": 2, "dense3x3_nhwc": 2, "resnext_1x1_nhwc": 2, "mobilenet_dw_nhwc": 2}


def wl_kwargs(wl):
    return dict(stride=wl.stride, padding=wl.padding, dilation=wl.dilation, groups=wl.groups)


@pytest.mark.parametrize("name", WORKLOAD_ORDER)
def test_workload_reduced_batch_full_tensors(name):
    """Every element, on the workload's own values cut to a few images."""
    wl = WORKLOADS[name]
    inp = make_inputs(name, batch=REDUCED_BATCH[name])
    kw = wl_kwargs(wl)
    say("workload %s reduced batch %d" % (name, REDUCED_BATCH[name]))
    ref = oracle_all(inp["x"], inp["w"], inp["b"], inp["dy"], kw)
    gpu = gpu_all_ops(inp["x"], inp["w"], inp["b"], inp["dy"], layout=wl.layout, **kw)
    compare_full(name, gpu, ref)


@pytest.mark.parametrize("name", WORKLOAD_ORDER)
def test_workload_full_size_sampled(name):
    """Full size, the dispatcher's own path (what the benchmark times); sampled
    elements computed one by one by the oracle."""
    wl = WORKLOADS[name]
    inp = make_inputs(name)
    kw = wl_kwargs(wl)
    x, w, b, dy = inp["x"], inp["w"], inp["b"], inp["dy"]
    say("workload %s full size" % name)
    y, dx, dw, db = gpu_all_ops(x, w, b, dy, layout=wl.layout, **kw)
    assert tuple(y.shape) == wl.dy_shape and tuple(dx.shape) == wl.x_shape
    assert tuple(dw.shape) == wl.w_shape and tuple(db.shape) == (wl.w_shape[0],)
    n = 384
    iy = sample_indices(y.numel(), n, 1)
    check(name + " fwd", gather(y, iy), *oracle.fwd(x, w, b, idx=iy, **kw))
    ix = sample_indices(dx.numel(), n, 2)
    check(name + " bwd_data", gather(dx, ix), *oracle.bwd_data(dy, w, x.shape, idx=ix, **kw))
    iw = sample_indices(dw.numel(), 128, 3)
    check(name + " bwd_filter", gather(dw, iw), *oracle.bwd_filter(x, dy, w.shape, idx=iw, **kw))
    check(name + " bwd_bias", db.cpu().numpy(), *oracle.bwd_bias(dy))
    # Smoke criteria of the clnn issue: right size, not all zeros, no NaN, no
    # 1e-38-scale values where data is dense.
    for t in (y, dx, dw):
        assert torch.isfinite(t).all() and (t != 0).any()


@pytest.mark.parametrize("name", WORKLOAD_ORDER)
def test_workload_integer_probes_exact(name):
    """Integer data in [-3, 3] at the workload's full shape: every partial sum is
    an exact fp32 integer, so GPU == oracle bit for bit (index mapping, group
    offsets, padding and shapes, whatever the summation order)."""
    wl = WORKLOADS[name]
    kw = wl_kwargs(wl)
    x = draw(("int", -3, 3), wl.x_shape, 11)
    w = draw(("int", -3, 3), wl.w_shape, 12)
    b = draw(("int", -3, 3), (wl.w_shape[0],), 13)
    dy = draw(("int", -3, 3), wl.dy_shape, 14)
    say("integer probes %s" % name)
    y, dx, dw, db = gpu_all_ops(x, w, b, dy, layout=wl.layout, **kw)
    iy = sample_indices(y.numel(), 256, 4)
    ix = sample_indices(dx.numel(), 256, 5)
    iw = sample_indices(dw.numel(), 96, 6)
    assert np.array_equal(gather(y, iy), oracle.fwd(x, w, b, idx=iy, **kw)[0]), name
    assert np.array_equal(gather(dx, ix), oracle.bwd_data(dy, w, x.shape, idx=ix, **kw)[0]), name
    assert np.array_equal(gather(dw, iw), oracle.bwd_filter(x, dy, w.shape, idx=iw, **kw)[0]), name
    assert np.array_equal(db.cpu().numpy().astype(np.float64), oracle.bwd_bias(dy)[0])


EDGE_CASES = [
    # flat-pixel MFMA conv: 48 outputs per group (three waves) with a partial
    # 2-channel reduction chunk on the forward pass, 18 outputs (two waves
    # across pixels) on gradInput; tiles spanning image boundaries
    (dict(N=3, C=18, K=48, H=12, W=12, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=1),
     {"fwd": "igemm", "bwd_data": "igemm"}),
    # two groups, 5x5, outputs past one 64-channel tile, ragged last tile
    (dict(N=2, C=2 * 20, K=2 * 70, H=11, W=13, kh=5, kw=5, sh=1, sw=1, ph=2, pw=2, dh=1, dw=1,
          G=2), {"fwd": "igemm", "bwd_data": "igemm"}),
    # small-group gradWeight over image runs: 37 images, 32 groups -> runs of
    # two images, the last run holding one
    (dict(N=37, C=128, K=128, H=12, W=14, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=32),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # row-per-DMA small-group kernels at the widest row (62 + 2 = 64 floats)
    (dict(N=2, C=8, K=8, H=5, W=62, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=2),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # ... without padding (tile columns start at the image edge) and with pad 2
    (dict(N=2, C=3, K=4, H=7, W=40, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    (dict(N=1, C=4, K=4, H=6, W=30, kh=3, kw=3, sh=1, sw=1, ph=2, pw=2, dh=1, dw=1, G=1),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # row-per-DMA small-group kernels over many (image, group) planes: 13 rows
    # make one band of each plane ragged, and gradWeight runs hold two images
    (dict(N=37, C=128, K=128, H=13, W=20, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=32),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # ... the widest tile with pad 2 (60 + 2 columns), 3 in / 7 out channels
    # per group (two output quads, the second partial; gradWeight streams one
    # input and two output quads)
    (dict(N=3, C=2 * 3, K=2 * 7, H=9, W=60, kh=3, kw=3, sh=1, sw=1, ph=1, pw=2, dh=1, dw=1, G=2),
     {"fwd": "smallgroup", "bwd_data": "direct", "bwd_filter": "smallgroup"}),
    # ... gradInput with 3 in / 6 out channels per group
    (dict(N=2, C=2 * 6, K=2 * 3, H=7, W=8, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=2),
     {"bwd_data": "smallgroup"}),
    # ... one input channel, three outputs, no padding
    (dict(N=2, C=1, K=3, H=6, W=8, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1),
     {"fwd": "smallgroup"}),
    # 5x5 small-group forward / gradInput: depthwise with channel multiplier 2 ...
    (dict(N=2, C=6, K=12, H=13, W=17, kh=5, kw=5, sh=1, sw=1, ph=2, pw=2, dh=1, dw=1, G=6),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "direct"}),
    # ... and two input channels per group at stride 2, unequal padding
    (dict(N=3, C=4, K=6, H=15, W=11, kh=5, kw=5, sh=2, sw=2, ph=1, pw=2, dh=1, dw=1, G=2),
     {"fwd": "smallgroup", "bwd_data": "direct", "bwd_filter": "direct"}),
    # 8 in / 8 out channels per group (ResNeXt's second stage): two groups per
    # 16-wide MFMA fragment on forward and gradInput; gradWeight streams 2 x 2
    # channel quads on the 4x4 MFMA blocks
    (dict(N=2, C=64, K=64, H=20, W=20, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=8),
     {"fwd": "igemm", "bwd_data": "igemm", "bwd_filter": "smallgroup"}),
    # streaming small-group gradWeight at stride 2: 8 x 8 channels per group
    # (ResNeXt's strided 3x3), 15 outputs a row ...
    (dict(N=3, C=32, K=32, H=28, W=30, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=4),
     {"bwd_filter": "smallgroup"}),
    # ... the widest strided row (31 outputs over 61 + 1 columns), odd height
    (dict(N=5, C=16, K=16, H=23, W=61, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=4),
     {"bwd_filter": "smallgroup"}),
    # ... 8 in / 4 out channels, no padding
    (dict(N=2, C=16, K=8, H=20, W=24, kh=3, kw=3, sh=2, sw=2, ph=0, pw=0, dh=1, dw=1, G=2),
     {"bwd_filter": "smallgroup"}),
    # ... at stride 1: 5 in / 3 out channels, pad 2
    (dict(N=2, C=10, K=6, H=17, W=33, kh=3, kw=3, sh=1, sw=1, ph=2, pw=2, dh=1, dw=1, G=2),
     {"bwd_filter": "smallgroup"}),
    # ... two units a wave (more units than two rounds of resident waves): 4 x 4
    # channels over 400 images, and 8 x 8 over 600
    (dict(N=400, C=128, K=128, H=8, W=8, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=32),
     {"bwd_filter": "smallgroup"}),
    (dict(N=600, C=64, K=64, H=8, W=8, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=8),
     {"bwd_filter": "smallgroup"}),
    # strided gradInput on the direct kernel (taps filtered once per element,
    # channels of the group innermost): 6 channels per group, stride 2; 2 per
    # group, strides 3 and 2 with dilation
    (dict(N=2, C=12, K=16, H=14, W=13, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=2),
     {"bwd_data": "direct"}),
    (dict(N=2, C=6, K=9, H=16, W=17, kh=5, kw=3, sh=3, sw=2, ph=2, pw=0, dh=2, dw=1, G=3),
     {"bwd_data": "direct"}),
    # strided gradInput on the MFMA flat kernel, reading dy as if upsampled by
    # the stride: 8 channels per group at stride 2 (odd and even sizes) ...
    (dict(N=2, C=16, K=16, H=18, W=17, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=2),
     {"bwd_data": "igemm"}),
    # ... 16 per group at strides 3 x 2 with unequal padding, 18 x 19 outputs ...
    (dict(N=3, C=2 * 16, K=2 * 24, H=18, W=19, kh=3, kw=3, sh=3, sw=2, ph=1, pw=0, dh=1, dw=1,
          G=2), {"bwd_data": "igemm"}),
    # ... and 5x5 at stride 2
    (dict(N=2, C=32, K=32, H=21, W=20, kh=5, kw=5, sh=2, sw=2, ph=2, pw=2, dh=1, dw=1, G=1),
     {"bwd_data": "igemm"}),
    # depthwise VALU kernel, four groups per workgroup: multiplier 3 over 6
    # groups (the last workgroup holds two), and multiplier 1 over 5 groups
    # (gradInput takes it too)
    (dict(N=2, C=6, K=18, H=21, W=30, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=6),
     {"fwd": "smallgroup", "bwd_data": "smallgroup"}),
    (dict(N=3, C=5, K=5, H=17, W=40, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=5),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # depthwise gradWeight on the row tile: multiplier 2 over 6 groups (the
    # last group block holds two) and 37 images (one per workgroup run)
    (dict(N=37, C=6, K=12, H=19, W=33, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=6),
     {"fwd": "smallgroup", "bwd_filter": "smallgroup"}),
    # strided gradInput on the small-group kernels (dy read as if upsampled):
    # depthwise 3x3 at stride 2, odd and even sizes ...
    (dict(N=2, C=8, K=8, H=15, W=14, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=8),
     {"fwd": "smallgroup", "bwd_data": "smallgroup"}),
    # ... and 4 in / 2 out channels (gradInput's view) at stride 2, dilation 2
    (dict(N=2, C=4, K=8, H=17, W=19, kh=3, kw=3, sh=2, sw=2, ph=2, pw=2, dh=2, dw=2, G=2),
     {"bwd_data": "smallgroup"}),
    # depthwise row kernels at stride 2: multiplier 2, pad 2 on the widest row
    # (31 outputs), 18 output rows in three bands, 37 images over the
    # gradWeight runs ...
    (dict(N=37, C=6, K=12, H=35, W=60, kh=3, kw=3, sh=2, sw=2, ph=1, pw=2, dh=1, dw=1, G=6),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # ... and multiplier 1 with pad 1 (gradInput on the depthwise kernel over dy
    # upsampled by 2: 61-wide rows with pad 1, 17 dy rows)
    (dict(N=2, C=5, K=5, H=33, W=61, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=5),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # depthwise gradInput at stride 2 split by output phase: pad 2 (the first
    # phase row and column start one dx row and column early), 50 phase rows in
    # four bands, 50 phase columns, six groups (the second block of four holds two)
    (dict(N=2, C=6, K=6, H=100, W=100, kh=3, kw=3, sh=2, sw=2, ph=2, pw=2, dh=1, dw=1, G=6),
     {"bwd_data": "smallgroup"}),
    # ... odd sizes with pad 0 and 1 (the last phase row and column are half outside dx)
    (dict(N=3, C=5, K=5, H=19, W=23, kh=3, kw=3, sh=2, sw=2, ph=0, pw=1, dh=1, dw=1, G=5),
     {"fwd": "smallgroup", "bwd_data": "smallgroup", "bwd_filter": "smallgroup"}),
    # fully-connected gradWeight with few output tiles and many rows: the rows
    # split over workgroup slices, partials added in slice order
    (dict(N=5000, C=8, K=16, H=3, W=3, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1),
     {"fwd": "fc", "bwd_data": "fc", "bwd_filter": "fc"}),
    # direct gradWeight with 1024-thread blocks (at least 16K pixels): depthwise
    # 5x5, and 8 per group at stride 2
    (dict(N=4, C=8, K=8, H=64, W=64, kh=5, kw=5, sh=1, sw=1, ph=2, pw=2, dh=1, dw=1, G=8),
     {"bwd_filter": "direct"}),
    (dict(N=8, C=16, K=16, H=96, W=96, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=2),
     {"bwd_filter": "direct"}),
    # strided forward on the flat kernel: 8 per group at stride 2 (a tile spans
    # 30 input rows: the 24-segment instance) ...
    (dict(N=2, C=16, K=16, H=40, W=40, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=2),
     {"fwd": "igemm", "bwd_data": "igemm"}),
    # ... and 80 outputs (two fragments) on 100-wide rows (the 16-segment one)
    (dict(N=1, C=80, K=80, H=12, W=100, kh=3, kw=3, sh=2, sw=2, ph=1, pw=1, dh=1, dw=1, G=1),
     {"fwd": "igemm", "bwd_data": "igemm"}),
]


@pytest.mark.parametrize("case", range(len(EDGE_CASES)))
def test_kernel_edge_cases(case):
    """Shapes at the edges of the tiled kernels' layouts, on the dispatcher's
    own choice (asserted), every element against the oracle."""
    d, paths = EDGE_CASES[case]
    kw = conv_kwargs(d)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], **kw)
    for op, name in paths.items():
        chosen = G.gconv_select_path(desc, getattr(G, "OP_" + op.upper()))
        assert G.PATH_NAMES[chosen] == name, (d, op, G.PATH_NAMES[chosen])
    x, w, b = tensors(d, 1500 + case)
    y_ref, _ = oracle.fwd(x, w, b, **kw)
    dy = draw(("normal", 1.0), y_ref.shape, 1510 + case)
    say("edge case %s" % d)
    compare_full("edge %s" % d, gpu_all_ops(x, w, b, dy, **kw), oracle_all(x, w, b, dy, kw))


# The flattened-pixel MFMA kernel takes tiles of consecutive pixels over the
# N x Ho x Wo output, so a tile may end one image and start the next; its LDS
# tile then holds both parts, each with its own halo rows. On short images
# (few output rows against the tile's pixel span) the two parts together hold
# more rows than one image has. These layers put such a tile on each kernel
# layout (256- and 128-pixel tiles, packed and unpacked groups, stride 2 with
# dilation, the upsampled gradInput).
SPAN_CASES = [
    dict(N=2, C=7, K=35, H=7, W=52, kh=3, kw=3, sh=1, sw=1, ph=0, pw=1, dh=1, dw=1, G=7),
    dict(N=3, C=64, K=32, H=29, W=41, kh=3, kw=3, sh=2, sw=2, ph=1, pw=0, dh=2, dw=2, G=8),
    dict(N=3, C=32, K=8, H=6, W=43, kh=3, kw=3, sh=1, sw=2, ph=1, pw=1, dh=1, dw=1, G=8),
    dict(N=2, C=8, K=64, H=7, W=50, kh=3, kw=3, sh=1, sw=1, ph=0, pw=2, dh=1, dw=1, G=8),
    dict(N=2, C=21, K=93, H=13, W=24, kh=3, kw=3, sh=2, sw=1, ph=1, pw=0, dh=2, dw=1, G=3),
    # the same kind of span with the dispatcher choosing the MFMA path itself
    dict(N=3, C=32, K=64, H=5, W=52, kh=3, kw=3, sh=1, sw=1, ph=0, pw=1, dh=1, dw=1, G=2),
]


@pytest.mark.parametrize("case", range(len(SPAN_CASES)))
def test_flat_tiles_spanning_short_images(case):
    """Tiles that cross from one short image into the next, on the MFMA path
    (forced, and the dispatcher's choice), NCHW and channels-last, every
    element against the oracle."""
    from test_gpu_nhwc import gpu_nhwc, refs
    d = SPAN_CASES[case]
    kw = conv_kwargs(d)
    x, w, b = tensors(d, 3400 + case)
    y_ref, _ = oracle.fwd(x, w, b, **kw)
    dy = draw(("normal", 1.0), y_ref.shape, 3410 + case)
    ref = oracle_all(x, w, b, dy, kw)
    say("span case %s" % d)
    # (a layout whose staged rows no longer fit the kernel's registers is
    # declined, GCONV_ERR_UNSUPPORTED, rather than run)
    done = compare_full("igemm %s" % d, run_path(G.PATH_IGEMM, x, w, b, dy, kw), ref)
    assert "fwd" in done or "bwd_data" in done, (d, done)
    compare_full("auto %s" % d, run_path(G.PATH_AUTO, x, w, b, dy, kw), ref)
    rn = refs(x, w, b, dy, kw)
    for path in (G.PATH_IGEMM, G.PATH_AUTO):
        G.gconv_set_path_override(path)
        try:
            got = gpu_nhwc(x, w, b, dy, kw)
        finally:
            G.gconv_set_path_override(G.PATH_AUTO)
        for op in OPS:
            if got[op] is not None:
                val, mag = rn[op]
                check("nhwc %s %s %s" % (G.PATH_NAMES[path], op, d), got[op].cpu().numpy(), val, mag)


# Fully-connected layers whose GEMMs have at least a tile per CU take the
# balanced form: 512 blocks share the (tile, stage) sequence evenly, a tile
# held by two or three blocks is summed from their parts in block order.
# These put each FC GEMM on it in turn (ragged tiles, groups, ReLU).
SK_CASES = [
    # forward: 6 x 47 = 282 tiles of 2 stages
    (dict(N=700, C=4, K=6000, H=3, W=3, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1), True),
    # gradInput: 6 x 43 = 258 tiles (64 output channels: 2 stages)
    (dict(N=650, C=600, K=64, H=3, W=3, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1), False),
    # gradWeight: 16 x 18 = 288 tiles of 10 stages (300 images)
    (dict(N=300, C=256, K=2048, H=3, W=3, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1), False),
    # four groups: forward 5 x 14 x 4 = 280 tiles
    (dict(N=520, C=256, K=6800, H=3, W=3, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=4), True),
]


@pytest.mark.parametrize("case", range(len(SK_CASES)))
def test_fc_balanced_form(case):
    """FC GEMMs on the balanced form: every element against the oracle,
    integer data bit for bit."""
    d, relu = SK_CASES[case]
    kw = conv_kwargs(d)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], **kw)
    assert G.PATH_NAMES[G.gconv_select_path(desc, G.OP_FWD)] == "fc", d
    for dist, seed in ((("normal", 1.0), 3500), (("int", -3, 3), 3550)):
        say("fc balanced %s relu %s %s" % (d, relu, dist[0]))
        x, w, b = tensors(d, seed + 10 * case, dist=dist)
        y_ref, ya = oracle.fwd(x, w, b, relu=relu, **kw)
        dy = draw(dist, y_ref.shape, seed + 10 * case + 5)
        dx_ref, dxa = oracle.bwd_data(dy, w, x.shape, **kw)
        dw_ref, dwa = oracle.bwd_filter(x, dy, w.shape, **kw)
        y = G.gconv_fwd(dev(x), dev(w), dev(b), relu=relu, **kw)
        dx = G.gconv_bwd_data(dev(dy), dev(w), x.shape, **kw)
        dwg = G.gconv_bwd_filter(dev(x), dev(dy), w.shape, **kw)
        torch.cuda.synchronize()
        for tag, got, val, mag in (("fwd", y, y_ref, ya), ("bwd_data", dx, dx_ref, dxa),
                                   ("bwd_filter", dwg, dw_ref, dwa)):
            g = got.cpu().numpy()
            assert g.shape == val.shape, (d, tag)
            if dist[0] == "int":
                assert np.array_equal(g.astype(np.float64), val), (d, tag)
            else:
                check("fc balanced %s %s" % (tag, d), g, val, mag)


# GEMMs of more tiles than the chip holds blocks at once, with short
# reductions: the pointwise forward and gradInput, the channels-last 1x1 GEMM
# and FC forward and gradWeight (ragged stages and tiles, groups, ReLU, tile
# counts that 512 does not divide).
MANY_TILE_CASES = [
    # pointwise: forward 2 x 29 x 16 = 928 tiles of 5 stages, gradInput 928 of 7
    (dict(N=16, C=136, K=200, H=60, W=60, kh=1, kw=1, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1), True, "nchw"),
    # two groups: 41 x 16 = 656 tiles of 3 stages each way
    (dict(N=8, C=144, K=192, H=72, W=72, kh=1, kw=1, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=2), True, "nchw"),
    # channels-last 1x1: one GEMM of 113 x 2 x 4 = 904 tiles (forward)
    (dict(N=16, C=136, K=200, H=60, W=60, kh=1, kw=1, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1), False, "nhwc"),
    # FC gradWeight: 16 x 36 = 576 tiles over 100 images (4 stages, ragged)
    (dict(N=100, C=512, K=2048, H=3, W=3, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1), False, "nchw"),
    # FC forward: 16 x 47 = 752 tiles of 2 stages
    (dict(N=2000, C=4, K=6000, H=3, W=3, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1), True, "nchw"),
]


@pytest.mark.parametrize("case", range(len(MANY_TILE_CASES)))
def test_gemm_many_short_tiles(case):
    """Every element of the forward, gradInput and gradWeight against the
    oracle, integer data bit for bit."""
    d, relu, layout = MANY_TILE_CASES[case]
    kw = conv_kwargs(d)
    nhwc = layout == "nhwc"
    store = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 3, 1))) if nhwc else (lambda a: a)
    back = (lambda t: t.permute(0, 3, 1, 2).contiguous()) if nhwc else (lambda t: t)
    for dist, seed in ((("normal", 1.0), 3700), (("int", -3, 3), 3750)):
        say("gemm many tiles %s relu %s %s %s" % (d, relu, layout, dist[0]))
        x, w, b = tensors(d, seed + 10 * case, dist=dist)
        y_ref, ya = oracle.fwd(x, w, b, relu=relu, **kw)
        dy = draw(dist, y_ref.shape, seed + 10 * case + 5)
        dx_ref, dxa = oracle.bwd_data(dy, w, x.shape, **kw)
        dw_ref, dwa = oracle.bwd_filter(x, dy, w.shape, **kw)
        y = back(G.gconv_fwd(dev(store(x)), dev(w), dev(b), relu=relu, layout=layout, **kw))
        dx = back(G.gconv_bwd_data(dev(store(dy)), dev(w), store(x).shape, layout=layout, **kw))
        dwg = G.gconv_bwd_filter(dev(store(x)), dev(store(dy)), w.shape, layout=layout, **kw)
        torch.cuda.synchronize()
        for tag, got, val, mag in (("fwd", y, y_ref, ya), ("bwd_data", dx, dx_ref, dxa),
                                   ("bwd_filter", dwg, dw_ref, dwa)):
            g = got.cpu().numpy()
            assert g.shape == val.shape, (d, tag)
            if dist[0] == "int":
                assert np.array_equal(g.astype(np.float64), val), (d, tag)
            else:
                check("gemm many tiles %s %s" % (tag, d), g, val, mag)


# FC GEMMs whose blocks run long reductions stage the row-contiguous operand
# (gradInput's filter, gradWeight's dy) as [8][row][4]. Too large for the full
# oracle in seconds, so sampled elements are computed one by one.
LONG_FC = [
    # gradInput 9 x 32 = 288 tiles of 64 stages (balanced form), gradWeight
    # 16 x 32 = 512 whole tiles of 35 stages (1100 images, the last stage ragged)
    dict(N=1100, C=256, K=2048, H=4, W=4, kh=4, kw=4, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1),
    # gradInput over 1500 output planes (47 stages, the last ragged, balanced
    # form); gradWeight 12 x 32 = 384 tiles in two slices of 18 stages
    dict(N=1100, C=256, K=1500, H=4, W=4, kh=4, kw=4, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1),
    # whole rounds, then a balanced tail: forward 9 x 61 = 549 tiles of 32 stages (512 whole,
    # 37 balanced); gradWeight 61 x 8 = 488 tiles in two slices of 18 stages
    dict(N=1100, C=64, K=7800, H=4, W=4, kh=4, kw=4, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1),
    # a tail of fewer (tile, stage) pairs than blocks: gradWeight 11 x 47 = 517 tiles, 5 balanced
    # tiles of 35 stages (the last ragged) over 175 blocks
    dict(N=1100, C=376, K=1408, H=4, W=4, kh=4, kw=4, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1),
]


@pytest.mark.parametrize("case", range(len(LONG_FC)))
def test_fc_long_reductions_sampled(case):
    d = LONG_FC[case]
    kw = conv_kwargs(d)
    for dist, seed in ((("normal", 1.0), 3800 + 10 * case), (("int", -3, 3), 3850 + 10 * case)):
        say("fc long reductions %s %s" % (d, dist[0]))
        x, w, b = tensors(d, seed, dist=dist)
        dy = draw(dist, (d["N"], d["K"], 1, 1), seed + 5)
        y, dx, dwg, _ = gpu_all_ops(x, w, b, dy, **kw)
        iy = sample_indices(y.numel(), 256, seed + 1)
        ix = sample_indices(dx.numel(), 256, seed + 2)
        iw = sample_indices(dwg.numel(), 256, seed + 3)
        for tag, got, (val, mag) in (
                ("fwd", gather(y, iy), oracle.fwd(x, w, b, idx=iy, **kw)),
                ("bwd_data", gather(dx, ix), oracle.bwd_data(dy, w, x.shape, idx=ix, **kw)),
                ("bwd_filter", gather(dwg, iw), oracle.bwd_filter(x, dy, w.shape, idx=iw, **kw))):
            if dist[0] == "int":
                assert np.array_equal(got.astype(np.float64), val), tag
            else:
                check("fc long %s" % tag, got, val, mag)


def test_fc_all_ones_bit_exact():
    """The all-ones fully-connected problem of the cudnn.torch issue: every
    element of all four results equals its integer closed form."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fc_all_ones.json")))
    x = torch.ones(g["x_shape"], device="cuda")
    w = torch.ones(g["w_shape"], device="cuda")
    b = torch.ones(g["w_shape"][0], device="cuda")
    dy = torch.ones(g["dy_shape"], device="cuda")
    say("fc all ones")
    y = G.gconv_fwd(x, w, b)
    dx = G.gconv_bwd_data(dy, w, x.shape)
    dw = G.gconv_bwd_filter(x, dy, w.shape)
    db = G.gconv_bwd_bias(dy)
    torch.cuda.synchronize()
    ex = g["expected"]
    assert tuple(y.shape) == tuple(g["dy_shape"])
    assert bool((y == ex["output"]).all()) and bool((dx == ex["gradInput"]).all())
    assert bool((dw == ex["gradWeight"]).all()) and bool((db == ex["gradBias"]).all())


# ----------------------------------------------------------------- robustness

def test_deterministic_bitwise():
    d = dict(N=4, C=64, H=20, W=20, K=64, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=2)
    kw = conv_kwargs(d)
    x, w, b = tensors(d, 1)
    dy = draw(("normal", 1.0), (4, 64, 20, 20), 2)
    a = gpu_all_ops(x, w, b, dy, **kw)
    c = gpu_all_ops(x, w, b, dy, **kw)
    for u, v in zip(a, c):
        assert torch.equal(u, v)


@pytest.mark.parametrize("name", ["tiny_grouped", "resnext_32x4d", "dense3x3", "dense3x3_nhwc", "fc_mode"])
def test_hip_graph_replay(name):
    """The four ops of a step captured in one HIP graph (prepared plans, no
    allocation or memset inside) and replayed several times, with eager work
    and synchronisations in between: every replay equals the eager results
    bit for bit. The channels-last workload captures its reorderings through
    the workspace as well."""
    wl = WORKLOADS[name]
    inp = make_inputs(name, batch=REDUCED_BATCH[name])
    kw = dict(wl_kwargs(wl), layout=wl.layout)
    store = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 3, 1))) if wl.layout == "nhwc" else (lambda a: a)
    x, w, dy = dev(store(inp["x"])), dev(inp["w"]), dev(store(inp["dy"]))
    b = None if inp["b"] is None else dev(inp["b"])
    N, K, Ho, Wo = (x.shape[0],) + tuple(wl.dy_shape[1:])
    y = torch.empty((N, Ho, Wo, K) if wl.layout == "nhwc" else (N, K, Ho, Wo), device="cuda")
    dx, dw = torch.empty_like(x), torch.empty_like(w)
    db = torch.empty(w.shape[0], device="cuda")
    plans = [G.Plan.fwd(x, w, b, y, **kw), G.Plan.bwd_data(dy, w, dx, **kw),
             G.Plan.bwd_filter(x, dy, dw, **kw), G.Plan.bwd_bias(dy, db, layout=wl.layout)]
    torch.cuda.synchronize()
    eager = [t.clone() for t in (y, dx, dw, db)]
    say("hip graph %s" % name)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        # plans run on the stream they were built on: rebuild them on the capture stream
        plans = [G.Plan.fwd(x, w, b, y, **kw), G.Plan.bwd_data(dy, w, dx, **kw),
                 G.Plan.bwd_filter(x, dy, dw, **kw), G.Plan.bwd_bias(dy, db, layout=wl.layout)]
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            for p in plans:
                p()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        for t in (y, dx, dw, db):
            t.fill_(float("nan"))           # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, e in zip((y, dx, dw, db), eager):
            assert torch.equal(t, e), (name, rep)


def test_guard_bands_untouched():
    """Outputs written into the middle of sentinel-filled buffers: no store
    lands outside the result (tile edges)."""
    d = dict(N=3, C=30, H=13, W=17, K=45, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=3)
    kw = conv_kwargs(d)
    x, w, b = tensors(d, 3)
    xd, wd, bd = dev(x), dev(w), dev(b)
    y_ref = G.gconv_fwd(xd, wd, bd, **kw)
    dyd = dev(draw(("normal", 1.0), tuple(y_ref.shape), 4))
    pad = 4096
    for path in [G.PATH_AUTO] + ALL_PATHS:
        G.gconv_set_path_override(path)
        try:
            for shape, fn in (
                    (tuple(y_ref.shape), lambda o: G.gconv_fwd(xd, wd, bd, out=o, **kw)),
                    (x.shape, lambda o: G.gconv_bwd_data(dyd, wd, x.shape, out=o, **kw)),
                    (w.shape, lambda o: G.gconv_bwd_filter(xd, dyd, w.shape, out=o, **kw)),
                    ((d["K"],), lambda o: G.gconv_bwd_bias(dyd, out=o))):
                n = int(np.prod(shape))
                buf = torch.full((n + 2 * pad,), 12345.0, device="cuda")
                try:
                    fn(buf[pad:pad + n].view(shape))
                except G.GconvError as e:
                    if e.status == 6:
                        continue
                    raise
                torch.cuda.synchronize()
                assert bool((buf[:pad] == 12345.0).all()) and bool((buf[pad + n:] == 12345.0).all())
        finally:
            G.gconv_set_path_override(G.PATH_AUTO)


def test_empty_batch_on_gpu():
    d = dict(N=0, C=8, H=6, W=6, K=4, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=2)
    kw = conv_kwargs(d)
    x = torch.zeros((0, 8, 6, 6), device="cuda")
    w = dev(tensors(d, 5)[1])
    dy = torch.zeros((0, 4, 6, 6), device="cuda")
    y = G.gconv_fwd(x, w, **kw)
    dx = G.gconv_bwd_data(dy, w, x.shape, **kw)
    dw = G.gconv_bwd_filter(x, dy, w.shape, out=torch.full(w.shape, 7.0, device="cuda"), **kw)
    db = G.gconv_bwd_bias(dy, out=torch.full((4,), 7.0, device="cuda"))
    torch.cuda.synchronize()
    assert y.shape == (0, 4, 6, 6) and dx.shape == (0, 8, 6, 6)
    assert bool((dw == 0).all()) and bool((db == 0).all())


def test_binding_rejects_bad_tensors():
    x = torch.zeros((2, 8, 5, 5), device="cuda")
    w = torch.zeros((4, 4, 3, 3), device="cuda")
    with pytest.raises(ValueError):
        G.gconv_fwd(x.double(), w, groups=2)
    with pytest.raises(ValueError):
        G.gconv_fwd(x.cpu(), w, groups=2)
    with pytest.raises(ValueError):
        G.gconv_fwd(x.transpose(2, 3), w, groups=2)
    with pytest.raises(ValueError):
        G.gconv_fwd(x, w, groups=3)
    with pytest.raises(ValueError):
        G.gconv_bwd_data(torch.zeros((2, 4, 4, 4), device="cuda"), w, x.shape, groups=2)


def test_c_abi_symbols_directly():
    """The four ops called through their own C symbols (gconv_fwd itself, not the
    binding's gconv_fwd_ex), with plain device pointers, a caller-owned workspace
    and torch's current stream, on a grouped descriptor whose gradWeight and
    gradBias use the workspace; every result against the oracle."""
    import ctypes
    from grouped_convolution_amd import binding as B
    lib = B.load()
    d = dict(N=3, C=32, K=48, H=13, W=11, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=2)
    kw = conv_kwargs(d)
    x, w, b = tensors(d, 3900)
    y_ref, _ = oracle.fwd(x, w, b, **kw)
    dy = draw(("normal", 1.0), y_ref.shape, 3903)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], **kw)
    ho, wo = ctypes.c_int64(), ctypes.c_int64()
    assert lib.gconv_output_dims(ctypes.byref(desc), ctypes.byref(ho), ctypes.byref(wo)) == 0
    assert (ho.value, wo.value) == y_ref.shape[2:]
    xd, wd, bd, dyd = dev(x), dev(w), dev(b), dev(dy)
    y = torch.empty(y_ref.shape, device="cuda")
    dx = torch.empty(x.shape, device="cuda")
    dw = torch.empty(w.shape, device="cuda")
    db = torch.empty((d["K"],), device="cuda")
    sizes = []
    for op in range(4):
        n = ctypes.c_size_t()
        assert lib.gconv_workspace_size(ctypes.byref(desc), op, ctypes.byref(n)) == 0
        sizes.append(n.value)
    ws = torch.empty(max(max(sizes) // 4, 1), device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    D = ctypes.byref(desc)
    say("raw C-ABI calls %s, workspaces %s" % (d, sizes))
    assert lib.gconv_fwd(D, P(xd), P(wd), P(bd), P(y), P(ws), ctypes.c_size_t(sizes[0]), st) == 0
    assert lib.gconv_bwd_data(D, P(dyd), P(wd), P(dx), P(ws), ctypes.c_size_t(sizes[1]), st) == 0
    assert lib.gconv_bwd_filter(D, P(xd), P(dyd), P(dw), P(ws), ctypes.c_size_t(sizes[2]), st) == 0
    assert lib.gconv_bwd_bias(D, P(dyd), P(db), P(ws), ctypes.c_size_t(sizes[3]), st) == 0
    assert lib.gconv_last_error() == b""
    torch.cuda.synchronize()
    compare_full("raw C ABI", (y, dx, dw, db), oracle_all(x, w, b, dy, kw))
    # gconv_fwd without a bias pointer
    assert lib.gconv_fwd(D, P(xd), P(wd), None, P(y), P(ws), ctypes.c_size_t(sizes[0]), st) == 0
    torch.cuda.synchronize()
    val, mag = oracle.fwd(x, w, None, **kw)
    check("raw gconv_fwd no bias", y.cpu().numpy(), val, mag)
