"""The allocation-free gradWeight entry point, gconv_bwd_filter_static, called
through the C ABI: its result equals gconv_bwd_filter's (same kernels, same
summation order, so bit for bit) on two calls in a row, the second with a
smaller input, on shapes whose gradWeight keeps split partials in its scratch;
a descriptor that needs more scratch than the static array holds is refused
before anything runs."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from cases import conv_kwargs, tensors
from gpu_util import say
from grouped_convolution_amd.workloads import draw

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import grouped_convolution_amd as G  # noqa: E402
from grouped_convolution_amd import binding as B  # noqa: E402

SCRATCH_BYTES = 64 << 20

# (descriptor, family the dispatcher picks): each gradWeight keeps split partials
# (or channels-last copies) in the scratch.
CASES = [
    (dict(N=8, C=64, K=64, H=28, W=28, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=1), "igemm", "nchw"),
    (dict(N=6, C=32, K=32, H=30, W=26, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=8), "smallgroup", "nchw"),
    (dict(N=4, C=64, K=48, H=20, W=20, kh=1, kw=1, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1), "pointwise", "nchw"),
    (dict(N=3, C=32, K=32, H=15, W=17, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=1), "igemm", "nhwc"),
    # fully-connected gradWeight in the balanced form (16 x 18 = 288 tiles over 300 images, then
    # 150): its split tiles' parts go through the array, the second call over fewer stages
    (dict(N=300, C=256, K=2048, H=3, W=3, kh=3, kw=3, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, G=1), "fc", "nchw"),
]


def _run(lib, d, layout, seed):
    kw = conv_kwargs(d)
    x, _, _ = tensors(d, seed, bias=False)
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], layout=layout, **kw)
    Ho, Wo = G.gconv_output_dims(desc)
    dy = draw(("normal", 1.0), (d["N"], d["K"], Ho, Wo), seed + 3)
    to = (lambda a: np.ascontiguousarray(a.transpose(0, 2, 3, 1))) if layout == "nhwc" else (lambda a: a)
    xd = torch.from_numpy(to(x)).cuda()
    dyd = torch.from_numpy(to(dy)).cuda()
    wshape = (d["K"], d["C"] // d["G"], d["kh"], d["kw"])
    want = G.gconv_bwd_filter(xd, dyd, wshape, layout=layout, **kw)
    got = torch.full(wshape, float("nan"), device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    status = lib.gconv_bwd_filter_static(ctypes.byref(desc), ctypes.c_void_p(xd.data_ptr()),
                                         ctypes.c_void_p(dyd.data_ptr()), ctypes.c_void_p(got.data_ptr()), st)
    assert status == 0, (status, lib.gconv_last_error())
    torch.cuda.synchronize()
    return got.cpu().numpy(), want.cpu().numpy(), G.gconv_workspace_size(desc, G.OP_BWD_FILTER)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_static_matches_workspace_entry_point(case):
    lib = B.load()
    d, family, layout = CASES[case]
    desc = G.make_desc(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], layout=layout, **conv_kwargs(d))
    assert G.PATH_NAMES[G.gconv_select_path(desc, G.OP_BWD_FILTER)] == family
    # a smaller second call (fully-connected mode keeps its kernel == input)
    small = dict(d, N=max(1, d["N"] // 2)) if family == "fc" else dict(d, N=max(1, d["N"] // 2), H=d["H"] - 3)
    for i, dd in enumerate((d, small)):
        say("no-alloc gradWeight %s %s call %d" % (layout, dd, i))
        got, want, nws = _run(lib, dd, layout, 4100 + 10 * case + i)
        assert 0 < nws <= SCRATCH_BYTES, nws
        assert np.array_equal(got, want), (dd, float(np.nanmax(np.abs(got - want))))


def test_static_refuses_more_than_its_scratch():
    lib = B.load()
    # channels-last 3x3 gradWeight: its two reordered copies alone take 2 x 38.5 MB
    desc = G.make_desc(48, 64, 56, 56, 64, 3, 3, padding=1, layout="nhwc")
    assert G.gconv_workspace_size(desc, G.OP_BWD_FILTER) > SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    status = lib.gconv_bwd_filter_static(ctypes.byref(desc), fake, ctypes.c_void_p(0x100000000),
                                         ctypes.c_void_p(0x200000000), None)
    assert status == 4  # GCONV_ERR_WORKSPACE, before any launch
    assert b"static scratch" in lib.gconv_last_error()
