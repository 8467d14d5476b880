"""ctypes binding of libgconv.so (the C ABI declared in include/gconv.h).

Argument marshalling only: tensors must already be float32, contiguous and on
the GPU; outputs and the workspace are allocated here with torch (device
memory is torch's), and every op is enqueued on torch's current HIP stream.
Nothing is computed in Python or by torch. When the library is missing the
first call raises; there is no fallback.

Names mirror the C entry points: gconv_fwd, gconv_bwd_data, gconv_bwd_filter,
gconv_bwd_bias, gconv_output_dims, gconv_workspace_size, gconv_select_path,
gconv_set_path_override.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgconv.so")

OK = 0
STATUS = {0: "GCONV_OK", 1: "GCONV_ERR_NULL", 2: "GCONV_ERR_SHAPE", 3: "GCONV_ERR_GROUPS",
          4: "GCONV_ERR_WORKSPACE", 5: "GCONV_ERR_HIP", 6: "GCONV_ERR_UNSUPPORTED",
          7: "GCONV_ERR_ARG"}
OP_FWD, OP_BWD_DATA, OP_BWD_FILTER, OP_BWD_BIAS = 0, 1, 2, 3
PATH_AUTO, PATH_DIRECT, PATH_SMALLGROUP, PATH_IGEMM, PATH_FC, PATH_POINTWISE = 0, 1, 2, 3, 4, 5
EPILOGUE_NONE, EPILOGUE_RELU = 0, 1
LAYOUT_NCHW, LAYOUT_NHWC = 0, 1
PATH_NAMES = {PATH_AUTO: "auto", PATH_DIRECT: "direct", PATH_SMALLGROUP: "smallgroup",
              PATH_IGEMM: "igemm", PATH_FC: "fc", PATH_POINTWISE: "pointwise"}

# Every symbol include/gconv.h declares.
EXPORTS = ("gconv_output_dims", "gconv_workspace_size", "gconv_fwd", "gconv_fwd_ex", "gconv_bwd_data",
           "gconv_bwd_filter", "gconv_bwd_filter_static", "gconv_bwd_bias", "gconv_select_path",
           "gconv_set_path_override", "gconv_status_string", "gconv_last_error", "gconv_version")


class GconvError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%s): %s" % (func, STATUS.get(status, status),
                                                     _status_string(status), detail))


class gconv_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "N", "C", "H", "W", "K", "kh", "kw", "stride_h", "stride_w", "pad_h", "pad_w",
        "dil_h", "dil_w", "groups", "pad_h_extra", "pad_w_extra", "layout")]


_lib = None


def load(path: str = LIB_PATH):
    """Load libgconv.so and declare its signatures (once per process)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libgconv.so is not built (expected at %s); run "
                           "`python -m grouped_convolution_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    D = ctypes.POINTER(gconv_desc)
    i64p = ctypes.POINTER(ctypes.c_int64)
    sig = {
        "gconv_output_dims": [D, i64p, i64p],
        "gconv_workspace_size": [D, I, ctypes.POINTER(ctypes.c_size_t)],
        "gconv_fwd": [D, P, P, P, P, P, S, P],
        "gconv_fwd_ex": [D, P, P, P, I, P, P, S, P],
        "gconv_bwd_data": [D, P, P, P, P, S, P],
        "gconv_bwd_filter": [D, P, P, P, P, S, P],
        "gconv_bwd_filter_static": [D, P, P, P, P],
        "gconv_bwd_bias": [D, P, P, P, S, P],
        "gconv_select_path": [D, I, ctypes.POINTER(ctypes.c_int)],
        "gconv_set_path_override": [I],
        "gconv_status_string": [I],
        "gconv_last_error": [],
        "gconv_version": [],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.gconv_status_string.restype = ctypes.c_char_p
    lib.gconv_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _status_string(status: int) -> str:
    return load().gconv_status_string(status).decode()


def _check(status: int, func: str):
    if status != OK:
        raise GconvError(status, func, load().gconv_last_error().decode())


def _pair(v, name):
    if isinstance(v, (tuple, list)):
        if len(v) != 2:
            raise ValueError("%s must be an int or a pair" % name)
        return int(v[0]), int(v[1])
    return int(v), int(v)


def _padding(v):
    """int, (pad_h, pad_w) or (top, bottom, left, right) -> (top, left, bottom - top, right - left)."""
    if isinstance(v, (tuple, list)) and len(v) == 4:
        t, b, l, r = (int(e) for e in v)
        return t, l, b - t, r - l
    ph, pw = _pair(v, "padding")
    return ph, pw, 0, 0


def same_padding(H, W, kh, kw, stride=1, dilation=1):
    """TensorFlow's "same" padding as (top, bottom, left, right): Ho = ceil(H / stride), the
    total padding split with the odd row or column at the end."""
    out = []
    for n, k, s, d in zip((H, W), (kh, kw), _pair(stride, "stride"), _pair(dilation, "dilation")):
        total = max((-(-n // s) - 1) * s + (k - 1) * d + 1 - n, 0)
        out += [total // 2, total - total // 2]
    return tuple(out)


def _layout(v) -> int:
    """"nchw" / "nhwc" (or LAYOUT_NCHW / LAYOUT_NHWC) -> gconv_layout."""
    if isinstance(v, str):
        key = v.lower()
        if key not in ("nchw", "nhwc"):
            raise ValueError("layout must be 'nchw' or 'nhwc', got %r" % v)
        return LAYOUT_NHWC if key == "nhwc" else LAYOUT_NCHW
    if int(v) not in (LAYOUT_NCHW, LAYOUT_NHWC):
        raise ValueError("unknown layout %r" % (v,))
    return int(v)


def make_desc(N, C, H, W, K, kh, kw, stride=1, padding=0, dilation=1, groups=1,
              layout="nchw") -> gconv_desc:
    """`padding` is an int, a pair (pad_h, pad_w) or a 4-tuple (top, bottom, left, right);
    `layout` ("nchw" or "nhwc") is that of x, dx, y and dy."""
    sh, sw = _pair(stride, "stride")
    ph, pw, eh, ew = _padding(padding)
    dh, dw = _pair(dilation, "dilation")
    return gconv_desc(int(N), int(C), int(H), int(W), int(K), int(kh), int(kw), sh, sw, ph, pw,
                      dh, dw, int(groups), eh, ew, _layout(layout))


def _act_shape(N, C, H, W, layout):
    """The 4-D shape of an activation with N images, C channels, H x W pixels."""
    return (N, H, W, C) if _layout(layout) == LAYOUT_NHWC else (N, C, H, W)


def _act_dims(shape, layout):
    """(N, C, H, W) of an activation tensor shape in `layout`."""
    N, a, b, c = (int(v) for v in shape)
    return (N, c, a, b) if _layout(layout) == LAYOUT_NHWC else (N, a, b, c)


def gconv_output_dims(desc: gconv_desc):
    ho, wo = ctypes.c_int64(), ctypes.c_int64()
    _check(load().gconv_output_dims(ctypes.byref(desc), ctypes.byref(ho), ctypes.byref(wo)),
           "gconv_output_dims")
    return ho.value, wo.value


def gconv_workspace_size(desc: gconv_desc, op: int) -> int:
    n = ctypes.c_size_t()
    _check(load().gconv_workspace_size(ctypes.byref(desc), int(op), ctypes.byref(n)),
           "gconv_workspace_size")
    return n.value


def gconv_select_path(desc: gconv_desc, op: int) -> int:
    p = ctypes.c_int()
    _check(load().gconv_select_path(ctypes.byref(desc), int(op), ctypes.byref(p)),
           "gconv_select_path")
    return p.value


def gconv_set_path_override(path: int):
    _check(load().gconv_set_path_override(int(path)), "gconv_set_path_override")


def version() -> int:
    return int(load().gconv_version())


# ---------------------------------------------------------------- tensor level

def _torch():
    import torch
    return torch


def _dev_f32(t, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.float32:
        raise ValueError("%s must be float32, got %s" % (name, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (row-major in its layout)" % name)
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(desc, op, device, workspace):
    n = gconv_workspace_size(desc, op)
    if n == 0:
        return None, 0
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < n:
            raise ValueError("workspace holds %d bytes, %d needed"
                             % (workspace.numel() * workspace.element_size(), n))
        return workspace, workspace.numel() * workspace.element_size()
    torch = _torch()
    return torch.empty(n, dtype=torch.uint8, device=device), n


def _out(out, shape, like, name):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=like.device)
    _dev_f32(out, name)
    if tuple(out.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(out.shape), tuple(shape)))
    return out


def gconv_fwd(x, w, bias=None, *, stride=1, padding=0, dilation=1, groups=1, out=None,
              workspace=None, relu=False, layout="nchw"):
    """y = conv(x, w) + bias; x [N,C,H,W] (or [N,H,W,C] with layout="nhwc", giving y
    [N,Ho,Wo,K]), w [K,C/groups,kh,kw], bias [K] or None.
    With relu=True the kernels store max(y, 0) (gconv_fwd_ex, GCONV_EPILOGUE_RELU)."""
    _dev_f32(x, "x")
    _dev_f32(w, "w")
    if x.dim() != 4 or w.dim() != 4:
        raise ValueError("x and w must be 4-D (NCHW or NHWC, and [K, C/groups, kh, kw])")
    N, C, H, W = _act_dims(x.shape, layout)
    K, Cg, kh, kw = w.shape
    if groups < 1 or C % groups or Cg * groups != C:
        raise ValueError("channels_in C=%d must equal w.shape[1]*groups = %d*%d"
                         % (C, Cg, groups))
    if bias is not None:
        _dev_f32(bias, "bias")
        if tuple(bias.shape) != (K,):
            raise ValueError("bias must have shape [K]=[%d]" % K)
    desc = make_desc(N, C, H, W, K, kh, kw, stride, padding, dilation, groups, layout)
    Ho, Wo = gconv_output_dims(desc)
    y = _out(out, _act_shape(N, K, Ho, Wo, layout), x, "out")
    ws, nws = _workspace(desc, OP_FWD, x.device, workspace)
    _check(load().gconv_fwd_ex(ctypes.byref(desc), _ptr(x), _ptr(w), _ptr(bias),
                               EPILOGUE_RELU if relu else EPILOGUE_NONE, _ptr(y), _ptr(ws), nws,
                               _stream(x.device)), "gconv_fwd_ex")
    return y


def gconv_bwd_data(dy, w, x_shape, *, stride=1, padding=0, dilation=1, groups=1, out=None,
                   workspace=None, layout="nchw"):
    """gradInput [N,C,H,W] from dy [N,K,Ho,Wo] and w [K,C/groups,kh,kw] (x_shape, dy and
    the result in `layout`)."""
    _dev_f32(dy, "dy")
    _dev_f32(w, "w")
    N, C, H, W = _act_dims(x_shape, layout)
    K, Cg, kh, kw = w.shape
    if groups < 1 or Cg * groups != C:
        raise ValueError("channels_in C=%d must equal w.shape[1]*groups = %d*%d"
                         % (C, Cg, groups))
    desc = make_desc(N, C, H, W, K, kh, kw, stride, padding, dilation, groups, layout)
    Ho, Wo = gconv_output_dims(desc)
    if tuple(dy.shape) != _act_shape(N, K, Ho, Wo, layout):
        raise ValueError("dy has shape %s, expected %s"
                         % (tuple(dy.shape), _act_shape(N, K, Ho, Wo, layout)))
    dx = _out(out, _act_shape(N, C, H, W, layout), dy, "out")
    ws, nws = _workspace(desc, OP_BWD_DATA, dy.device, workspace)
    _check(load().gconv_bwd_data(ctypes.byref(desc), _ptr(dy), _ptr(w), _ptr(dx), _ptr(ws), nws,
                                 _stream(dy.device)), "gconv_bwd_data")
    return dx


def gconv_bwd_filter(x, dy, w_shape, *, stride=1, padding=0, dilation=1, groups=1, out=None,
                     workspace=None, layout="nchw"):
    """gradWeight [K,C/groups,kh,kw] from x [N,C,H,W] and dy [N,K,Ho,Wo] (x and dy in
    `layout`; overwrites)."""
    _dev_f32(x, "x")
    _dev_f32(dy, "dy")
    N, C, H, W = _act_dims(x.shape, layout)
    K, Cg, kh, kw = (int(v) for v in w_shape)
    if groups < 1 or Cg * groups != C:
        raise ValueError("channels_in C=%d must equal w_shape[1]*groups = %d*%d"
                         % (C, Cg, groups))
    desc = make_desc(N, C, H, W, K, kh, kw, stride, padding, dilation, groups, layout)
    Ho, Wo = gconv_output_dims(desc)
    if tuple(dy.shape) != _act_shape(N, K, Ho, Wo, layout):
        raise ValueError("dy has shape %s, expected %s"
                         % (tuple(dy.shape), _act_shape(N, K, Ho, Wo, layout)))
    dw = _out(out, (K, Cg, kh, kw), x, "out")
    ws, nws = _workspace(desc, OP_BWD_FILTER, x.device, workspace)
    _check(load().gconv_bwd_filter(ctypes.byref(desc), _ptr(x), _ptr(dy), _ptr(dw), _ptr(ws),
                                   nws, _stream(x.device)), "gconv_bwd_filter")
    return dw


def gconv_bwd_bias(dy, *, out=None, workspace=None, layout="nchw"):
    """gradBias [K] = sum of dy [N,K,Ho,Wo] (or [N,Ho,Wo,K]) over (n, ho, wo) (overwrites)."""
    _dev_f32(dy, "dy")
    if dy.dim() != 4:
        raise ValueError("dy must be 4-D [N, K, Ho, Wo] or [N, Ho, Wo, K]")
    N, K, Ho, Wo = _act_dims(dy.shape, layout)
    # Only N, K, Ho, Wo matter: describe dy as the output of a 1x1 conv.
    desc = make_desc(N, K, Ho, Wo, K, 1, 1, layout=layout)
    db = _out(out, (K,), dy, "out")
    ws, nws = _workspace(desc, OP_BWD_BIAS, dy.device, workspace)
    _check(load().gconv_bwd_bias(ctypes.byref(desc), _ptr(dy), _ptr(db), _ptr(ws), nws,
                                 _stream(dy.device)), "gconv_bwd_bias")
    return db


class Plan:
    """One op with its arguments marshalled once, for repeated launches.

    ``Plan.fwd(x, w, bias, y, ...)`` etc. validate exactly like the functions
    above and keep the ctypes argument tuple; calling the plan enqueues the op
    on the stream it was built with and checks the status. The tensors must
    stay alive (and keep their storage) as long as the plan is used."""

    def __init__(self, fn_name, args, keep):
        self._fn = getattr(load(), fn_name)
        self._name = fn_name
        self._args = args
        self._keep = keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != OK:
            _check(st, self._name)

    @staticmethod
    def _prep(desc, op, device, workspace):
        ws, nws = _workspace(desc, op, device, workspace)
        return ws, nws, _stream(device)

    @classmethod
    def fwd(cls, x, w, bias, y, *, stride=1, padding=0, dilation=1, groups=1, workspace=None,
            relu=False, layout="nchw"):
        gconv_fwd(x, w, bias, stride=stride, padding=padding, dilation=dilation, groups=groups,
                  out=y, workspace=workspace, relu=relu, layout=layout)  # validates (and runs) once
        N, C, H, W = _act_dims(x.shape, layout)
        K, _, kh, kw = w.shape
        desc = make_desc(N, C, H, W, K, kh, kw, stride, padding, dilation, groups, layout)
        ws, nws, st = cls._prep(desc, OP_FWD, x.device, workspace)
        act = EPILOGUE_RELU if relu else EPILOGUE_NONE
        return cls("gconv_fwd_ex", (ctypes.byref(desc), _ptr(x), _ptr(w), _ptr(bias), act, _ptr(y),
                                    _ptr(ws), nws, st), (desc, x, w, bias, y, ws))

    @classmethod
    def bwd_data(cls, dy, w, dx, *, stride=1, padding=0, dilation=1, groups=1, workspace=None,
                 layout="nchw"):
        gconv_bwd_data(dy, w, dx.shape, stride=stride, padding=padding, dilation=dilation,
                       groups=groups, out=dx, workspace=workspace, layout=layout)
        N, C, H, W = _act_dims(dx.shape, layout)
        K, _, kh, kw = w.shape
        desc = make_desc(N, C, H, W, K, kh, kw, stride, padding, dilation, groups, layout)
        ws, nws, st = cls._prep(desc, OP_BWD_DATA, dy.device, workspace)
        return cls("gconv_bwd_data", (ctypes.byref(desc), _ptr(dy), _ptr(w), _ptr(dx), _ptr(ws),
                                      nws, st), (desc, dy, w, dx, ws))

    @classmethod
    def bwd_filter(cls, x, dy, dw, *, stride=1, padding=0, dilation=1, groups=1,
                   workspace=None, layout="nchw"):
        gconv_bwd_filter(x, dy, dw.shape, stride=stride, padding=padding, dilation=dilation,
                         groups=groups, out=dw, workspace=workspace, layout=layout)
        N, C, H, W = _act_dims(x.shape, layout)
        K, _, kh, kw = dw.shape
        desc = make_desc(N, C, H, W, K, kh, kw, stride, padding, dilation, groups, layout)
        ws, nws, st = cls._prep(desc, OP_BWD_FILTER, x.device, workspace)
        return cls("gconv_bwd_filter", (ctypes.byref(desc), _ptr(x), _ptr(dy), _ptr(dw),
                                        _ptr(ws), nws, st), (desc, x, dy, dw, ws))

    @classmethod
    def bwd_bias(cls, dy, db, *, workspace=None, layout="nchw"):
        gconv_bwd_bias(dy, out=db, workspace=workspace, layout=layout)
        N, K, Ho, Wo = _act_dims(dy.shape, layout)
        desc = make_desc(N, K, Ho, Wo, K, 1, 1, layout=layout)
        ws, nws, st = cls._prep(desc, OP_BWD_BIAS, dy.device, workspace)
        return cls("gconv_bwd_bias", (ctypes.byref(desc), _ptr(dy), _ptr(db), _ptr(ws), nws, st),
                   (desc, dy, db, ws))
