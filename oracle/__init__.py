"""CPU fp64 oracle for grouped 2-D convolution (NCHW).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library
(``grouped_convolution_amd``) never imports it and shares no code with it.

The arithmetic lives in ``gconv_oracle.c`` (plain C, fp64 direct loops written
as gathers, one loop nest per op). This module only marshals numpy arrays:
inputs of any real dtype are promoted to float64 (exact for float32), and each
call returns ``(value, A)`` where ``A`` holds, per element, the sum of
|product| over that element's reduction (plus |bias| in the forward pass).

Ops (names follow the Torch module passes the pages discuss):
  fwd(x, w, b)            -> y        ("[Feature request] Groups support for
                                         SpatialConvolutionMM": updateOutput)
  bwd_data(dy, w, ...)    -> gradInput   (updateGradInput)
  bwd_filter(x, dy, ...)  -> gradWeight  (accGradParameters, weight part)
  bwd_bias(dy)            -> gradBias    (DLPrimitives Blog, "Pointwise
                                          Broadcast Reduce": sum over 0,2,3)
  fwd(..., relu=True)     -> max(y, 0)   (an element-wise operation on the
                                          forward output, the same section)

``padding`` is an int, a pair (pad_h, pad_w), or (top, bottom, left, right):
the end padding may differ from the start (DLPrimitives Blog, "TensorFlow").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gconv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgconv_oracle.so")

__all__ = ["build", "bind", "output_dims", "fwd", "bwd_data", "bwd_filter", "bwd_bias",
           "num_threads", "OracleError"]


class OracleError(ValueError):
    pass


class _Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "N", "C", "H", "W", "K", "kh", "kw",
        "stride_h", "stride_w", "pad_h", "pad_w", "dil_h", "dil_w", "groups",
        "pad_h_end", "pad_w_end")]


def build(force: bool = True) -> str:
    """Compile gconv_oracle.c with gcc into libgconv_oracle.so (next to it)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def bind(lib):
    """Declare the C signatures on a loaded oracle library and return it."""
    p_d = ctypes.POINTER(ctypes.c_double)
    p_i = ctypes.POINTER(ctypes.c_int64)
    p_desc = ctypes.POINTER(_Desc)
    lib.oracle_output_dims.argtypes = [p_desc, p_i, p_i]
    lib.oracle_fwd.argtypes = [p_desc, p_d, p_d, p_d, p_i, ctypes.c_int64, p_d, p_d]
    lib.oracle_bwd_data.argtypes = [p_desc, p_d, p_d, p_i, ctypes.c_int64, p_d, p_d]
    lib.oracle_bwd_filter.argtypes = [p_desc, p_d, p_d, p_i, ctypes.c_int64, p_d, p_d]
    lib.oracle_bwd_bias.argtypes = [p_desc, p_d, p_i, ctypes.c_int64, p_d, p_d]
    lib.oracle_num_threads.argtypes = []
    for f in ("oracle_output_dims", "oracle_fwd", "oracle_bwd_data",
              "oracle_bwd_filter", "oracle_bwd_bias", "oracle_num_threads"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle runs on (OMP_NUM_THREADS, else all cores)."""
    return int(_load().oracle_num_threads())


def _pair(v):
    if isinstance(v, (tuple, list)):
        if len(v) != 2:
            raise OracleError("expected an int or a pair, got %r" % (v,))
        return int(v[0]), int(v[1])
    return int(v), int(v)


def _pads(padding):
    """int, (pad_h, pad_w), or (top, bottom, left, right) -> (top, left, bottom, right)."""
    if isinstance(padding, (tuple, list)) and len(padding) == 4:
        t, b, l, r = (int(v) for v in padding)
        return t, l, b, r
    ph, pw = _pair(padding)
    return ph, pw, ph, pw


def _desc(N, C, H, W, K, kh, kw, stride, padding, dilation, groups) -> _Desc:
    sh, sw = _pair(stride)
    ph, pw, pb, pr = _pads(padding)
    dh, dw = _pair(dilation)
    return _Desc(N, C, H, W, K, kh, kw, sh, sw, ph, pw, dh, dw, int(groups), pb, pr)


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, kind=ctypes.c_double):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(kind))


def output_dims(N, C, H, W, K, kh, kw, stride=1, padding=0, dilation=1, groups=1):
    """(Ho, Wo), or OracleError for an invalid descriptor."""
    d = _desc(N, C, H, W, K, kh, kw, stride, padding, dilation, groups)
    ho, wo = ctypes.c_int64(), ctypes.c_int64()
    rc = _load().oracle_output_dims(ctypes.byref(d), ctypes.byref(ho), ctypes.byref(wo))
    if rc != 0:
        raise OracleError("invalid descriptor (code %d)" % rc)
    return ho.value, wo.value


def _run(fn, d, arrays, shape, idx):
    if idx is None:
        count = int(np.prod(shape))
        idx_arr = None
    else:
        idx_arr = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).ravel())
        count = idx_arr.size
    val = np.empty(count, np.float64)
    mag = np.empty(count, np.float64)
    rc = fn(ctypes.byref(d), *[_ptr(a) for a in arrays], _ptr(idx_arr, ctypes.c_int64),
            count, _ptr(val), _ptr(mag))
    if rc != 0:
        raise OracleError("oracle call failed (code %d)" % rc)
    if idx is None:
        return val.reshape(shape), mag.reshape(shape)
    return val, mag


def fwd(x, w, b=None, *, stride=1, padding=0, dilation=1, groups=1, idx=None, relu=False):
    """y = conv(x, w) + b. x [N,C,H,W], w [K,C/G,kh,kw], b [K] or None.

    With ``idx`` (flat indices into y), only those elements are computed. With
    ``relu``, y is replaced by max(y, 0) after the bias (NaN gives 0); A is
    unchanged (the activation adds no rounding)."""
    x, w = _f64(x), _f64(w)
    b = None if b is None else _f64(b)
    N, C, H, W = x.shape
    K, Cg, kh, kw = w.shape
    if Cg * int(groups) != C:
        raise OracleError("w.shape[1]*groups must equal C")
    if b is not None and b.shape != (K,):
        raise OracleError("bias must have shape [K]")
    d = _desc(N, C, H, W, K, kh, kw, stride, padding, dilation, groups)
    Ho, Wo = output_dims(N, C, H, W, K, kh, kw, stride, padding, dilation, groups)
    y, a = _run(_load().oracle_fwd, d, [x, w, b], (N, K, Ho, Wo), idx)
    if relu:
        y = np.where(y > 0.0, y, 0.0)
    return y, a


def bwd_data(dy, w, x_shape, *, stride=1, padding=0, dilation=1, groups=1, idx=None):
    """gradInput [N,C,H,W] from dy [N,K,Ho,Wo] and w [K,C/G,kh,kw]."""
    dy, w = _f64(dy), _f64(w)
    N, C, H, W = (int(s) for s in x_shape)
    K, Cg, kh, kw = w.shape
    if Cg * int(groups) != C:
        raise OracleError("w.shape[1]*groups must equal C")
    d = _desc(N, C, H, W, K, kh, kw, stride, padding, dilation, groups)
    Ho, Wo = output_dims(N, C, H, W, K, kh, kw, stride, padding, dilation, groups)
    if dy.shape != (N, K, Ho, Wo):
        raise OracleError("dy has shape %r, expected %r" % (dy.shape, (N, K, Ho, Wo)))
    return _run(_load().oracle_bwd_data, d, [dy, w], (N, C, H, W), idx)


def bwd_filter(x, dy, w_shape, *, stride=1, padding=0, dilation=1, groups=1, idx=None):
    """gradWeight [K,C/G,kh,kw] from x [N,C,H,W] and dy [N,K,Ho,Wo]."""
    x, dy = _f64(x), _f64(dy)
    N, C, H, W = x.shape
    K, Cg, kh, kw = (int(s) for s in w_shape)
    if Cg * int(groups) != C:
        raise OracleError("w_shape[1]*groups must equal C")
    d = _desc(N, C, H, W, K, kh, kw, stride, padding, dilation, groups)
    Ho, Wo = output_dims(N, C, H, W, K, kh, kw, stride, padding, dilation, groups)
    if dy.shape != (N, K, Ho, Wo):
        raise OracleError("dy has shape %r, expected %r" % (dy.shape, (N, K, Ho, Wo)))
    return _run(_load().oracle_bwd_filter, d, [x, dy], (K, Cg, kh, kw), idx)


def bwd_bias(dy, idx=None):
    """gradBias [K] = sum of dy [N,K,Ho,Wo] over (n, ho, wo)."""
    dy = _f64(dy)
    N, K, Ho, Wo = dy.shape
    # The reduction needs only dy's shape: describe it as a 1x1 conv of a
    # [N,K,Ho,Wo] input, whose output extent is (Ho, Wo).
    d = _desc(N, K, Ho, Wo, K, 1, 1, 1, 0, 1, 1)
    return _run(_load().oracle_bwd_bias, d, [dy], (K,), idx)
