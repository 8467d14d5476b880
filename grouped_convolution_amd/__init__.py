"""grouped_convolution_amd: grouped 2-D convolution (NCHW or NHWC, float32) for AMD MI355X.

The compute path is libgconv.so: hand-written HIP kernels for gfx950 behind
the C ABI in include/gconv.h. This package is its thin Python binding
(``binding``), its in-tree build (``build``), and seeded synthetic inputs
(``workloads``). Importing the package loads nothing; the first op call loads
the library and raises if it is missing.
"""
from .binding import (GconvError, Plan, LAYOUT_NCHW, LAYOUT_NHWC, OP_BWD_BIAS, OP_BWD_DATA, OP_BWD_FILTER, OP_FWD, PATH_AUTO,
                      PATH_DIRECT, PATH_FC, PATH_IGEMM, PATH_NAMES, PATH_POINTWISE, PATH_SMALLGROUP, gconv_bwd_bias,
                      gconv_bwd_data, gconv_bwd_filter, gconv_desc, gconv_fwd, gconv_output_dims,
                      gconv_select_path, gconv_set_path_override, gconv_workspace_size, make_desc,
                      same_padding)

__all__ = ["GconvError", "Plan", "gconv_desc", "make_desc", "gconv_fwd", "gconv_bwd_data",
           "gconv_bwd_filter", "gconv_bwd_bias", "gconv_output_dims", "gconv_workspace_size",
           "gconv_select_path", "gconv_set_path_override", "OP_FWD", "OP_BWD_DATA",
           "OP_BWD_FILTER", "OP_BWD_BIAS", "PATH_AUTO", "PATH_DIRECT", "PATH_SMALLGROUP",
           "PATH_IGEMM", "PATH_FC", "PATH_POINTWISE", "PATH_NAMES", "same_padding", "LAYOUT_NCHW",
           "LAYOUT_NHWC"]
