"""grouped_convolution_amd: grouped 2-D convolution (NCHW, fp32) on MI355X."""
