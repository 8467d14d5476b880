/*
 * gconv.h -- C ABI of the grouped 2-D convolution library for AMD MI355X
 * (gfx950). Channels-first (NCHW) float32.
 *
 * The operation ("[Feature request] Groups support for SpatialConvolutionMM",
 * the opening definition of groups): the C input planes and the K output
 * planes are each split into `groups` contiguous blocks, and output block g
 * is computed from input block g only. With Cg = C/groups and Kg = K/groups:
 *
 *   y[n,k,ho,wo] = bias[k] + sum_{c<Cg, i<kh, j<kw}
 *                  w[k,c,i,j] * x[n, g*Cg + c, ho*stride_h - pad_h + i*dil_h,
 *                                               wo*stride_w - pad_w + j*dil_w]
 *
 * with g = k / Kg, x read as 0 outside [0,H) x [0,W) (zero padding), and no
 * kernel flip (cross-correlation: a kernel-sized input gives exactly the
 * Linear layer on the flattened input, as "SpatialConvolution running in
 * fully-connected mode is very slow, even with R4" relies on).
 *
 * Tensor layouts (all dense, row-major, float32, device memory):
 *   x, dx  [N, C, H, W]
 *   w, dw  [K, C/groups, kh, kw]    (K * C/groups filter planes)
 *   bias, db [K]
 *   y, dy  [N, K, Ho, Wo],  Ho = floor((H + pad_h + pad_h_end - dil_h*(kh-1) - 1)/stride_h) + 1
 *                           (likewise Wo), pad_h_end = pad_h + pad_h_extra
 * or, with layout = GCONV_LAYOUT_NHWC (channels last, the layout the
 * DLPrimitives Blog measures oneDNN fastest in), x, dx [N, H, W, C] and
 * y, dy [N, Ho, Wo, K]; w, dw and the bias keep their layouts.
 *
 * Ownership and execution. The caller owns every buffer; the library never
 * allocates device memory. Every op is enqueued on the caller's HIP stream
 * (`stream` is a hipStream_t; NULL means the default stream) and returns once
 * its kernels are enqueued. Inputs are read only. Outputs are overwritten in
 * full (gradWeight and gradBias are not accumulated into); outputs must not
 * overlap any input. Results are deterministic: the same inputs on the same
 * device give bit-identical outputs (no floating-point atomics).
 *
 * Empty batch. N == 0 is valid: forward and gradInput write nothing, and
 * gradWeight and gradBias are set to 0 (sums over no images). Pointers to
 * tensors with no elements may be NULL.
 *
 * Errors. Every function returns a gconv_status. Descriptor and argument
 * errors are detected on the host before anything is enqueued, and nothing
 * is written. GCONV_ERR_HIP reports a failed launch. gconv_last_error()
 * gives a readable detail of the calling thread's last failure (e.g. which
 * dimension does not divide by groups).
 */
#ifndef GCONV_H
#define GCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Convolution descriptor. K is the total number of output planes, not the
 * per-group count. The fields follow the constructor the clnn issue quotes
 * (nInputPlane, nOutputPlane, kW, kH, dW, dH, padW, padH, groups), plus
 * batch, input extent and dilation. Valid when N >= 0, C,H,W,K,kh,kw >= 1,
 * stride >= 1, dil >= 1, pad >= 0, pad + pad_extra >= 0, groups >= 1,
 * layout a gconv_layout,
 * C % groups == 0, K % groups == 0 and Ho, Wo >= 1 ("Support groups in
 * DenseConvDims": the channel counts must agree with the tensors and with the
 * group split).
 *
 * Asymmetric padding (DLPrimitives Blog, "TensorFlow": TensorFlow's "same"
 * padding can put one more zero row or column at the end of an axis than at
 * its start, which cuDNN cannot express). pad_h / pad_w are the zero rows at
 * the top and columns at the left; the bottom and right get pad_h +
 * pad_h_extra and pad_w + pad_w_extra. The end padding only sets Ho and Wo;
 * no padded copy of x is made. A zero-initialised pad_*_extra gives the
 * symmetric padding of the formula above.
 */
typedef struct gconv_desc {
    int64_t N, C, H, W;
    int64_t K;
    int64_t kh, kw;
    int64_t stride_h, stride_w;
    int64_t pad_h, pad_w;
    int64_t dil_h, dil_w;
    int64_t groups;
    int64_t pad_h_extra, pad_w_extra;  /* end padding minus start padding (0: symmetric) */
    int64_t layout;                    /* gconv_layout of x, dx, y, dy (0: NCHW) */
} gconv_desc;

/*
 * Activation layout. NHWC: a 1x1 stride-1 unpadded layer with one group is
 * one GEMM over the N*H*W rows (the fully-connected path, no reordering);
 * gradBias sums the [N*Ho*Wo, K] rows of dy directly; depthwise layers (one
 * channel per group, 3x3 or 5x5) run on channels-last kernels of their own
 * (gradWeight there when C % 4 == 0 and no family is forced; x and dy that
 * are not 16-byte aligned take 4-byte loads). Every other NHWC op
 * reorders its NHWC inputs to NCHW in the workspace, runs the NCHW kernels
 * there and reorders the NHWC outputs back (the MFMA implicit-GEMM forward
 * and gradInput store y and dx channels-last themselves), so
 * gconv_workspace_size() then includes those copies (x and y for the forward
 * pass, dy and dx for gradInput, x and dy for gradWeight).
 */
typedef enum gconv_layout {
    GCONV_LAYOUT_NCHW = 0,
    GCONV_LAYOUT_NHWC = 1
} gconv_layout;

typedef enum gconv_status {
    GCONV_OK = 0,
    GCONV_ERR_NULL = 1,        /* a required pointer is NULL */
    GCONV_ERR_SHAPE = 2,       /* a dimension < 1, a bad stride/pad/dilation, or Ho/Wo < 1 */
    GCONV_ERR_GROUPS = 3,      /* C or K not divisible by groups */
    GCONV_ERR_WORKSPACE = 4,   /* workspace smaller than gconv_workspace_size(), or misaligned */
    GCONV_ERR_HIP = 5,         /* a HIP runtime call or kernel launch failed */
    GCONV_ERR_UNSUPPORTED = 6, /* valid descriptor the forced path cannot run */
    GCONV_ERR_ARG = 7          /* other bad argument, e.g. an output overlapping an input */
} gconv_status;

typedef enum gconv_op {
    GCONV_OP_FWD = 0,
    GCONV_OP_BWD_DATA = 1,
    GCONV_OP_BWD_FILTER = 2,
    GCONV_OP_BWD_BIAS = 3
} gconv_op;

/* Kernel families the dispatcher routes between. */
typedef enum gconv_path {
    GCONV_PATH_AUTO = 0,       /* the dispatcher's own choice (default) */
    GCONV_PATH_DIRECT = 1,     /* general direct kernels: any valid descriptor */
    GCONV_PATH_SMALLGROUP = 2, /* few channels per group: HBM-bound 4x4x1-MFMA kernels */
    GCONV_PATH_IGEMM = 3,      /* fp32-MFMA implicit GEMM, groups in the grid */
    GCONV_PATH_FC = 4,         /* kernel == input: plain fp32-MFMA GEMM */
    GCONV_PATH_POINTWISE = 5   /* 1x1, stride 1, no padding: one fp32-MFMA GEMM per
                                  (image, group), gradWeight split over images */
} gconv_path;

/*
 * Output extent of the descriptor: the floor rule above, which fits every
 * shape the pages print ("Support groups in DenseConvDims": a 3x3 kernel
 * takes the 28x28 grouped benchmark input to 26x26; "SpatialConvolution
 * running in fully-connected mode is very slow, even with R4": a 6x6 kernel
 * on a 6x6 input gives the 1x1 output MatConvNet's gradient shape shows).
 * Writes *Ho and *Wo and returns GCONV_OK, or returns the descriptor's error
 * status (GCONV_ERR_SHAPE when the dilated kernel exceeds the padded input)
 * and writes nothing. Host only; launches nothing.
 */
int gconv_output_dims(const gconv_desc* d, int64_t* Ho, int64_t* Wo);

/*
 * Bytes of device workspace `op` (a gconv_op) needs for this descriptor (0
 * when none), written to *bytes. Pass at least this much to the op, 16-byte
 * aligned (GCONV_ERR_WORKSPACE otherwise); the workspace may be NULL when 0.
 * The contents need no initialisation and are scratch after the call. The
 * size comes back through *bytes so that an invalid descriptor or op can
 * return its status (GCONV_ERR_SHAPE, GCONV_ERR_GROUPS, GCONV_ERR_ARG) rather
 * than a size a caller might allocate. Host only.
 */
int gconv_workspace_size(const gconv_desc* d, int op, size_t* bytes);

/*
 * Forward pass (updateOutput in the clnn issue): y = conv(x, w) + bias.
 * `bias` may be NULL (no bias); otherwise bias[k] is added to every element
 * of output plane k (DLPrimitives Blog, "Pointwise Broadcast Reduce": the
 * [C] bias broadcast over [B,C,H,W]). One launch covers every group.
 */
int gconv_fwd(const gconv_desc* d, const float* x, const float* w, const float* bias, float* y,
              void* workspace, size_t workspace_bytes, void* stream);

/* Element-wise activations the forward pass can apply in its epilogue. */
typedef enum gconv_epilogue {
    GCONV_EPILOGUE_NONE = 0,   /* y = conv(x, w) + bias */
    GCONV_EPILOGUE_RELU = 1    /* y = max(conv(x, w) + bias, 0); NaN becomes 0 */
} gconv_epilogue;

/*
 * Forward pass with an element-wise activation applied to each output as it
 * is stored, after the bias (DLPrimitives Blog, "Pointwise Broadcast Reduce":
 * element-wise operations over the conv's output, broadcast over [B,C,H,W]),
 * so the activation costs no extra pass over y. Same arguments as gconv_fwd
 * plus `epilogue`, a gconv_epilogue; any other value is GCONV_ERR_ARG.
 * gconv_fwd is gconv_fwd_ex with GCONV_EPILOGUE_NONE.
 */
int gconv_fwd_ex(const gconv_desc* d, const float* x, const float* w, const float* bias, int epilogue,
                 float* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gradInput (updateGradInput in the clnn issue): dx = d<y,dy>/dx, the exact
 * adjoint of the forward map. dx[n, g*Cg+c, h, w] sums w[k,c,i,j] *
 * dy[n,k,ho,wo] over the k of group g and the taps (i, j) whose window
 * position (ho, wo) reads (h, w); input pixels no window reads get 0.
 */
int gconv_bwd_data(const gconv_desc* d, const float* dy, const float* w, float* dx,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * gradWeight (the weight half of accGradParameters in the clnn issue):
 * dw[k,c,i,j] = sum_{n,ho,wo} dy[n,k,ho,wo] * x[n, g*Cg+c, h(ho,i), w(wo,j)].
 * Overwrites dw. Uses the workspace for split reductions.
 */
int gconv_bwd_filter(const gconv_desc* d, const float* x, const float* dy, float* dw,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * gradWeight without a workspace argument and without allocating, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Same arguments, results
 * and errors as gconv_bwd_filter, whose kernels it runs; what that call keeps
 * in the workspace (split partials, channels-last copies) goes to a static
 * device array of 64 MiB instead, one per device, held until the process
 * ends. A descriptor that needs more (gconv_workspace_size) returns
 * GCONV_ERR_WORKSPACE before anything is enqueued. The stream must belong to
 * the current device (GCONV_ERR_ARG otherwise); the array's device address is
 * looked up on the first call on each device. Nothing in the array needs to
 * start at zero: every call writes what it reads. All calls on one device
 * share the array, so calls that overlap on one device (concurrent streams,
 * or threads) race and give wrong results; serialise them.
 */
int gconv_bwd_filter_static(const gconv_desc* d, const float* x, const float* dy, float* dw, void* stream);

/*
 * gradBias: db[k] = sum_{n,ho,wo} dy[n,k,ho,wo] (DLPrimitives Blog,
 * "Pointwise Broadcast Reduce": the sum of dy over dims 0, 2 and 3).
 * Only N, K, Ho, Wo and the layout of the descriptor matter. Overwrites db.
 */
int gconv_bwd_bias(const gconv_desc* d, const float* dy, float* db, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Kernel family the dispatcher would run `op` on for this descriptor
 * (gradBias is one reduction for every shape and reports GCONV_PATH_DIRECT).
 */
int gconv_select_path(const gconv_desc* d, int op, int* path);

/*
 * Force every later call in this process onto one kernel family (for
 * cross-checking each family against the others); GCONV_PATH_AUTO restores
 * the dispatcher's choice. A forced family that cannot run a descriptor
 * makes that call return GCONV_ERR_UNSUPPORTED. Not meant for concurrent use.
 */
int gconv_set_path_override(int path);

const char* gconv_status_string(int status);

/*
 * Readable detail of the calling thread's last failed call, "" after a call
 * that succeeded ("Support groups in DenseConvDims" adds a channel check so
 * that a bad group split gets a clear message: here, e.g., "input channels
 * C=10 not divisible by groups=3"). The string is owned by the library and
 * stays valid until the thread's next call into it.
 */
const char* gconv_last_error(void);

/* Library version: major*10000 + minor*100 + patch. */
int gconv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GCONV_H */
