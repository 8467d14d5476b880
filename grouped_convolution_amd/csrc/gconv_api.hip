// gconv_api.hip -- the C ABI (include/gconv.h): descriptor validation, output
// extents, routing between kernel families, workspace sizing and error
// reporting. Everything here runs on the host; kernels live in the other
// translation units.
#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "gconv.h"
#include "gconv_internal.h"

namespace gconv {
namespace {

thread_local std::string g_last_error;
std::atomic<int> g_path_override{GCONV_PATH_AUTO};

int fail(int status, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

// Output extent with p0 zero rows before the input and p1 after it.
int64_t out_extent(int64_t in, int64_t k, int64_t s, int64_t p0, int64_t p1, int64_t d)
{
    const int64_t num = in + p0 + p1 - d * (k - 1) - 1;
    return num < 0 ? 0 : num / s + 1;
}

constexpr int64_t kMaxDim = (int64_t)1 << 30;

// Check the descriptor ("Support groups in DenseConvDims": channel counts
// must agree with the group split, with a clear message when they do not)
// and derive the shape every kernel uses.
int make_shape(const gconv_desc* d, Shape* s)
{
    if (!d) return fail(GCONV_ERR_NULL, "descriptor is NULL");
    if (d->N < 0 || d->C < 1 || d->H < 1 || d->W < 1 || d->K < 1 || d->kh < 1 || d->kw < 1)
        return fail(GCONV_ERR_SHAPE,
                    "need N>=0 and C,H,W,K,kh,kw>=1 (got N=%lld C=%lld H=%lld W=%lld K=%lld "
                    "kh=%lld kw=%lld)",
                    (long long)d->N, (long long)d->C, (long long)d->H, (long long)d->W,
                    (long long)d->K, (long long)d->kh, (long long)d->kw);
    if (d->stride_h < 1 || d->stride_w < 1 || d->dil_h < 1 || d->dil_w < 1 || d->pad_h < 0 ||
        d->pad_w < 0)
        return fail(GCONV_ERR_SHAPE, "need stride>=1, dilation>=1, pad>=0");
    if (d->pad_h_extra < -kMaxDim || d->pad_h_extra > kMaxDim || d->pad_w_extra < -kMaxDim ||
        d->pad_w_extra > kMaxDim)
        return fail(GCONV_ERR_UNSUPPORTED, "a padding exceeds 2^30");
    const int64_t pad_h_end = d->pad_h + d->pad_h_extra, pad_w_end = d->pad_w + d->pad_w_extra;
    if (pad_h_end < 0 || pad_w_end < 0)
        return fail(GCONV_ERR_SHAPE, "end padding pad+pad_extra must be >= 0 (got %lld, %lld)",
                    (long long)pad_h_end, (long long)pad_w_end);
    if (d->layout != GCONV_LAYOUT_NCHW && d->layout != GCONV_LAYOUT_NHWC)
        return fail(GCONV_ERR_ARG, "unknown layout %lld", (long long)d->layout);
    if (d->groups < 1) return fail(GCONV_ERR_GROUPS, "groups=%lld must be >= 1",
                                   (long long)d->groups);
    if (d->C % d->groups != 0)
        return fail(GCONV_ERR_GROUPS, "input channels C=%lld not divisible by groups=%lld",
                    (long long)d->C, (long long)d->groups);
    if (d->K % d->groups != 0)
        return fail(GCONV_ERR_GROUPS, "output channels K=%lld not divisible by groups=%lld",
                    (long long)d->K, (long long)d->groups);
    const int64_t dims[] = {d->N, d->C, d->H, d->W, d->K, d->kh, d->kw, d->stride_h,
                            d->stride_w, d->pad_h, d->pad_w, d->dil_h, d->dil_w,
                            pad_h_end, pad_w_end};
    for (int64_t v : dims)
        if (v > kMaxDim) return fail(GCONV_ERR_UNSUPPORTED, "a dimension exceeds 2^30");
    const int64_t Ho = out_extent(d->H, d->kh, d->stride_h, d->pad_h, pad_h_end, d->dil_h);
    const int64_t Wo = out_extent(d->W, d->kw, d->stride_w, d->pad_w, pad_w_end, d->dil_w);
    if (Ho < 1 || Wo < 1)
        return fail(GCONV_ERR_SHAPE,
                    "empty output: the dilated kernel (%lldx%lld) exceeds the padded input",
                    (long long)(d->dil_h * (d->kh - 1) + 1), (long long)(d->dil_w * (d->kw - 1) + 1));
    s->N = (int)d->N; s->C = (int)d->C; s->H = (int)d->H; s->W = (int)d->W; s->K = (int)d->K;
    s->kh = (int)d->kh; s->kw = (int)d->kw;
    s->sh = (int)d->stride_h; s->sw = (int)d->stride_w;
    s->ph = (int)d->pad_h; s->pw = (int)d->pad_w;
    s->ph_end = (int)pad_h_end; s->pw_end = (int)pad_w_end;
    s->dh = (int)d->dil_h; s->dw = (int)d->dil_w;
    s->G = (int)d->groups; s->Cg = (int)(d->C / d->groups); s->Kg = (int)(d->K / d->groups);
    s->Ho = (int)Ho; s->Wo = (int)Wo;
    s->nhwc = d->layout == GCONV_LAYOUT_NHWC;
    s->x_elems = d->N * d->C * d->H * d->W;
    s->w_elems = d->K * (d->C / d->groups) * d->kh * d->kw;
    s->y_elems = d->N * d->K * Ho * Wo;
    // Keep every per-image and per-filter extent in 32 bits for the kernels.
    if ((int64_t)s->C * s->H * s->W > INT32_MAX || (int64_t)s->K * s->Ho * s->Wo > INT32_MAX ||
        (int64_t)s->Cg * s->kh * s->kw > INT32_MAX || s->w_elems > INT32_MAX)
        return fail(GCONV_ERR_UNSUPPORTED, "per-image or weight extent exceeds 2^31 elements");
    return GCONV_OK;
}

bool overlap(const void* a, int64_t a_elems, const void* b, int64_t b_elems)
{
    if (!a || !b || a_elems == 0 || b_elems == 0) return false;
    const char* pa = (const char*)a;
    const char* pb = (const char*)b;
    return pa < pb + b_elems * 4 && pb < pa + a_elems * 4;
}

// ---- channels-last (NHWC) ------------------------------------------------------
//
// An NHWC op runs on an NCHW shape, its "effective" shape:
//   - gradBias: dy [N*Ho*Wo, K] is the [rows, K] gradient of a 1x1 output;
//   - 1x1, stride 1, no padding, one group: y [N*H*W, K] = x [N*H*W, C] times
//     w [K, C] transposed, i.e. fully-connected mode over N*H*W rows (the
//     cudnn.torch issue: a 1x1 convolution is a Linear layer on the pixels);
//   - otherwise the NCHW shape itself, with the NHWC activations reordered
//     into NCHW copies in the workspace ("staged").
bool nhwc_as_gemm(const Shape& s)
{
    return s.kh == 1 && s.kw == 1 && s.sh == 1 && s.sw == 1 && s.ph == 0 && s.pw == 0 && s.ph_end == 0 &&
           s.pw_end == 0 && s.G == 1 && (int64_t)s.N * s.H * s.W < (int64_t(1) << 30);
}

Shape flat_rows(const Shape& s, int64_t rows, int C, int K)
{
    Shape f = s;
    f.nhwc = 0;
    f.N = (int)rows; f.C = C; f.H = 1; f.W = 1; f.K = K;
    f.kh = 1; f.kw = 1; f.sh = 1; f.sw = 1; f.ph = 0; f.pw = 0; f.ph_end = 0; f.pw_end = 0;
    f.dh = 1; f.dw = 1;
    f.G = 1; f.Cg = C; f.Kg = K;
    f.Ho = 1; f.Wo = 1;
    f.x_elems = rows * C; f.w_elems = (int64_t)K * C; f.y_elems = rows * K;
    return f;
}

int choose_path(const Shape& s, int op);

// NHWC depthwise on its own kernels: forward and gradInput where the NCHW
// dispatcher would pick the small-group family for the same shape, gradWeight
// whenever no family is forced (16-byte channel groups).
bool dw_nhwc_native(const Shape& s, int op)
{
    Shape e = s;
    e.nhwc = 0;
    if (op == GCONV_OP_BWD_FILTER)
        return g_path_override.load() == GCONV_PATH_AUTO && dw_nhwc_wgrad_supported(s);
    return dw_nhwc_supported(s) && choose_path(e, op) == GCONV_PATH_SMALLGROUP;
}

Shape effective_shape(const Shape& s, int op, bool* staged, bool* native_dw = nullptr)
{
    *staged = false;
    if (native_dw) *native_dw = false;
    if (!s.nhwc) return s;
    // (rows beyond 2^30 are refused by the prologue)
    if (op == GCONV_OP_BWD_BIAS) return flat_rows(s, std::min<int64_t>((int64_t)s.N * s.Ho * s.Wo, 1 << 30), s.K, s.K);
    if (nhwc_as_gemm(s)) {
        const Shape f = flat_rows(s, (int64_t)s.N * s.H * s.W, s.C, s.K);
        if (fc_supported(f)) return f;
    }
    // Depthwise forward and gradInput read NHWC natively (the small-group
    // family's choice; a forced family stages as below).
    if (op != GCONV_OP_BWD_BIAS && dw_nhwc_native(s, op)) {
        Shape e = s;
        e.nhwc = 0;
        if (native_dw) *native_dw = true;
        return e;
    }
    Shape e = s;
    e.nhwc = 0;
    *staged = true;
    return e;
}

constexpr size_t kStageAlign = 256;
size_t stage_bytes(int64_t elems) { return ((size_t)elems * 4 + kStageAlign - 1) / kStageAlign * kStageAlign; }

// Workspace of a staged op: its two NCHW copies, then the NCHW op's own.
size_t staging_bytes(const Shape& s, int op)
{
    switch (op) {
        case GCONV_OP_FWD: return stage_bytes(s.x_elems) + stage_bytes(s.y_elems);
        case GCONV_OP_BWD_DATA: return stage_bytes(s.y_elems) + stage_bytes(s.x_elems);
        case GCONV_OP_BWD_FILTER: return stage_bytes(s.x_elems) + stage_bytes(s.y_elems);
        default: return 0;
    }
}

// ---- routing ----------------------------------------------------------------

bool path_supports(int path, const Shape& s, int op)
{
    if (op == GCONV_OP_BWD_BIAS) return true;  // one reduction serves every path
    switch (path) {
        case GCONV_PATH_DIRECT: return true;
        case GCONV_PATH_IGEMM:
            if (op == GCONV_OP_FWD) return igemm_fwd_supported(s);
            if (op == GCONV_OP_BWD_DATA) return igemm_bwd_data_supported(s);
            if (op == GCONV_OP_BWD_FILTER) return igemm_bwd_filter_supported(s);
            return false;
        case GCONV_PATH_FC: return fc_supported(s);
        case GCONV_PATH_POINTWISE: return pointwise_supported(s);
        case GCONV_PATH_SMALLGROUP:
            if (op == GCONV_OP_FWD) return smallgroup_fwd_supported(s);
            if (op == GCONV_OP_BWD_DATA) return smallgroup_bwd_data_supported(s);
            if (op == GCONV_OP_BWD_FILTER) return smallgroup_bwd_filter_supported(s);
            return false;
        default: return false;
    }
}

// Static routing by shape. MFMA implicit GEMM when the per-group contraction
// is a real dense GEMM (at least 8 output channels per group for forward and
// gradInput, 16 for gradWeight, and a reduction of at least 64); direct
// kernels otherwise. At 8 channels per group half of each 16-wide MFMA
// fragment is idle, and the forward and gradInput passes still run at twice
// the LDS-tiled direct kernels' rate (ResNeXt's 8-per-group stage); the
// gradWeight kernel there runs at half the direct kernel's rate.
int choose_path(const Shape& s, int op)
{
    const int forced = g_path_override.load();
    if (forced != GCONV_PATH_AUTO) return forced;
    // gradBias is one reduction kernel pair whatever the shape; it reports
    // the direct path.
    if (op == GCONV_OP_BWD_BIAS) return GCONV_PATH_DIRECT;
    const int T = s.kh * s.kw;
    // Kernel == input: one dense layer per group on the flattened image.
    if (is_fc_mode(s) && path_supports(GCONV_PATH_FC, s, op)) return GCONV_PATH_FC;
    // 1x1 at stride 1 without padding: the plane of each (image, group) is a
    // matrix, and the convolution is a GEMM with the group's weight block.
    if (s.kh == 1 && s.kw == 1 && path_supports(GCONV_PATH_POINTWISE, s, op)) return GCONV_PATH_POINTWISE;
    // Depthwise gradWeight (one input channel per group): the depthwise row
    // kernel of the small-group family where it applies, else the sliced
    // direct gradWeight kernel; neither spends arithmetic on absent channels.
    if (op == GCONV_OP_BWD_FILTER && s.Cg == 1 && smallgroup_dw_wgrad_ok(s)) return GCONV_PATH_SMALLGROUP;
    if (op == GCONV_OP_BWD_FILTER && s.Cg == 1 && s.Kg <= 8 && (s.kh == 3 || s.kh == 5) &&
        s.kh == s.kw)
        return GCONV_PATH_DIRECT;
    // Strided gradInput with at least 4 channels per group on both sides: the
    // MFMA path's sub-pixel form (one launch storing whole dx rows) where it
    // applies, also ahead of the small-group kernels (4 per group, 256
    // channels, 56 x 56 at stride 2: 179 -> 98 us).
    if (op == GCONV_OP_BWD_DATA && (s.sh > 1 || s.sw > 1) && s.Cg >= 4 && s.Kg >= 4 &&
        igemm_bwd_data_subpixel_ok(s))
        return GCONV_PATH_IGEMM;
    // A handful of channels per group (ResNeXt-style, depthwise-like): the
    // HBM-bound 4x4x1-MFMA kernels.
    if (path_supports(GCONV_PATH_SMALLGROUP, s, op)) return GCONV_PATH_SMALLGROUP;
    if (op == GCONV_OP_FWD && s.Kg >= 8 && s.Cg * T >= 64 &&
        path_supports(GCONV_PATH_IGEMM, s, op))
        return GCONV_PATH_IGEMM;
    if (op == GCONV_OP_BWD_DATA && s.Cg >= 8 && s.Kg * T >= 64 &&
        path_supports(GCONV_PATH_IGEMM, s, op))
        return GCONV_PATH_IGEMM;
    if (op == GCONV_OP_BWD_FILTER && s.Cg >= 16 && s.Kg >= 16 &&
        path_supports(GCONV_PATH_IGEMM, s, op))
        return GCONV_PATH_IGEMM;
    return GCONV_PATH_DIRECT;
}

size_t workspace_for(const Shape& s, int op, int path)
{
    if (op == GCONV_OP_BWD_BIAS) return bias_workspace_bytes(s);
    if (op == GCONV_OP_BWD_FILTER && path == GCONV_PATH_IGEMM && s.N > 0)
        return igemm_bwd_filter_workspace(s);
    if (op == GCONV_OP_BWD_FILTER && path == GCONV_PATH_SMALLGROUP && s.N > 0)
        return smallgroup_bwd_filter_workspace(s);
    if (op == GCONV_OP_BWD_FILTER && path == GCONV_PATH_POINTWISE && s.N > 0)
        return pointwise_bwd_filter_workspace(s);
    if (op == GCONV_OP_BWD_FILTER && path == GCONV_PATH_FC && s.N > 0)
        return fc_bwd_filter_workspace(s);
    if ((op == GCONV_OP_FWD || op == GCONV_OP_BWD_DATA) && path == GCONV_PATH_FC && s.N > 0)
        return fc_data_workspace(s, op);
    if (op == GCONV_OP_BWD_FILTER && path == GCONV_PATH_DIRECT && s.N > 0)
        return direct_bwd_filter_workspace(s);
    return 0;
}

// Common prologue of the four ops: shape, effective (NCHW) shape, path,
// workspace checks.
struct Prep {
    Shape s;      // the descriptor's shape
    Shape e;      // the NCHW shape the kernels run (== s for NCHW)
    int path;
    bool staged;  // NHWC activations reordered through the workspace
    bool native;  // NHWC depthwise forward / gradInput on its own kernel
};

// Workspace of an op on its effective shape.
size_t op_workspace(const Shape& s, const Shape& e, int op, int path, bool staged, bool native)
{
    if (native) return op == GCONV_OP_BWD_FILTER ? dw_nhwc_wgrad_workspace(s) : 0;
    size_t ws = workspace_for(e, op, path);
    // The MFMA gradWeight reads channels-last tensors in place where they are
    // aligned (its partials only); the size covers the reordering route too.
    if (staged && op == GCONV_OP_BWD_FILTER && path == GCONV_PATH_IGEMM && igemm_bwd_filter_nhwc_supported(e))
        ws = std::max(ws, igemm_bwd_filter_nhwc_workspace(e));
    return ws + (staged ? staging_bytes(s, op) : 0);
}

int prologue(const gconv_desc* d, int op, Prep* p, void* ws, size_t ws_bytes)
{
    int st = make_shape(d, &p->s);
    if (st != GCONV_OK) return st;
    if (p->s.nhwc && op == GCONV_OP_BWD_BIAS && (int64_t)p->s.N * p->s.Ho * p->s.Wo >= (int64_t(1) << 30))
        return fail(GCONV_ERR_UNSUPPORTED, "NHWC gradBias over 2^30 or more rows");
    p->e = effective_shape(p->s, op, &p->staged, &p->native);
    p->path = choose_path(p->e, op);
    if (!path_supports(p->path, p->e, op))
        return fail(GCONV_ERR_UNSUPPORTED, "forced path %d cannot run this descriptor for op %d",
                    p->path, op);
    const size_t need = op_workspace(p->s, p->e, op, p->path, p->staged, p->native);
    if (ws_bytes < need || (need > 0 && ws == nullptr))
        return fail(GCONV_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes,
                    need);
    // Partial sums are read back with 16-byte loads.
    if (need > 0 && ((uintptr_t)ws & 15) != 0)
        return fail(GCONV_ERR_WORKSPACE, "workspace pointer %p is not 16-byte aligned", ws);
    return GCONV_OK;
}

// The kernels of one op on an NCHW shape.
int run_fwd(const Shape& s, int path, const float* x, const float* w, const float* bias, float* y,
            float* ws, hipStream_t hs)
{
    switch (path) {
        case GCONV_PATH_DIRECT: direct_fwd(s, x, w, bias, y, hs); return GCONV_OK;
        case GCONV_PATH_IGEMM:
            if (!igemm_fwd(s, x, w, bias, y, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "no MFMA kernel instance for this shape");
            return GCONV_OK;
        case GCONV_PATH_FC:
            if (!fc_fwd(s, x, w, bias, y, ws, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "fully-connected forward needs its workspace");
            return GCONV_OK;
        case GCONV_PATH_POINTWISE: pointwise_fwd(s, x, w, bias, y, hs); return GCONV_OK;
        case GCONV_PATH_SMALLGROUP:
            if (!smallgroup_fwd(s, x, w, bias, y, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "no small-group kernel instance for this shape");
            return GCONV_OK;
        default: return fail(GCONV_ERR_UNSUPPORTED, "no kernel for path %d", path);
    }
}

int run_bwd_data(const Shape& s, int path, const float* dy, const float* w, float* dx, float* ws,
                 hipStream_t hs)
{
    switch (path) {
        case GCONV_PATH_DIRECT: direct_bwd_data(s, dy, w, dx, hs); return GCONV_OK;
        case GCONV_PATH_IGEMM:
            if (!igemm_bwd_data(s, dy, w, dx, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "no MFMA kernel instance for this shape");
            return GCONV_OK;
        case GCONV_PATH_FC:
            if (!fc_bwd_data(s, dy, w, dx, ws, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "fully-connected gradInput needs its workspace");
            return GCONV_OK;
        case GCONV_PATH_POINTWISE: pointwise_bwd_data(s, dy, w, dx, hs); return GCONV_OK;
        case GCONV_PATH_SMALLGROUP:
            if (!smallgroup_bwd_data(s, dy, w, dx, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "no small-group kernel instance for this shape");
            return GCONV_OK;
        default: return fail(GCONV_ERR_UNSUPPORTED, "no kernel for path %d", path);
    }
}

int run_bwd_filter(const Shape& s, int path, const float* x, const float* dy, float* dw, float* ws,
                   hipStream_t hs)
{
    switch (path) {
        case GCONV_PATH_DIRECT: direct_bwd_filter(s, x, dy, dw, ws, hs); return GCONV_OK;
        case GCONV_PATH_IGEMM:
            if (!igemm_bwd_filter(s, x, dy, dw, ws, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "no MFMA kernel instance for this shape");
            return GCONV_OK;
        case GCONV_PATH_FC:
            if (!fc_bwd_filter(s, x, dy, dw, ws, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "fully-connected gradWeight needs its workspace");
            return GCONV_OK;
        case GCONV_PATH_POINTWISE:
            if (!pointwise_bwd_filter(s, x, dy, dw, ws, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "pointwise gradWeight needs its workspace");
            return GCONV_OK;
        case GCONV_PATH_SMALLGROUP:
            if (!smallgroup_bwd_filter(s, x, dy, dw, ws, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "no small-group kernel instance for this shape");
            return GCONV_OK;
        default: return fail(GCONV_ERR_UNSUPPORTED, "no kernel for path %d", path);
    }
}

// NHWC [N][R][Cc] -> NCHW [N][Cc][R] (or back, with R and Cc swapped).
int reorder(const float* src, float* dst, int64_t N, int64_t R, int64_t Cc, hipStream_t hs)
{
    if (!transpose_batched(src, dst, N, R, Cc, hs))
        return fail(GCONV_ERR_UNSUPPORTED, "layout reordering extent exceeds 2^30");
    return GCONV_OK;
}

// ---- the allocation-free gradWeight (gconv_bwd_filter_static) -----------------
//
// Device memory for what gconv_bwd_filter keeps in the caller's workspace
// (split partials, channels-last copies). Every device the library runs on
// holds its own copy of this array until the process ends. On the host the
// array's name is only a stand-in: kernels get the address hipGetSymbolAddress
// returns for the current device, looked up once per device.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

}  // namespace
}  // namespace gconv

static __device__ __align__(256) float scratch[gconv::kScratchBytes / sizeof(float)];

namespace gconv {
namespace {

// Device address of `scratch` on the device `stream` runs on, which must be
// the current device.
int scratch_address(hipStream_t stream, void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GCONV_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(GCONV_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices - 1);
    if (stream) {
        int sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return fail(GCONV_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
        if (sdev != dev)
            return fail(GCONV_ERR_ARG, "the stream belongs to device %d but device %d is current", sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(GCONV_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return GCONV_OK;
}

int epilogue()
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GCONV_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
    g_last_error.clear();
    return GCONV_OK;
}

}  // namespace
}  // namespace gconv

using namespace gconv;

extern "C" {

int gconv_output_dims(const gconv_desc* d, int64_t* Ho, int64_t* Wo)
{
    Shape s;
    const int st = make_shape(d, &s);
    if (st != GCONV_OK) return st;
    if (!Ho || !Wo) return fail(GCONV_ERR_NULL, "output pointer is NULL");
    *Ho = s.Ho;
    *Wo = s.Wo;
    return GCONV_OK;
}

int gconv_workspace_size(const gconv_desc* d, int op, size_t* bytes)
{
    Shape s;
    const int st = make_shape(d, &s);
    if (st != GCONV_OK) return st;
    if (!bytes) return fail(GCONV_ERR_NULL, "bytes pointer is NULL");
    if (op < GCONV_OP_FWD || op > GCONV_OP_BWD_BIAS) return fail(GCONV_ERR_ARG, "bad op %d", op);
    bool staged, native;
    const Shape e = effective_shape(s, op, &staged, &native);
    *bytes = op_workspace(s, e, op, choose_path(e, op), staged, native);
    return GCONV_OK;
}

int gconv_select_path(const gconv_desc* d, int op, int* path)
{
    Shape s;
    const int st = make_shape(d, &s);
    if (st != GCONV_OK) return st;
    if (!path) return fail(GCONV_ERR_NULL, "path pointer is NULL");
    if (op < GCONV_OP_FWD || op > GCONV_OP_BWD_BIAS) return fail(GCONV_ERR_ARG, "bad op %d", op);
    bool staged;
    *path = choose_path(effective_shape(s, op, &staged), op);
    return GCONV_OK;
}

int gconv_set_path_override(int path)
{
    if (path < GCONV_PATH_AUTO || path > GCONV_PATH_POINTWISE)
        return fail(GCONV_ERR_ARG, "unknown path %d", path);
    g_path_override.store(path);
    return GCONV_OK;
}

int gconv_fwd(const gconv_desc* d, const float* x, const float* w, const float* bias, float* y,
              void* workspace, size_t workspace_bytes, void* stream)
{
    return gconv_fwd_ex(d, x, w, bias, GCONV_EPILOGUE_NONE, y, workspace, workspace_bytes, stream);
}

int gconv_fwd_ex(const gconv_desc* d, const float* x, const float* w, const float* bias, int act,
                 float* y, void* workspace, size_t workspace_bytes, void* stream)
{
    Prep p;
    if (act != GCONV_EPILOGUE_NONE && act != GCONV_EPILOGUE_RELU)
        return fail(GCONV_ERR_ARG, "unknown epilogue %d", act);
    int st = prologue(d, GCONV_OP_FWD, &p, workspace, workspace_bytes);
    if (st != GCONV_OK) return st;
    const Shape& s = p.s;
    p.e.relu = act == GCONV_EPILOGUE_RELU;
    if (!w || (s.N > 0 && (!x || !y)))
        return fail(GCONV_ERR_NULL, "x, w and y must be non-NULL");
    if (overlap(y, s.y_elems, x, s.x_elems) || overlap(y, s.y_elems, w, s.w_elems) ||
        overlap(y, s.y_elems, bias, bias ? s.K : 0))
        return fail(GCONV_ERR_ARG, "y overlaps an input");
    hipStream_t hs = (hipStream_t)stream;
    (void)hipGetLastError();
    if (s.N == 0) return epilogue();
    if (p.native) {
        Shape sr = s;
        sr.relu = p.e.relu;
        dw_nhwc_fwd(sr, x, w, bias, y, hs);
    } else if (!p.staged) {
        st = run_fwd(p.e, p.path, x, w, bias, y, (float*)workspace, hs);
    } else {
        char* base = (char*)workspace;
        float* xs = (float*)base;
        float* ys = (float*)(base + stage_bytes(s.x_elems));
        float* rest = (float*)(base + staging_bytes(s, GCONV_OP_FWD));
        const bool a16 = ((uintptr_t)x & 15) == 0;
        if (p.path == GCONV_PATH_IGEMM && a16 && igemm_nhwc_io_supported(p.e, GCONV_OP_FWD)) {
            // The flat MFMA kernel reads x and stores y channels-last itself.
            if (!igemm_fwd_nhwc_io(p.e, x, w, bias, y, hs))
                st = fail(GCONV_ERR_UNSUPPORTED, "no MFMA kernel instance for this shape");
            return st != GCONV_OK ? st : epilogue();
        }
        st = reorder(x, xs, s.N, (int64_t)s.H * s.W, s.C, hs);
        // The flat MFMA kernel stores y channels-last itself.
        if (st == GCONV_OK && p.path == GCONV_PATH_IGEMM && igemm_nhwc_out_supported(p.e, GCONV_OP_FWD)) {
            if (!igemm_fwd_nhwc_out(p.e, xs, w, bias, y, hs))
                st = fail(GCONV_ERR_UNSUPPORTED, "no MFMA kernel instance for this shape");
        } else {
            if (st == GCONV_OK) st = run_fwd(p.e, p.path, xs, w, bias, ys, rest, hs);
            if (st == GCONV_OK) st = reorder(ys, y, s.N, s.K, (int64_t)s.Ho * s.Wo, hs);
        }
    }
    return st != GCONV_OK ? st : epilogue();
}

int gconv_bwd_data(const gconv_desc* d, const float* dy, const float* w, float* dx,
                   void* workspace, size_t workspace_bytes, void* stream)
{
    Prep p;
    int st = prologue(d, GCONV_OP_BWD_DATA, &p, workspace, workspace_bytes);
    if (st != GCONV_OK) return st;
    const Shape& s = p.s;
    if (!w || (s.N > 0 && (!dy || !dx)))
        return fail(GCONV_ERR_NULL, "dy, w and dx must be non-NULL");
    if (overlap(dx, s.x_elems, dy, s.y_elems) || overlap(dx, s.x_elems, w, s.w_elems))
        return fail(GCONV_ERR_ARG, "dx overlaps an input");
    hipStream_t hs = (hipStream_t)stream;
    (void)hipGetLastError();
    if (s.N == 0) return epilogue();
    if (p.native) {
        dw_nhwc_bwd_data(s, dy, w, dx, hs);
    } else if (!p.staged) {
        st = run_bwd_data(p.e, p.path, dy, w, dx, (float*)workspace, hs);
    } else {
        char* base = (char*)workspace;
        float* dys = (float*)base;
        float* dxs = (float*)(base + stage_bytes(s.y_elems));
        float* rest = (float*)(base + staging_bytes(s, GCONV_OP_BWD_DATA));
        const bool a16 = ((uintptr_t)dy & 15) == 0;
        if (p.path == GCONV_PATH_IGEMM && a16 && igemm_nhwc_io_supported(p.e, GCONV_OP_BWD_DATA)) {
            // The flat MFMA kernel reads dy and stores dx channels-last itself.
            if (!igemm_bwd_data_nhwc_io(p.e, dy, w, dx, hs))
                st = fail(GCONV_ERR_UNSUPPORTED, "no MFMA kernel instance for this shape");
            return st != GCONV_OK ? st : epilogue();
        }
        st = reorder(dy, dys, s.N, (int64_t)s.Ho * s.Wo, s.K, hs);
        if (st == GCONV_OK && p.path == GCONV_PATH_IGEMM && igemm_nhwc_out_supported(p.e, GCONV_OP_BWD_DATA)) {
            if (!igemm_bwd_data_nhwc_out(p.e, dys, w, dx, hs))
                st = fail(GCONV_ERR_UNSUPPORTED, "no MFMA kernel instance for this shape");
        } else {
            if (st == GCONV_OK) st = run_bwd_data(p.e, p.path, dys, w, dxs, rest, hs);
            if (st == GCONV_OK) st = reorder(dxs, dx, s.N, s.C, (int64_t)s.H * s.W, hs);
        }
    }
    return st != GCONV_OK ? st : epilogue();
}

int gconv_bwd_filter(const gconv_desc* d, const float* x, const float* dy, float* dw,
                     void* workspace, size_t workspace_bytes, void* stream)
{
    Prep p;
    int st = prologue(d, GCONV_OP_BWD_FILTER, &p, workspace, workspace_bytes);
    if (st != GCONV_OK) return st;
    const Shape& s = p.s;
    if (!dw || (s.N > 0 && (!x || !dy)))
        return fail(GCONV_ERR_NULL, "x, dy and dw must be non-NULL");
    if (overlap(dw, s.w_elems, x, s.x_elems) || overlap(dw, s.w_elems, dy, s.y_elems))
        return fail(GCONV_ERR_ARG, "dw overlaps an input");
    hipStream_t hs = (hipStream_t)stream;
    (void)hipGetLastError();
    if (s.N == 0) {
        fill_zero(dw, s.w_elems, hs);  // a sum over no images
        return epilogue();
    }
    if (p.native) {
        if (!dw_nhwc_bwd_filter(s, x, dy, dw, (float*)workspace, hs))
            st = fail(GCONV_ERR_UNSUPPORTED, "no channels-last depthwise gradWeight plan for this shape");
    } else if (!p.staged) {
        st = run_bwd_filter(p.e, p.path, x, dy, dw, (float*)workspace, hs);
    } else if (p.path == GCONV_PATH_IGEMM && ((uintptr_t)x & 15) == 0 && ((uintptr_t)dy & 15) == 0 &&
               igemm_bwd_filter_nhwc_supported(p.e)) {
        // The MFMA gradWeight reads x and dy channels-last itself.
        if (!igemm_bwd_filter_nhwc(p.e, x, dy, dw, (float*)workspace, hs))
            st = fail(GCONV_ERR_UNSUPPORTED, "no MFMA kernel instance for this shape");
    } else {
        char* base = (char*)workspace;
        float* xs = (float*)base;
        float* dys = (float*)(base + stage_bytes(s.x_elems));
        float* rest = (float*)(base + staging_bytes(s, GCONV_OP_BWD_FILTER));
        st = reorder(x, xs, s.N, (int64_t)s.H * s.W, s.C, hs);
        if (st == GCONV_OK) st = reorder(dy, dys, s.N, (int64_t)s.Ho * s.Wo, s.K, hs);
        if (st == GCONV_OK) st = run_bwd_filter(p.e, p.path, xs, dys, dw, rest, hs);
    }
    return st != GCONV_OK ? st : epilogue();
}

int gconv_bwd_filter_static(const gconv_desc* d, const float* x, const float* dy, float* dw, void* stream)
{
    size_t need = 0;
    int st = gconv_workspace_size(d, GCONV_OP_BWD_FILTER, &need);
    if (st != GCONV_OK) return st;
    if (need > kScratchBytes)
        return fail(GCONV_ERR_WORKSPACE, "this gradWeight needs %zu bytes of scratch; the static scratch holds %zu",
                    need, kScratchBytes);
    void* ws = nullptr;
    st = scratch_address((hipStream_t)stream, &ws);
    if (st != GCONV_OK) return st;
    return gconv_bwd_filter(d, x, dy, dw, ws, kScratchBytes, stream);
}

int gconv_bwd_bias(const gconv_desc* d, const float* dy, float* db, void* workspace,
                   size_t workspace_bytes, void* stream)
{
    Prep p;
    int st = prologue(d, GCONV_OP_BWD_BIAS, &p, workspace, workspace_bytes);
    if (st != GCONV_OK) return st;
    const Shape& s = p.s;
    if (!db || (s.N > 0 && !dy)) return fail(GCONV_ERR_NULL, "dy and db must be non-NULL");
    if (overlap(db, s.K, dy, s.y_elems)) return fail(GCONV_ERR_ARG, "db overlaps dy");
    hipStream_t hs = (hipStream_t)stream;
    (void)hipGetLastError();
    if (s.N == 0) {
        fill_zero(db, s.K, hs);
        return epilogue();
    }
    // NHWC: the effective shape reads dy as [N*Ho*Wo, K] rows.
    bias_reduce(p.e, dy, db, (float*)workspace, hs);
    return epilogue();
}

const char* gconv_status_string(int status)
{
    switch (status) {
        case GCONV_OK: return "ok";
        case GCONV_ERR_NULL: return "null pointer";
        case GCONV_ERR_SHAPE: return "invalid shape";
        case GCONV_ERR_GROUPS: return "channels not divisible by groups";
        case GCONV_ERR_WORKSPACE: return "workspace too small or misaligned";
        case GCONV_ERR_HIP: return "HIP error";
        case GCONV_ERR_UNSUPPORTED: return "unsupported";
        case GCONV_ERR_ARG: return "invalid argument";
        default: return "unknown status";
    }
}

const char* gconv_last_error(void) { return g_last_error.c_str(); }

int gconv_version(void) { return 110; }

}  // extern "C"
