// gconv_api.hip -- the C ABI (include/gconv.h): descriptor validation, output
// extents, routing between kernel families, workspace sizing and error
// reporting. Everything here runs on the host; kernels live in the other
// translation units.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
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
    if (op == GCONV_OP_BWD_FILTER && path == GCONV_PATH_DIRECT && s.N > 0)
        return direct_bwd_filter_workspace(s);
    return 0;
}

// Common prologue of the four ops: shape, path, workspace checks.
int prologue(const gconv_desc* d, int op, Shape* s, int* path, void* ws, size_t ws_bytes)
{
    int st = make_shape(d, s);
    if (st != GCONV_OK) return st;
    *path = choose_path(*s, op);
    if (!path_supports(*path, *s, op))
        return fail(GCONV_ERR_UNSUPPORTED, "forced path %d cannot run this descriptor for op %d",
                    *path, op);
    const size_t need = workspace_for(*s, op, *path);
    if (ws_bytes < need || (need > 0 && ws == nullptr))
        return fail(GCONV_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes,
                    need);
    // Partial sums are read back with 16-byte loads.
    if (need > 0 && ((uintptr_t)ws & 15) != 0)
        return fail(GCONV_ERR_WORKSPACE, "workspace pointer %p is not 16-byte aligned", ws);
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
    *bytes = workspace_for(s, op, choose_path(s, op));
    return GCONV_OK;
}

int gconv_select_path(const gconv_desc* d, int op, int* path)
{
    Shape s;
    const int st = make_shape(d, &s);
    if (st != GCONV_OK) return st;
    if (!path) return fail(GCONV_ERR_NULL, "path pointer is NULL");
    if (op < GCONV_OP_FWD || op > GCONV_OP_BWD_BIAS) return fail(GCONV_ERR_ARG, "bad op %d", op);
    *path = choose_path(s, op);
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
    Shape s;
    int path;
    if (act != GCONV_EPILOGUE_NONE && act != GCONV_EPILOGUE_RELU)
        return fail(GCONV_ERR_ARG, "unknown epilogue %d", act);
    int st = prologue(d, GCONV_OP_FWD, &s, &path, workspace, workspace_bytes);
    if (st != GCONV_OK) return st;
    s.relu = act == GCONV_EPILOGUE_RELU;
    if (!w || (s.N > 0 && (!x || !y)))
        return fail(GCONV_ERR_NULL, "x, w and y must be non-NULL");
    if (overlap(y, s.y_elems, x, s.x_elems) || overlap(y, s.y_elems, w, s.w_elems) ||
        overlap(y, s.y_elems, bias, bias ? s.K : 0))
        return fail(GCONV_ERR_ARG, "y overlaps an input");
    hipStream_t hs = (hipStream_t)stream;
    (void)hipGetLastError();
    if (s.N == 0) return epilogue();
    switch (path) {
        case GCONV_PATH_DIRECT: direct_fwd(s, x, w, bias, y, hs); break;
        case GCONV_PATH_IGEMM:
            if (!igemm_fwd(s, x, w, bias, y, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "no MFMA kernel instance for this shape");
            break;
        case GCONV_PATH_FC: fc_fwd(s, x, w, bias, y, hs); break;
        case GCONV_PATH_POINTWISE: pointwise_fwd(s, x, w, bias, y, hs); break;
        case GCONV_PATH_SMALLGROUP:
            if (!smallgroup_fwd(s, x, w, bias, y, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "no small-group kernel instance for this shape");
            break;
        default: return fail(GCONV_ERR_UNSUPPORTED, "no kernel for path %d", path);
    }
    return epilogue();
}

int gconv_bwd_data(const gconv_desc* d, const float* dy, const float* w, float* dx,
                   void* workspace, size_t workspace_bytes, void* stream)
{
    Shape s;
    int path;
    int st = prologue(d, GCONV_OP_BWD_DATA, &s, &path, workspace, workspace_bytes);
    if (st != GCONV_OK) return st;
    if (!w || (s.N > 0 && (!dy || !dx)))
        return fail(GCONV_ERR_NULL, "dy, w and dx must be non-NULL");
    if (overlap(dx, s.x_elems, dy, s.y_elems) || overlap(dx, s.x_elems, w, s.w_elems))
        return fail(GCONV_ERR_ARG, "dx overlaps an input");
    hipStream_t hs = (hipStream_t)stream;
    (void)hipGetLastError();
    if (s.N == 0) return epilogue();
    switch (path) {
        case GCONV_PATH_DIRECT: direct_bwd_data(s, dy, w, dx, hs); break;
        case GCONV_PATH_IGEMM:
            if (!igemm_bwd_data(s, dy, w, dx, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "no MFMA kernel instance for this shape");
            break;
        case GCONV_PATH_FC: fc_bwd_data(s, dy, w, dx, hs); break;
        case GCONV_PATH_POINTWISE: pointwise_bwd_data(s, dy, w, dx, hs); break;
        case GCONV_PATH_SMALLGROUP:
            if (!smallgroup_bwd_data(s, dy, w, dx, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "no small-group kernel instance for this shape");
            break;
        default: return fail(GCONV_ERR_UNSUPPORTED, "no kernel for path %d", path);
    }
    return epilogue();
}

int gconv_bwd_filter(const gconv_desc* d, const float* x, const float* dy, float* dw,
                     void* workspace, size_t workspace_bytes, void* stream)
{
    Shape s;
    int path;
    int st = prologue(d, GCONV_OP_BWD_FILTER, &s, &path, workspace, workspace_bytes);
    if (st != GCONV_OK) return st;
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
    switch (path) {
        case GCONV_PATH_DIRECT: direct_bwd_filter(s, x, dy, dw, (float*)workspace, hs); break;
        case GCONV_PATH_IGEMM:
            if (!igemm_bwd_filter(s, x, dy, dw, (float*)workspace, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "no MFMA kernel instance for this shape");
            break;
        case GCONV_PATH_FC: fc_bwd_filter(s, x, dy, dw, hs); break;
        case GCONV_PATH_POINTWISE:
            if (!pointwise_bwd_filter(s, x, dy, dw, (float*)workspace, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "pointwise gradWeight needs its workspace");
            break;
        case GCONV_PATH_SMALLGROUP:
            if (!smallgroup_bwd_filter(s, x, dy, dw, (float*)workspace, hs))
                return fail(GCONV_ERR_UNSUPPORTED, "no small-group kernel instance for this shape");
            break;
        default: return fail(GCONV_ERR_UNSUPPORTED, "no kernel for path %d", path);
    }
    return epilogue();
}

int gconv_bwd_bias(const gconv_desc* d, const float* dy, float* db, void* workspace,
                   size_t workspace_bytes, void* stream)
{
    Shape s;
    int path;
    int st = prologue(d, GCONV_OP_BWD_BIAS, &s, &path, workspace, workspace_bytes);
    if (st != GCONV_OK) return st;
    if (!db || (s.N > 0 && !dy)) return fail(GCONV_ERR_NULL, "dy and db must be non-NULL");
    if (overlap(db, s.K, dy, s.y_elems)) return fail(GCONV_ERR_ARG, "db overlaps dy");
    hipStream_t hs = (hipStream_t)stream;
    (void)hipGetLastError();
    if (s.N == 0) {
        fill_zero(db, s.K, hs);
        return epilogue();
    }
    bias_reduce(s, dy, db, (float*)workspace, hs);
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

int gconv_version(void) { return 100; }

}  // extern "C"
