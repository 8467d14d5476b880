// gconv_internal.h -- shapes and launcher declarations shared by the host
// dispatcher and the kernel translation units of the grouped-convolution
// library. Not part of the public ABI (that is include/gconv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gconv {

// A validated descriptor with the derived quantities every kernel needs.
// 32-bit fields: the dispatcher refuses extents that do not fit.
struct Shape {
    int N, C, H, W, K, kh, kw;
    int sh, sw, ph, pw, dh, dw;
    // Zero rows after the input and columns right of it. The kernels index
    // with the leading pads (ph, pw) and take the extent from Ho, Wo, so the
    // end pads matter only to shape checks.
    int ph_end, pw_end;
    int G, Cg, Kg;  // groups, input and output planes per group
    int Ho, Wo;
    // element counts (64-bit) of x, w, y
    int64_t x_elems, w_elems, y_elems;
    int relu = 0;   // forward only: y = max(conv + bias, 0)
    int nhwc = 0;   // activations channels-last (gconv_layout NHWC)
};

// The forward epilogue's activation: max(v, 0), with 0 (not NaN) for NaN.
__host__ __device__ inline float relu_if(float v, int relu) { return (relu && !(v > 0.f)) ? 0.f : v; }

inline bool is_fc_mode(const Shape& s)
{
    // Kernel covers the whole (unpadded) input: the conv is one dense layer
    // on the flattened image ("SpatialConvolution running in fully-connected
    // mode is very slow, even with R4", the View + Linear replacement). Only
    // undilated taps read every input pixel once: a dilated kernel the size of
    // the input reaches past it, into the end padding, and is not a Linear
    // layer (dilation is moot on an axis with a single tap).
    return s.kh == s.H && s.kw == s.W && s.ph == 0 && s.pw == 0 && (s.dh == 1 || s.kh == 1) &&
           (s.dw == 1 || s.kw == 1) && s.Ho == 1 && s.Wo == 1;
}

// ---- general direct kernels (any valid descriptor) -------------------------
void direct_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y,
                hipStream_t st);
void direct_bwd_data(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st);
void direct_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws,
                       hipStream_t st);
size_t direct_bwd_filter_workspace(const Shape& s);

// LDS-tiled direct kernels for up to 32 output channels per group; return
// false (nothing launched) where they do not apply.
bool direct_tile_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y,
                     hipStream_t st);
bool direct_tile_bwd_data(const Shape& s, const float* dy, const float* w, float* dx,
                          hipStream_t st);
bool direct_tile_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws,
                            hipStream_t st);
size_t direct_tile_bwd_filter_workspace(const Shape& s);

// ---- fp32-MFMA implicit GEMM (forward; gradInput, strided in sub-pixel form) ---
// *_supported() tell whether the family covers a shape; the launchers return
// false if no kernel instance matches (the dispatcher checks support first).
bool igemm_fwd_supported(const Shape& s);
bool igemm_bwd_data_supported(const Shape& s);
// Strided gradInput in the MFMA path's sub-pixel form (NCHW dy).
bool igemm_bwd_data_subpixel_ok(const Shape& s);
bool igemm_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y,
               hipStream_t st);
bool igemm_bwd_data(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st);
// The same ops writing y or dx channels-last (NHWC) where the flat kernel runs.
bool igemm_nhwc_out_supported(const Shape& s, int op);
bool igemm_fwd_nhwc_out(const Shape& s, const float* x, const float* w, const float* bias, float* y,
                        hipStream_t st);
bool igemm_bwd_data_nhwc_out(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st);
// ... and reading x or dy channels-last too (no reordering).
bool igemm_nhwc_io_supported(const Shape& s, int op);
bool igemm_fwd_nhwc_io(const Shape& s, const float* x, const float* w, const float* bias, float* y, hipStream_t st);
bool igemm_bwd_data_nhwc_io(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st);

// ---- fp32-MFMA gradWeight (split pixel reduction + deterministic reduce) -----
bool igemm_bwd_filter_supported(const Shape& s);
size_t igemm_bwd_filter_workspace(const Shape& s);
bool igemm_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws,
                      hipStream_t st);
// The same with channels-last x [N][H][W][C] and dy [N][Ho][Wo][K] read in
// place (s: the layer's NCHW shape; whole channel quads per group, 16-byte
// aligned tensors, else false and nothing launched).
bool igemm_bwd_filter_nhwc_supported(const Shape& s);
size_t igemm_bwd_filter_nhwc_workspace(const Shape& s);
bool igemm_bwd_filter_nhwc(const Shape& s, const float* x, const float* dy, float* dw, float* ws, hipStream_t st);

// ---- few channels per group: v_mfma_f32_4x4x1 kernels (HBM-bound shapes) ------
bool smallgroup_fwd_supported(const Shape& s);
bool smallgroup_bwd_data_supported(const Shape& s);
bool smallgroup_bwd_filter_supported(const Shape& s);
bool smallgroup_dw_wgrad_ok(const Shape& s);
size_t smallgroup_bwd_filter_workspace(const Shape& s);
bool smallgroup_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y,
                    hipStream_t st);
bool smallgroup_bwd_data(const Shape& s, const float* dy, const float* w, float* dx,
                         hipStream_t st);
bool smallgroup_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws,
                           hipStream_t st);

// ---- fully-connected mode (kernel == input): fp32-MFMA GEMMs ----------------
bool fc_supported(const Shape& s);
// Forward and gradInput split their reduction when the output tiles alone
// would leave part of the chip idle; the partials need fc_data_workspace().
size_t fc_data_workspace(const Shape& s, int op);
bool fc_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y, float* ws,
            hipStream_t st);
bool fc_bwd_data(const Shape& s, const float* dy, const float* w, float* dx, float* ws, hipStream_t st);
bool fc_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws, hipStream_t st);
size_t fc_bwd_filter_workspace(const Shape& s);

// ---- pointwise (1x1, stride 1, no padding): batched fp32-MFMA GEMMs --------------
bool pointwise_supported(const Shape& s);
size_t pointwise_bwd_filter_workspace(const Shape& s);
void pointwise_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y,
                   hipStream_t st);
void pointwise_bwd_data(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st);
bool pointwise_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws,
                          hipStream_t st);

// ---- reductions -------------------------------------------------------------
// db[k] = sum over (n, p < P) of dy[(n*K + k)*P + p], P = Ho*Wo.
size_t bias_workspace_bytes(const Shape& s);
// Depthwise (one channel per group) forward and gradInput on NHWC tensors.
bool dw_nhwc_supported(const Shape& s);
void dw_nhwc_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y, hipStream_t st);
void dw_nhwc_bwd_data(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st);
bool dw_nhwc_wgrad_supported(const Shape& s);
size_t dw_nhwc_wgrad_workspace(const Shape& s);
bool dw_nhwc_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws, hipStream_t st);
// dst[n] = src[n]^T for N row-major [R][Cc] matrices (NHWC <-> NCHW); false if
// the extents do not fit the kernel's 32-bit indices.
bool transpose_batched(const float* src, float* dst, int64_t N, int64_t R, int64_t Cc, hipStream_t st);
void bias_reduce(const Shape& s, const float* dy, float* db, float* ws, hipStream_t st);
// Fill `count` floats with zero (outputs of empty-batch reductions).
void fill_zero(float* p, int64_t count, hipStream_t st);

}  // namespace gconv
