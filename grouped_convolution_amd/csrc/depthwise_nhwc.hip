// depthwise_nhwc.hip -- depthwise convolution (one input and one output
// channel per group) on channels-last activations, forward and gradInput.
// In NHWC the channels of a pixel are contiguous, so a thread owns four
// consecutive channels of one output pixel and every tap is one 16-byte load
// that the wave's lanes read as one contiguous run of pixels x channels; the
// neighbouring pixels' overlapping windows are served from the caches. No
// reordering, no LDS: each output is a KS*KS-tap FMA chain per channel.
//   forward   y[n,ho,wo,c] = b[c] + sum_{i,j} w[c,i,j] * x[n, ho*sh - ph + i*dh, wo*sw - pw + j*dw, c]
//   gradInput dx[n,h,w,c]  = sum_{i,j} w[c,i,j] * dy[n, (h + ph - i*dh)/sh, (w + pw - j*dw)/sw, c]
//             over the taps whose quotients are exact and inside dy (the
//             adjoint of the forward correlation).
// The depthwise layers of the mobilenet family the DLPrimitives Blog
// validates are the target shapes; TensorFlow stores them channels-last.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "device_util.h"
#include "fastdiv.h"
#include "gconv_internal.h"

namespace gconv {
namespace {

constexpr int kRowPx = 4;  // outputs of a row per thread in the unit-stride kernels

// f(integral_constant<int, I>) for each I of the sequence, in order (a loop
// unrolled with the index usable as a constant expression).
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}


struct DwNhwcArgs {
    const float* in;     // x (forward) or dy (gradInput), NHWC
    const float* wgt;    // [C][KS][KS]
    const float* bias;   // forward only, may be null
    float* out;          // y or dx, NHWC
    int N, C, Hin, Win, Hout, Wout;   // extents of `in` and `out`
    int sh, sw, dh, dw, ph, pw;       // of the forward convolution
    int relu;
    int CQ;                           // channel groups per pixel (C / 4 or C)
    int total;                        // N * Hout * Wout * CQ (< 2^31)
    FastDiv div_cq, div_wout, div_img;
};

template <int KS, bool BWD, bool VEC>
__global__ void __launch_bounds__(256) dw_nhwc_kernel(DwNhwcArgs a)
{
    constexpr int T = KS * KS;
    constexpr int V = VEC ? 4 : 1;  // channels per thread
    const int tid = blockIdx.x * 256 + threadIdx.x;
    if (tid >= a.total) return;
    // (n, oh, ow, cq) from the flat index.
    const int pix = (int)fastdiv((uint32_t)tid, a.div_cq);
    const int cq = tid - pix * a.CQ;
    const int per_img = a.Hout * a.Wout;
    const int n = (int)fastdiv((uint32_t)pix, a.div_img);
    const int p = pix - n * per_img;
    const int oh = (int)fastdiv((uint32_t)p, a.div_wout);
    const int ow = p - oh * a.Wout;
    const int c = cq * V;

    float wv[T][V];
    if constexpr (VEC && T % 4 == 1) {
        // The 4*T weights of channels c..c+3 are contiguous and 16-byte aligned.
        float wf[4 * T];
        const f4* w4 = reinterpret_cast<const f4*>(a.wgt + (size_t)c * T);
#pragma unroll
        for (int u = 0; u < T; ++u) {
            const f4 v = w4[u];
            wf[4 * u] = v.x; wf[4 * u + 1] = v.y; wf[4 * u + 2] = v.z; wf[4 * u + 3] = v.w;
        }
#pragma unroll
        for (int q = 0; q < V; ++q)
#pragma unroll
            for (int t = 0; t < T; ++t) wv[t][q] = wf[q * T + t];
    } else {
#pragma unroll
        for (int q = 0; q < V; ++q)
#pragma unroll
            for (int t = 0; t < T; ++t) wv[t][q] = a.wgt[(size_t)(c + q) * T + t];
    }
    float acc[V];
#pragma unroll
    for (int q = 0; q < V; ++q) acc[q] = (!BWD && a.bias) ? a.bias[c + q] : 0.f;

    const float* img = a.in + (size_t)n * a.Hin * a.Win * a.C + c;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        int h;
        bool hok;
        if (!BWD) {
            h = oh * a.sh - a.ph + i * a.dh;
            hok = (unsigned)h < (unsigned)a.Hin;
        } else {
            const int hh = oh + a.ph - i * a.dh;
            h = hh >= 0 ? hh / a.sh : -1;
            hok = hh >= 0 && h * a.sh == hh && h < a.Hin;
        }
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            int w;
            bool wok;
            if (!BWD) {
                w = ow * a.sw - a.pw + j * a.dw;
                wok = (unsigned)w < (unsigned)a.Win;
            } else {
                const int ww = ow + a.pw - j * a.dw;
                w = ww >= 0 ? ww / a.sw : -1;
                wok = ww >= 0 && w * a.sw == ww && w < a.Win;
            }
            if (hok && wok) {
                const float* src = img + ((size_t)h * a.Win + w) * a.C;
                if constexpr (VEC) {
                    const f4 v = *reinterpret_cast<const f4*>(src);
                    acc[0] = fmaf(wv[i * KS + j][0], v.x, acc[0]);
                    acc[1] = fmaf(wv[i * KS + j][1], v.y, acc[1]);
                    acc[2] = fmaf(wv[i * KS + j][2], v.z, acc[2]);
                    acc[3] = fmaf(wv[i * KS + j][3], v.w, acc[3]);
                } else {
                    acc[0] = fmaf(wv[i * KS + j][0], src[0], acc[0]);
                }
            }
        }
    }
    float* dst = a.out + ((size_t)n * per_img + p) * a.C + c;
    if constexpr (VEC) {
        f4 o;
        o.x = relu_if(acc[0], a.relu);
        o.y = relu_if(acc[1], a.relu);
        o.z = relu_if(acc[2], a.relu);
        o.w = relu_if(acc[3], a.relu);
        __builtin_nontemporal_store(o, reinterpret_cast<f4*>(dst));
    } else {
        __builtin_nontemporal_store(relu_if(acc[0], a.relu), dst);
    }
}

// Unit stride and dilation, four channels per thread: a thread computes PX
// consecutive outputs of one row, loading each row's PX + KS - 1 input
// columns once (a sliding window in registers) and its 4*KS*KS weights once.
// gradInput at unit stride is the forward correlation of dy with the
// tap-reversed filter (FLIP) and padding KS - 1 - p.
template <int KS, int PX, bool FLIP>
__global__ void __launch_bounds__(256) dw_nhwc_row_kernel(DwNhwcArgs a)
{
    constexpr int T = KS * KS, NC = PX + KS - 1;
    const int tid = blockIdx.x * 256 + threadIdx.x;
    if (tid >= a.total) return;
    const int pix = (int)fastdiv((uint32_t)tid, a.div_cq);   // (n, oh, ow block)
    const int cq = tid - pix * a.CQ;
    const int nb = (a.Wout + PX - 1) / PX;
    const int per_img = a.Hout * nb;
    const int n = (int)fastdiv((uint32_t)pix, a.div_img);
    const int p = pix - n * per_img;
    const int oh = (int)fastdiv((uint32_t)p, a.div_wout);      // div_wout holds nb here
    const int ow0 = (p - oh * nb) * PX;
    const int c = cq * 4;

    float wf[4 * T];
    const f4* w4 = reinterpret_cast<const f4*>(a.wgt + (size_t)c * T);
#pragma unroll
    for (int u = 0; u < T; ++u) {
        const f4 v = w4[u];
        wf[4 * u] = v.x; wf[4 * u + 1] = v.y; wf[4 * u + 2] = v.z; wf[4 * u + 3] = v.w;
    }
    // Weight of channel q at tap (i, j), tap-reversed for gradInput.
    auto wt = [&](int q, int i, int j) { return FLIP ? wf[q * T + (KS - 1 - i) * KS + (KS - 1 - j)] : wf[q * T + i * KS + j]; };

    f4 acc[PX];
#pragma unroll
    for (int u = 0; u < PX; ++u) {
        acc[u] = f4{0.f, 0.f, 0.f, 0.f};
        if (a.bias) {
            acc[u].x = a.bias[c]; acc[u].y = a.bias[c + 1]; acc[u].z = a.bias[c + 2]; acc[u].w = a.bias[c + 3];
        }
    }
    const float* img = a.in + (size_t)n * a.Hin * a.Win * a.C + c;
    const int wb = ow0 - a.pw;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        const int h = oh - a.ph + i;
        if ((unsigned)h >= (unsigned)a.Hin) continue;
        f4 col[NC];
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int w = wb + u;
            col[u] = (unsigned)w < (unsigned)a.Win ? *reinterpret_cast<const f4*>(img + ((size_t)h * a.Win + w) * a.C)
                                                    : f4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < PX; ++u)
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                acc[u].x = fmaf(wt(0, i, j), col[u + j].x, acc[u].x);
                acc[u].y = fmaf(wt(1, i, j), col[u + j].y, acc[u].y);
                acc[u].z = fmaf(wt(2, i, j), col[u + j].z, acc[u].z);
                acc[u].w = fmaf(wt(3, i, j), col[u + j].w, acc[u].w);
            }
    }
    float* dst = a.out + (((size_t)n * a.Hout + oh) * a.Wout + ow0) * a.C + c;
#pragma unroll
    for (int u = 0; u < PX; ++u) {
        if (ow0 + u >= a.Wout) break;
        f4 o = acc[u];
        o.x = relu_if(o.x, a.relu); o.y = relu_if(o.y, a.relu); o.z = relu_if(o.z, a.relu); o.w = relu_if(o.w, a.relu);
        __builtin_nontemporal_store(o, reinterpret_cast<f4*>(dst + (size_t)u * a.C));
    }
}

// Unit stride and dilation, 3x3, walking down the rows: a wave owns 64
// consecutive (group of V channels, run of PX outputs) units of one output
// row and a band of RB output rows, and streams the band's input rows once
// each, PF rows ahead. Input row h adds its tap row i to output row
// h + ph - i, whose sums sit in a ring of three accumulator rows in registers;
// an output row is stored as soon as its last input row is in. Loads and
// stores are buffer operations whose out-of-range offsets read 0 or are
// dropped, so a band is one straight run of code (two compiler fences a step
// keep its loads and sums in step order) and the compiler's waits count
// exactly the rows in flight. The cached row kernel below fetches every input
// row once for each output row that reads it, from whichever XCD runs that
// row; here a band fetches it once (its halo rows twice).
struct DwWalkArgs {
    const float* in;     // x (forward) or dy (gradInput), NHWC
    const float* wgt;    // [C][3][3]
    const float* bias;   // forward only, may be null
    float* out;          // y or dx, NHWC
    int Hin, Win, Hout, Wout, C, ph, pw, relu;
    int CV, units, strips, nbands, waves;
    FastDiv div_cv;
};

template <int V> struct VecOf;
template <> struct VecOf<1> { using T = float; };
template <> struct VecOf<4> { using T = f4; };

template <int V>
__device__ __forceinline__ typename VecOf<V>::T load_vec(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    if constexpr (V == 4) return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
    else return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

template <int V>
__device__ __forceinline__ void store_vec(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, typename VecOf<V>::T v)
{
    if constexpr (V == 4)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, v), r,
                                               byte_off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_off, 0, 0);
}

template <int V, int PX, int PF, int RB, bool FLIP>
__global__ void __launch_bounds__(256) dw_nhwc_walk_kernel(DwWalkArgs a)
{
    using vt = typename VecOf<V>::T;
    constexpr int T = 9, NC = PX + 2, NS = RB + 2, NB = PF + 1;
    constexpr uint32_t kColOOB = 0x40000000u, kRowOOB = 0x80000000u;
    const int lane = threadIdx.x & 63;
    const int gw = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (gw >= a.waves) return;
    const int strip = gw % a.strips;
    const int nbd = gw / a.strips;
    const int band = nbd % a.nbands;
    const int n = nbd / a.nbands;
    const int ul = strip * 64 + lane;
    const bool live = ul < a.units;
    const int u = live ? ul : a.units - 1;
    const int blk = (int)fastdiv((uint32_t)u, a.div_cv);
    const int c = (u - blk * a.CV) * V;
    const int ow0 = blk * PX;

    // Weights of the lane's V channels, tap-reversed for gradInput, and bias.
    vt wv[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int tt = FLIP ? T - 1 - t : t;
        if constexpr (V == 4) {
            wv[t] = f4{a.wgt[(size_t)c * T + tt], a.wgt[(size_t)(c + 1) * T + tt], a.wgt[(size_t)(c + 2) * T + tt],
                       a.wgt[(size_t)(c + 3) * T + tt]};
        } else {
            wv[t] = a.wgt[(size_t)c * T + tt];
        }
    }
    vt b0 = vt{};
    if (a.bias) {
        if constexpr (V == 4) b0 = f4{a.bias[c], a.bias[c + 1], a.bias[c + 2], a.bias[c + 3]};
        else b0 = a.bias[c];
    }

    const uint32_t rowi = (uint32_t)a.Win * a.C * 4u, rowo = (uint32_t)a.Wout * a.C * 4u;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.in + (size_t)n * a.Hin * a.Win * a.C, (uint32_t)a.Hin * rowi);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.out + (size_t)n * a.Hout * a.Wout * a.C, (uint32_t)a.Hout * rowo);
    const int r0 = band * RB;
    const int rows = min(RB, a.Hout - r0);
    const int hb = r0 - a.ph;
    uint32_t xo[NC], yo[PX];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        const int w = ow0 - a.pw + k;
        xo[k] = (unsigned)w < (unsigned)a.Win ? (uint32_t)(w * a.C + c) * 4u : kColOOB;
    }
#pragma unroll
    for (int p = 0; p < PX; ++p)
        yo[p] = live && ow0 + p < a.Wout ? (uint32_t)((r0 * a.Wout + ow0 + p) * a.C + c) * 4u : kColOOB;

    auto load = [&](int t, vt (&v)[NC]) {
        const int h = hb + t;
        const uint32_t hs = t < rows + 2 && (unsigned)h < (unsigned)a.Hin ? (uint32_t)h * rowi : kRowOOB;
#pragma unroll
        for (int k = 0; k < NC; ++k) v[k] = load_vec<V>(rx, xo[k] + hs);
    };

    vt acc[3][PX];
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int p = 0; p < PX; ++p) acc[k][p] = b0;
    vt win[NB][NC];
#pragma unroll
    for (int k = 0; k < PF; ++k) load(k, win[k]);
    unroll_seq(
        [&](auto sc) {
            constexpr int t = decltype(sc)::value;
            asm volatile("" ::: "memory");  // this step's loads stay after the previous step
            if constexpr (t + PF < NS) load(t + PF, win[(t + PF) % NB]);
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
                for (int p = 0; p < PX; ++p)
#pragma unroll
                    for (int j = 0; j < 3; ++j)
                        acc[(t - i + 3) % 3][p] =
                            __builtin_elementwise_fma(wv[i * 3 + j], win[t % NB][p + j], acc[(t - i + 3) % 3][p]);
            // Slot (t + 1) mod 3 is complete (output t - 2), or before step 2
            // holds only taps of rows above the band's first output.
            vt(&done)[PX] = acc[(t + 1) % 3];
            if constexpr (t >= 2) {
                const uint32_t rs = t - 2 < rows ? (uint32_t)(t - 2) * rowo : kRowOOB;
#pragma unroll
                for (int p = 0; p < PX; ++p) {
                    vt v = done[p];
                    if (a.relu) v = __builtin_elementwise_max(v, vt{});
                    store_vec<V>(ry, yo[p] + rs, v);
                }
            }
#pragma unroll
            for (int p = 0; p < PX; ++p) {
                done[p] = b0;
                asm volatile("" : "+v"(acc[0][p]), "+v"(acc[1][p]), "+v"(acc[2][p]));  // sums formed in this step
            }
        },
        std::make_integer_sequence<int, NS>{});
}

#ifndef GCONV_DW_WALK_V
#define GCONV_DW_WALK_V 4
#endif
#ifndef GCONV_DW_WALK_PX
#define GCONV_DW_WALK_PX 4
#endif
#ifndef GCONV_DW_WALK_PF
#define GCONV_DW_WALK_PF 2
#endif
#ifndef GCONV_DW_WALK_RB
#define GCONV_DW_WALK_RB 14
#endif

template <bool FLIP>
void launch_walk(const DwNhwcArgs& s, hipStream_t st)
{
    constexpr int V = GCONV_DW_WALK_V, PX = GCONV_DW_WALK_PX, RB = GCONV_DW_WALK_RB;
    DwWalkArgs a{};
    a.in = s.in; a.wgt = s.wgt; a.bias = s.bias; a.out = s.out;
    a.Hin = s.Hin; a.Win = s.Win; a.Hout = s.Hout; a.Wout = s.Wout; a.C = s.C;
    a.ph = s.ph; a.pw = s.pw; a.relu = s.relu;
    a.CV = s.C / V;
    a.div_cv = make_fastdiv((uint32_t)a.CV);
    a.units = a.CV * ((a.Wout + PX - 1) / PX);
    a.strips = (a.units + 63) / 64;
    a.nbands = (a.Hout + RB - 1) / RB;
    a.waves = (int)((int64_t)s.N * a.strips * a.nbands);
    const unsigned blocks = (unsigned)((a.waves + 3) / 4);
    hipLaunchKernelGGL((dw_nhwc_walk_kernel<V, PX, GCONV_DW_WALK_PF, RB, FLIP>), dim3(blocks), dim3(256), 0, st, a);
}

template <int KS, bool FLIP>
void launch_row(DwNhwcArgs a, hipStream_t st)
{
    const int nb = (a.Wout + kRowPx - 1) / kRowPx;
    a.total = (int)((int64_t)a.N * a.Hout * nb * a.CQ);
    a.div_img = make_fastdiv((uint32_t)(a.Hout * nb));
    a.div_wout = make_fastdiv((uint32_t)nb);
    const unsigned blocks = (unsigned)((a.total + 255) / 256);
    hipLaunchKernelGGL((dw_nhwc_row_kernel<KS, kRowPx, FLIP>), dim3(blocks), dim3(256), 0, st, a);
}

template <int KS, bool BWD>
void launch(const DwNhwcArgs& a, bool vec, hipStream_t st)
{
    const unsigned blocks = (unsigned)((a.total + 255) / 256);
    if (vec) hipLaunchKernelGGL((dw_nhwc_kernel<KS, BWD, true>), dim3(blocks), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((dw_nhwc_kernel<KS, BWD, false>), dim3(blocks), dim3(256), 0, st, a);
}

}  // namespace

// Depthwise (multiplier 1), square 3x3 or 5x5 filters, any stride, padding and dilation.
bool dw_nhwc_supported(const Shape& s)
{
    if (!(s.Cg == 1 && s.Kg == 1 && s.kh == s.kw && (s.kh == 3 || s.kh == 5) && s.N >= 1)) return false;
    // Flat thread indices (pixels x channels of either tensor) stay below 2^31.
    const int64_t px = (int64_t)s.N * std::max((int64_t)s.H * s.W, (int64_t)s.Ho * s.Wo);
    return px * s.C < (int64_t(1) << 31);
}

static DwNhwcArgs dw_args(const Shape& s, bool bwd, bool vec)
{
    DwNhwcArgs a{};
    a.N = s.N; a.C = s.C;
    a.Hin = bwd ? s.Ho : s.H; a.Win = bwd ? s.Wo : s.W;
    a.Hout = bwd ? s.H : s.Ho; a.Wout = bwd ? s.W : s.Wo;
    a.sh = s.sh; a.sw = s.sw; a.dh = s.dh; a.dw = s.dw; a.ph = s.ph; a.pw = s.pw;
    a.CQ = vec ? s.C / 4 : s.C;
    a.total = (int)((int64_t)s.N * a.Hout * a.Wout * a.CQ);
    a.div_cq = make_fastdiv((uint32_t)a.CQ);
    a.div_img = make_fastdiv((uint32_t)(a.Hout * a.Wout));
    a.div_wout = make_fastdiv((uint32_t)a.Wout);
    return a;
}

static bool vec_ok(const Shape& s, const void* p0, const void* p1)
{
    return (s.C & 3) == 0 && ((uintptr_t)p0 & 15) == 0 && ((uintptr_t)p1 & 15) == 0;
}

// gradWeight: dw[c,i,j] = sum_{n,oh,ow} dy[n,oh,ow,c] * x[n, oh*sh - ph + i*dh, ow*sw - pw + j*dw, c].
// A block takes a slice of the N*Ho*Wo output pixels for every channel:
// thread t owns channels 4*(t % CQ) .. +3 and pixel lane t / CQ of the NP =
// 256 / CQ lanes (consecutive threads read consecutive channels of one pixel,
// then the next pixel: each load instruction covers whole pixels). A thread
// keeps 4*KS*KS sums; the pixel lanes are added in order through LDS and the
// block writes its partial [C][KS*KS] (or dw itself when there is one slice);
// dw_nhwc_wgrad_reduce adds the slices in order.
struct DwWgradArgs {
    const float* x;
    const float* dy;
    float* out;                 // dw, or the workspace [nslice][C*KS*KS]
    int N, C, H, W, Ho, Wo, sh, sw, dh, dw, ph, pw;
    int CQ, NP;                 // channel quads, pixel lanes per block
    int slice, total;           // units per slice, units (pixels, or runs of kRowPx pixels of a row)
    int nb;                     // runs per output row (unit stride: ceil(Wo / kRowPx))
    FastDiv div_cq, div_hw, div_wo;
};

// Four consecutive channels of one pixel: one 16-byte load when the tensors
// are 16-byte aligned, four 4-byte loads otherwise (e.g. a view that starts
// one float into its allocation).
template <bool V4>
__device__ inline f4 ld_quad(const float* p)
{
    if constexpr (V4) return *reinterpret_cast<const f4*>(p);
    else return f4{p[0], p[1], p[2], p[3]};
}

template <int KS, bool RUN, bool V4 = true>
__global__ void __launch_bounds__(256) dw_nhwc_wgrad_kernel(DwWgradArgs a)
{
    constexpr int T = KS * KS;
    extern __shared__ float red[];  // [NP][CQ][4*T]
    const int t = threadIdx.x;
    const int lp = (int)fastdiv((uint32_t)t, a.div_cq);
    const int cq = t - lp * a.CQ;
    const bool active = lp < a.NP;
    const int c = cq * 4;
    const int sl = blockIdx.x;
    const int p0 = sl * a.slice, p1 = min(a.total, p0 + a.slice);
    float acc[4 * T];
#pragma unroll
    for (int e = 0; e < 4 * T; ++e) acc[e] = 0.f;
    if (active && RUN) {
        // Unit stride and dilation: unit p is a run of kRowPx outputs of one
        // row; each input row's kRowPx + KS - 1 columns are loaded once.
        constexpr int NC = kRowPx + KS - 1;
        for (int p = p0 + lp; p < p1; p += a.NP) {
            const int n = (int)fastdiv((uint32_t)p, a.div_hw);   // div_hw: Ho * nb
            const int q = p - n * a.Ho * a.nb;
            const int oh = (int)fastdiv((uint32_t)q, a.div_wo);  // div_wo: nb
            const int ow0 = (q - oh * a.nb) * kRowPx;
            f4 d[kRowPx];
#pragma unroll
            for (int u = 0; u < kRowPx; ++u)
                d[u] = ow0 + u < a.Wo ? *reinterpret_cast<const f4*>(a.dy + (((size_t)n * a.Ho + oh) * a.Wo + ow0 + u) * a.C + c)
                                      : f4{0.f, 0.f, 0.f, 0.f};
            const float* img = a.x + (size_t)n * a.H * a.W * a.C + c;
#pragma unroll
            for (int i = 0; i < KS; ++i) {
                const int h = oh - a.ph + i;
                if ((unsigned)h >= (unsigned)a.H) continue;
                f4 col[NC];
#pragma unroll
                for (int v = 0; v < NC; ++v) {
                    const int w = ow0 - a.pw + v;
                    col[v] = (unsigned)w < (unsigned)a.W ? *reinterpret_cast<const f4*>(img + ((size_t)h * a.W + w) * a.C)
                                                         : f4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int j = 0; j < KS; ++j) {
                    const int tt = i * KS + j;
#pragma unroll
                    for (int u = 0; u < kRowPx; ++u) {
                        acc[tt] = fmaf(d[u].x, col[u + j].x, acc[tt]);
                        acc[T + tt] = fmaf(d[u].y, col[u + j].y, acc[T + tt]);
                        acc[2 * T + tt] = fmaf(d[u].z, col[u + j].z, acc[2 * T + tt]);
                        acc[3 * T + tt] = fmaf(d[u].w, col[u + j].w, acc[3 * T + tt]);
                    }
                }
            }
        }
    } else if (active) {
        for (int p = p0 + lp; p < p1; p += a.NP) {
            const int n = (int)fastdiv((uint32_t)p, a.div_hw);
            const int q = p - n * a.Ho * a.Wo;
            const int oh = (int)fastdiv((uint32_t)q, a.div_wo);
            const int ow = q - oh * a.Wo;
            const f4 d = ld_quad<V4>(a.dy + (size_t)p * a.C + c);
            const float* img = a.x + (size_t)n * a.H * a.W * a.C + c;
#pragma unroll
            for (int i = 0; i < KS; ++i) {
                const int h = oh * a.sh - a.ph + i * a.dh;
                if ((unsigned)h >= (unsigned)a.H) continue;
#pragma unroll
                for (int j = 0; j < KS; ++j) {
                    const int w = ow * a.sw - a.pw + j * a.dw;
                    if ((unsigned)w >= (unsigned)a.W) continue;
                    const f4 v = ld_quad<V4>(img + ((size_t)h * a.W + w) * a.C);
                    const int tt = i * KS + j;
                    acc[tt] = fmaf(d.x, v.x, acc[tt]);
                    acc[T + tt] = fmaf(d.y, v.y, acc[T + tt]);
                    acc[2 * T + tt] = fmaf(d.z, v.z, acc[2 * T + tt]);
                    acc[3 * T + tt] = fmaf(d.w, v.w, acc[3 * T + tt]);
                }
            }
        }
    }
    if (active) {
        float* r = red + ((size_t)lp * a.CQ + cq) * (4 * T);
#pragma unroll
        for (int e = 0; e < 4 * T; ++e) r[e] = acc[e];
    }
    __syncthreads();
    // Thread e < C*T adds the NP lanes' sums of output e = c*T + tap in order.
    float* out = a.out + (size_t)sl * a.C * T;
    for (int e = t; e < a.C * T; e += 256) {
        const int ch = e / T, tap = e - (e / T) * T;
        const int off = (ch >> 2) * (4 * T) + (ch & 3) * T + tap;
        float sum = red[off];
        for (int l = 1; l < a.NP; ++l) sum += red[(size_t)l * a.CQ * (4 * T) + off];
        out[e] = sum;
    }
}

// dw[e] = sum over slices (in order) of ws[slice][e]: 16 outputs x 64 slice
// groups per 1024-thread block; thread (e, sg) adds slices sg, sg + 64, ... in
// order (16 loads in flight), then the 64 group sums are added in order.
// gradWeight at unit stride and dilation, 3x3, walking down the rows: a wave
// owns 64 consecutive (group of V channels, run of PX outputs) units of one
// image and a band of RB output rows. Each input row's (PX + 2)-column window
// and each dy row's PX columns are buffer loads of V floats (out-of-range
// offsets read 0), PF input rows ahead; input row t pairs its tap row i with
// dy row t - i, held in a ring of registers. A lane keeps the 9 taps x V
// channels of its unit and writes them as the partial [tap][channel] of
// (image, band, run of columns); dw_nhwc_wgrad_reduce adds the partials in
// order. The band is one straight run of code, so the compiler's waits count
// exactly the rows in flight.
struct DwWalkWArgs {
    const float* x;
    const float* dy;
    float* ws;           // [N * nbands * nb][9][C]
    int H, W, Ho, Wo, C, ph, pw;
    int CV, nb, units, strips, nbands, waves;
    FastDiv div_cv;
};

template <int V, int PX, int PF, int RB>
__global__ void __launch_bounds__(256) dw_nhwc_wgrad_walk_kernel(DwWalkWArgs a)
{
    using vt = typename VecOf<V>::T;
    constexpr int NC = PX + 2, NS = RB + 2, NB = PF + 1;
    constexpr int PFD = PF, NBD = PFD + 3;
    constexpr uint32_t kColOOB = 0x40000000u, kRowOOB = 0x80000000u;
    const int lane = threadIdx.x & 63;
    const int gw = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (gw >= a.waves) return;
    const int strip = gw % a.strips;
    const int nbd = gw / a.strips;
    const int band = nbd % a.nbands;
    const int n = nbd / a.nbands;
    const int ul = strip * 64 + lane;
    const bool live = ul < a.units;
    const int u = live ? ul : a.units - 1;
    const int blk = (int)fastdiv((uint32_t)u, a.div_cv);
    const int c = (u - blk * a.CV) * V;
    const int ow0 = blk * PX;

    const uint32_t rowx = (uint32_t)a.W * a.C * 4u, rowd = (uint32_t)a.Wo * a.C * 4u;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x + (size_t)n * a.H * a.W * a.C, (uint32_t)a.H * rowx);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dy + (size_t)n * a.Ho * a.Wo * a.C, (uint32_t)a.Ho * rowd);
    const int r0 = band * RB;
    const int rows = min(RB, a.Ho - r0);
    const int hb = r0 - a.ph;
    uint32_t xo[NC], dof[PX];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        const int w = ow0 - a.pw + k;
        xo[k] = live && (unsigned)w < (unsigned)a.W ? (uint32_t)(w * a.C + c) * 4u : kColOOB;
    }
#pragma unroll
    for (int p = 0; p < PX; ++p)
        dof[p] = live && ow0 + p < a.Wo ? (uint32_t)((r0 * a.Wo + ow0 + p) * a.C + c) * 4u : kColOOB;

    auto loadx = [&](int t, vt (&v)[NC]) {
        const int h = hb + t;
        const uint32_t hs = t < rows + 2 && (unsigned)h < (unsigned)a.H ? (uint32_t)h * rowx : kRowOOB;
#pragma unroll
        for (int k = 0; k < NC; ++k) v[k] = load_vec<V>(rx, xo[k] + hs);
    };
    auto loadd = [&](int q, vt (&v)[PX]) {
        const uint32_t qs = q < rows ? (uint32_t)q * rowd : kRowOOB;
#pragma unroll
        for (int p = 0; p < PX; ++p) v[p] = load_vec<V>(rd, dof[p] + qs);
    };

    vt acc[9];
#pragma unroll
    for (int e = 0; e < 9; ++e) acc[e] = vt{};
    vt xw[NB][NC], dw[NBD][PX];
#pragma unroll
    for (int k = 0; k < PF; ++k) loadx(k, xw[k]);
#pragma unroll
    for (int q = 0; q < PFD && q < RB; ++q) loadd(q, dw[q]);
    unroll_seq(
        [&](auto sc) {
            constexpr int t = decltype(sc)::value;
            // Steps stay in order: hoisting later rows' loads (the code
            // generator would issue all of them first) holds them all in
            // registers ...
            asm volatile("" ::: "memory");
            if constexpr (t + PF < NS) loadx(t + PF, xw[(t + PF) % NB]);
            if constexpr (t + PFD < RB) loadd(t + PFD, dw[(t + PFD) % NBD]);
            unroll_seq(
                [&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    if constexpr (t >= i && t - i < RB) {
#pragma unroll
                        for (int p = 0; p < PX; ++p)
#pragma unroll
                            for (int j = 0; j < 3; ++j)
                                acc[i * 3 + j] = __builtin_elementwise_fma(dw[(t - i) % NBD][p], xw[t % NB][p + j],
                                                                           acc[i * 3 + j]);
                    }
                },
                std::make_integer_sequence<int, 3>{});
            // ... and this step's sums are formed before the next step's
            // loads (else all FMAs sink below all loads).
            asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
                         "+v"(acc[6]), "+v"(acc[7]), "+v"(acc[8]));
        },
        std::make_integer_sequence<int, NS>{});

    if (!live) return;
    // Partial [slice][tap][channel]: consecutive lanes write consecutive channels.
    float* out = a.ws + (((size_t)n * a.nbands + band) * a.nb + blk) * ((size_t)a.C * 9) + c;
#pragma unroll
    for (int e = 0; e < 9; ++e) *reinterpret_cast<vt*>(out + (size_t)e * a.C) = acc[e];
}

// TM: the partials are [slice][tap][channel] (the walk's); dw is [channel][tap].
template <bool TM = false>
__global__ void __launch_bounds__(1024) dw_nhwc_wgrad_reduce(const float* __restrict__ ws, float* __restrict__ dw,
                                                             int E, int nslice, int C = 0)
{
    __shared__ float part[64][17];
    const int el = threadIdx.x & 15, sg = threadIdx.x >> 4;
    const int e = blockIdx.x * 16 + el;
    float sum = 0.f;
    if (e < E) {
        int k = sg;
        for (; k + 15 * 64 < nslice; k += 16 * 64) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = ws[(size_t)(k + u * 64) * E + e];
#pragma unroll
            for (int u = 0; u < 16; ++u) sum += v[u];
        }
        for (; k < nslice; k += 64) sum += ws[(size_t)k * E + e];
    }
    part[sg][el] = sum;
    __syncthreads();
    if (sg != 0 || e >= E) return;
    sum = part[0][el];
    for (int i = 1; i < 64; ++i) sum += part[i][el];
    if constexpr (TM) dw[(e % C) * 9 + e / C] = sum;
    else dw[e] = sum;
}

static bool dw_wgrad_plan(const Shape& s, DwWgradArgs* out, int* nslice)
{
    if (!dw_nhwc_supported(s) || (s.C & 3) != 0) return false;
    DwWgradArgs a{};
    a.N = s.N; a.C = s.C; a.H = s.H; a.W = s.W; a.Ho = s.Ho; a.Wo = s.Wo;
    a.sh = s.sh; a.sw = s.sw; a.dh = s.dh; a.dw = s.dw; a.ph = s.ph; a.pw = s.pw;
    a.CQ = s.C / 4;
    if (a.CQ > 256) return false;
    a.NP = 256 / a.CQ;
    const int T = s.kh * s.kw;
    if ((size_t)a.NP * a.CQ * 4 * T * 4 > 64 * 1024) return false;
    const bool run = s.sh == 1 && s.sw == 1 && s.dh == 1 && s.dw == 1;
    a.nb = run ? (s.Wo + kRowPx - 1) / kRowPx : s.Wo;
    a.total = s.N * s.Ho * a.nb;
    // About 1024 slices, each giving every pixel lane at least a few units.
    int64_t want = std::min<int64_t>(1024, std::max<int64_t>(1, a.total / ((run ? 1 : 4) * a.NP)));
    a.slice = (int)((a.total + want - 1) / want);
    *nslice = (a.total + a.slice - 1) / a.slice;
    a.div_cq = make_fastdiv((uint32_t)a.CQ);
    a.div_hw = make_fastdiv((uint32_t)(s.Ho * a.nb));
    a.div_wo = make_fastdiv((uint32_t)a.nb);
    if (out) *out = a;
    return true;
}

bool dw_nhwc_wgrad_supported(const Shape& s)
{
    int ns;
    return dw_wgrad_plan(s, nullptr, &ns);
}

#ifndef GCONV_DWN_WALKW_V
#define GCONV_DWN_WALKW_V 1
#endif
#ifndef GCONV_DWN_WALKW_PX
#define GCONV_DWN_WALKW_PX 8
#endif
#ifndef GCONV_DWN_WALKW_PF
#define GCONV_DWN_WALKW_PF 4
#endif
#ifndef GCONV_DWN_WALKW_RB
#define GCONV_DWN_WALKW_RB 28
#endif

// The walking gradWeight: 3x3 at unit stride and dilation, channel quads.
static bool dw_walkw_plan(const Shape& s, DwWalkWArgs* out)
{
#ifdef GCONV_DWN_NO_WALKW
    (void)s; (void)out;
    return false;
#else
    constexpr int V = GCONV_DWN_WALKW_V, PX = GCONV_DWN_WALKW_PX, RB = GCONV_DWN_WALKW_RB;
    if (!(s.kh == 3 && s.kw == 3 && s.sh == 1 && s.sw == 1 && s.dh == 1 && s.dw == 1)) return false;
    if (!dw_nhwc_supported(s) || (s.C & 3) != 0) return false;
    if ((int64_t)s.H * s.W * s.C * 4 >= (int64_t(1) << 30) || (int64_t)s.Ho * s.Wo * s.C * 4 >= (int64_t(1) << 30))
        return false;
    DwWalkWArgs a{};
    a.H = s.H; a.W = s.W; a.Ho = s.Ho; a.Wo = s.Wo; a.C = s.C; a.ph = s.ph; a.pw = s.pw;
    a.CV = s.C / V;
    a.nb = (s.Wo + PX - 1) / PX;
    a.units = a.CV * a.nb;
    a.strips = (a.units + 63) / 64;
    a.nbands = (s.Ho + RB - 1) / RB;
    const int64_t waves = (int64_t)s.N * a.nbands * a.strips;
    const int64_t slices = (int64_t)s.N * a.nbands * a.nb;
    if (waves >= (int64_t(1) << 30) || slices * s.C * 9 >= (int64_t(1) << 31)) return false;
    a.waves = (int)waves;
    a.div_cv = make_fastdiv((uint32_t)a.CV);
    if (out) *out = a;
    return true;
#endif
}

size_t dw_nhwc_wgrad_workspace(const Shape& s)
{
    DwWgradArgs a;
    int ns;
    if (!dw_wgrad_plan(s, &a, &ns)) return 0;
    size_t bytes = ns > 1 ? (size_t)ns * s.C * s.kh * s.kw * sizeof(float) : 0;
    DwWalkWArgs wa;
    // (the walk needs 16-byte aligned tensors; the workspace covers both routes)
    if (dw_walkw_plan(s, &wa)) bytes = std::max(bytes, (size_t)s.N * wa.nbands * wa.nb * s.C * 9 * sizeof(float));
    return bytes;
}

bool dw_nhwc_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws, hipStream_t st)
{
    DwWgradArgs a;
    int ns;
    if (!dw_wgrad_plan(s, &a, &ns)) return false;
    DwWalkWArgs wa;
    if (ws && dw_walkw_plan(s, &wa) && ((uintptr_t)x & 15) == 0 && ((uintptr_t)dy & 15) == 0) {
        wa.x = x; wa.dy = dy; wa.ws = ws;
        hipLaunchKernelGGL((dw_nhwc_wgrad_walk_kernel<GCONV_DWN_WALKW_V, GCONV_DWN_WALKW_PX, GCONV_DWN_WALKW_PF,
                                                      GCONV_DWN_WALKW_RB>),
                           dim3((unsigned)((wa.waves + 3) / 4)), dim3(256), 0, st, wa);
        const int E = s.C * 9;
        hipLaunchKernelGGL(dw_nhwc_wgrad_reduce<true>, dim3((E + 15) / 16), dim3(1024), 0, st, ws, dw, E,
                           s.N * wa.nbands * wa.nb, s.C);
        return true;
    }
    if (ns > 1 && !ws) return false;
    a.x = x; a.dy = dy; a.out = ns > 1 ? ws : dw;
    const int T = s.kh * s.kw;
    const size_t lds = (size_t)a.NP * a.CQ * 4 * T * sizeof(float);
    const bool run = s.sh == 1 && s.sw == 1 && s.dh == 1 && s.dw == 1;
    if (((uintptr_t)x & 15) || ((uintptr_t)dy & 15)) {
        // Tensors that are not 16-byte aligned: the one-pixel units with
        // 4-byte loads (the run units hold windows of 16-byte loads). The plan
        // (slices, units per slice) is the same, so is the workspace.
        if (run) {
            a.nb = s.Wo;
            a.total = s.N * s.Ho * s.Wo;
            a.slice = (int)(((int64_t)a.total + ns - 1) / ns);
            ns = (a.total + a.slice - 1) / a.slice;
            a.div_hw = make_fastdiv((uint32_t)(s.Ho * s.Wo));
            a.div_wo = make_fastdiv((uint32_t)s.Wo);
            a.out = ns > 1 ? ws : dw;
        }
        if (s.kh == 3) hipLaunchKernelGGL((dw_nhwc_wgrad_kernel<3, false, false>), dim3(ns), dim3(256), lds, st, a);
        else hipLaunchKernelGGL((dw_nhwc_wgrad_kernel<5, false, false>), dim3(ns), dim3(256), lds, st, a);
    } else if (s.kh == 3) {
        if (run) hipLaunchKernelGGL((dw_nhwc_wgrad_kernel<3, true>), dim3(ns), dim3(256), lds, st, a);
        else hipLaunchKernelGGL((dw_nhwc_wgrad_kernel<3, false>), dim3(ns), dim3(256), lds, st, a);
    } else {
        if (run) hipLaunchKernelGGL((dw_nhwc_wgrad_kernel<5, true>), dim3(ns), dim3(256), lds, st, a);
        else hipLaunchKernelGGL((dw_nhwc_wgrad_kernel<5, false>), dim3(ns), dim3(256), lds, st, a);
    }
    if (ns > 1) {
        const int E = s.C * T;
        hipLaunchKernelGGL(dw_nhwc_wgrad_reduce<false>, dim3((E + 15) / 16), dim3(1024), 0, st, ws, dw, E, ns);
    }
    return true;
}

static bool unit(const Shape& s) { return s.sh == 1 && s.sw == 1 && s.dh == 1 && s.dw == 1; }
// 3x3 walks down the rows; 5x5 (a ring of five accumulator rows and a
// seven-column window) would leave one wave a SIMD, and keeps the row kernel.
// The walk's buffer offsets cover one image of either tensor below 2^30 bytes.
static bool walk_ok(const Shape& s)
{
    return s.kh == 3 && (int64_t)s.H * s.W * s.C * 4 < (int64_t(1) << 30) &&
           (int64_t)s.Ho * s.Wo * s.C * 4 < (int64_t(1) << 30) &&
           (int64_t)s.N * std::max(s.H, s.Ho) * ((std::max(s.W, s.Wo) + 3) / 4 * s.C / 4 + 64) < (int64_t(1) << 30);
}

void dw_nhwc_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y, hipStream_t st)
{
    const bool vec = vec_ok(s, x, y) && ((uintptr_t)w & 15) == 0;
    DwNhwcArgs a = dw_args(s, false, vec);
    a.in = x; a.wgt = w; a.bias = bias; a.out = y; a.relu = s.relu;
    if (vec && unit(s)) {
#ifndef GCONV_DW_NHWC_NO_WALK
        if (walk_ok(s)) {
            launch_walk<false>(a, st);
            return;
        }
#endif
        if (s.kh == 3) launch_row<3, false>(a, st);
        else launch_row<5, false>(a, st);
        return;
    }
    if (s.kh == 3) launch<3, false>(a, vec, st);
    else launch<5, false>(a, vec, st);
}

void dw_nhwc_bwd_data(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st)
{
    const bool vec = vec_ok(s, dy, dx) && ((uintptr_t)w & 15) == 0;
    DwNhwcArgs a = dw_args(s, true, vec);
    a.in = dy; a.wgt = w; a.bias = nullptr; a.out = dx; a.relu = 0;
    if (vec && unit(s)) {
        // The forward correlation of dy with the reversed taps and padding k - 1 - p.
        a.ph = s.kh - 1 - s.ph;
        a.pw = s.kw - 1 - s.pw;
#ifndef GCONV_DW_NHWC_NO_WALK
        if (walk_ok(s)) {
            launch_walk<true>(a, st);
            return;
        }
#endif
        if (s.kh == 3) launch_row<3, true>(a, st);
        else launch_row<5, true>(a, st);
        return;
    }
    if (s.kh == 3) launch<3, true>(a, vec, st);
    else launch<5, true>(a, vec, st);
}

}  // namespace gconv
