// direct.hip -- general direct kernels for grouped 2-D convolution (NCHW fp32).
//
// These run any valid descriptor (stride, padding, dilation, any group
// split) and are the fallback every specialised family is checked against.
// One launch covers all groups: the group of an output plane is derived from
// its channel index, and each group's planes are reached by offsets into the
// caller's tensors, never by copies ("[Feature request] Groups support for
// SpatialConvolutionMM": narrow() as a zero-copy offset, and the request for a
// single kernel over all groups).
#include "gconv_internal.h"

namespace gconv {

namespace {

constexpr int kBlock = 256;

// Sum of `v` over the 256 threads of a block, in a fixed order (wave64
// butterfly, then the four wave totals in index order). Valid in thread 0.
__device__ __forceinline__ float block_sum_256(float v, float* lds4)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) lds4[wave] = v;
    __syncthreads();
    float t = 0.f;
    if (threadIdx.x == 0) t = ((lds4[0] + lds4[1]) + lds4[2]) + lds4[3];
    return t;
}

// y[n,k,ho,wo]: one thread per output element, grid-stride.
__global__ void __launch_bounds__(kBlock)
direct_fwd_kernel(Shape s, const float* __restrict__ x, const float* __restrict__ w,
                  const float* __restrict__ bias, float* __restrict__ y)
{
    const int64_t total = s.y_elems;
    const int64_t HW = (int64_t)s.H * s.W;
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kBlock) {
        const int wo = (int)(e % s.Wo);
        int64_t t = e / s.Wo;
        const int ho = (int)(t % s.Ho);
        t /= s.Ho;
        const int k = (int)(t % s.K);
        const int64_t n = t / s.K;
        const int g = k / s.Kg;
        const float* xg = x + (n * s.C + (int64_t)g * s.Cg) * HW;
        const float* wk = w + (int64_t)k * s.Cg * s.kh * s.kw;
        float acc = 0.f;
        for (int c = 0; c < s.Cg; ++c) {
            for (int i = 0; i < s.kh; ++i) {
                const int h = ho * s.sh - s.ph + i * s.dh;
                if (h < 0 || h >= s.H) continue;
                for (int j = 0; j < s.kw; ++j) {
                    const int ww = wo * s.sw - s.pw + j * s.dw;
                    if (ww < 0 || ww >= s.W) continue;
                    acc = fmaf(wk[(c * s.kh + i) * s.kw + j], xg[c * HW + (int64_t)h * s.W + ww],
                               acc);
                }
            }
        }
        if (bias) acc += bias[k];
        y[e] = relu_if(acc, s.relu);
    }
}

// dx[n, g*Cg+c, h, w]: one thread per input element; gathers the taps whose
// window reads (h, w): ho = (h + ph - i*dh) / sh when exact and in range.
__global__ void __launch_bounds__(kBlock)
direct_bwd_data_kernel(Shape s, const float* __restrict__ dy, const float* __restrict__ w,
                       float* __restrict__ dx)
{
    const int64_t total = s.x_elems;
    const int64_t P = (int64_t)s.Ho * s.Wo;
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kBlock) {
        const int ww = (int)(e % s.W);
        int64_t t = e / s.W;
        const int h = (int)(t % s.H);
        t /= s.H;
        const int ca = (int)(t % s.C);
        const int64_t n = t / s.C;
        const int g = ca / s.Cg, c = ca % s.Cg;
        // Taps first: whether window (ho, wo) reads (h, ww) through tap (i, j)
        // does not depend on the output channel, so the stride tests run once
        // per tap and the channels of the group are the inner loop.
        const float* dyn = dy + (n * s.K + (int64_t)g * s.Kg) * P;
        const float* wgc = w + ((int64_t)g * s.Kg * s.Cg + c) * s.kh * s.kw;
        const int64_t wk = (int64_t)s.Cg * s.kh * s.kw;  // w stride between output channels
        float acc = 0.f;
        for (int i = 0; i < s.kh; ++i) {
            const int th = h + s.ph - i * s.dh;
            if (th < 0 || th % s.sh != 0) continue;
            const int ho = th / s.sh;
            if (ho >= s.Ho) continue;
            for (int j = 0; j < s.kw; ++j) {
                const int tw = ww + s.pw - j * s.dw;
                if (tw < 0 || tw % s.sw != 0) continue;
                const int wo = tw / s.sw;
                if (wo >= s.Wo) continue;
                const float* dp = dyn + (int64_t)ho * s.Wo + wo;
                const float* wp = wgc + i * s.kw + j;
                for (int k = 0; k < s.Kg; ++k) acc = fmaf(wp[k * wk], dp[k * P], acc);
            }
        }
        dx[e] = acc;
    }
}

// dw[k,c,i,j]: one block per weight element (grid-stride over elements); the
// block's threads stride over the N*Ho*Wo reduction, then a fixed-order block sum.
__global__ void __launch_bounds__(kBlock)
direct_bwd_filter_kernel(Shape s, const float* __restrict__ x, const float* __restrict__ dy,
                         float* __restrict__ dw)
{
    __shared__ float lds4[4];
    const int64_t P = (int64_t)s.Ho * s.Wo, HW = (int64_t)s.H * s.W;
    const int64_t total = (int64_t)s.N * P;
    for (int64_t e = blockIdx.x; e < s.w_elems; e += gridDim.x) {
        const int j = (int)(e % s.kw);
        const int i = (int)((e / s.kw) % s.kh);
        const int c = (int)((e / ((int64_t)s.kw * s.kh)) % s.Cg);
        const int k = (int)(e / ((int64_t)s.kw * s.kh * s.Cg));
        const int g = k / s.Kg;
        float acc = 0.f;
        for (int64_t t = threadIdx.x; t < total; t += kBlock) {
            const int64_t n = t / P;
            const int p = (int)(t % P);
            const int ho = p / s.Wo, wo = p % s.Wo;
            const int h = ho * s.sh - s.ph + i * s.dh;
            const int ww = wo * s.sw - s.pw + j * s.dw;
            if (h < 0 || h >= s.H || ww < 0 || ww >= s.W) continue;
            acc = fmaf(dy[(n * s.K + k) * P + p],
                       x[(n * s.C + (int64_t)g * s.Cg + c) * HW + (int64_t)h * s.W + ww], acc);
        }
        const float tot = block_sum_256(acc, lds4);
        if (threadIdx.x == 0) dw[e] = tot;
        __syncthreads();  // lds4 is reused by the next element
    }
}

// Small problems (a few hundred KB: the whole layer fits the caches many
// times over) are bound by the latency of their longest dependent chain, not
// by bandwidth; the kernels below trade every staging step for parallelism.
//
// Forward: eight lanes per output (consecutive lanes), lane q taking input
// channels q, q + 8, ..., three channels' taps loaded at once (the data is cold:
// each dependent round of loads costs an HBM latency); the eight partial sums
// are combined by a fixed butterfly, so the result does not depend on
// scheduling.
template <int KS>
__global__ void __launch_bounds__(kBlock) direct_small_fwd_kernel(Shape s, const float* __restrict__ x,
                                                                  const float* __restrict__ w,
                                                                  const float* __restrict__ bias,
                                                                  float* __restrict__ y)
{
    const int64_t gt = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t e = gt >> 3;
    const int q = (int)(gt & 7);
    const bool live = e < s.y_elems;
    float acc = 0.f;
    int k = 0;
    if (live) {
        const int wo = (int)(e % s.Wo);
        int64_t t = e / s.Wo;
        const int ho = (int)(t % s.Ho);
        t /= s.Ho;
        k = (int)(t % s.K);
        const int64_t n = t / s.K;
        const int g = k / s.Kg;
        const int64_t HW = (int64_t)s.H * s.W;
        const float* xg = x + (n * s.C + (int64_t)g * s.Cg) * HW;
        const float* wk = w + (int64_t)k * s.Cg * KS * KS;
        for (int c0 = q; c0 < s.Cg; c0 += 24) {
            float xv[3][KS * KS], wv[3][KS * KS];
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                const int c = c0 + 8 * u;
                const bool cok = c < s.Cg;
                const float* xc = xg + c * HW;
                const float* wc = wk + c * KS * KS;
#pragma unroll
                for (int i = 0; i < KS; ++i) {
                    const int h = ho * s.sh - s.ph + i * s.dh;
                    const bool hok = cok && (unsigned)h < (unsigned)s.H;
#pragma unroll
                    for (int j = 0; j < KS; ++j) {
                        const int ww = wo * s.sw - s.pw + j * s.dw;
                        const bool ok = hok && (unsigned)ww < (unsigned)s.W;
                        xv[u][i * KS + j] = ok ? xc[(int64_t)h * s.W + ww] : 0.f;
                        wv[u][i * KS + j] = ok ? wc[i * KS + j] : 0.f;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 3; ++u)
#pragma unroll
                for (int t = 0; t < KS * KS; ++t) acc = fmaf(wv[u][t], xv[u][t], acc);
        }
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    acc += __shfl_xor(acc, 4, 64);
    if (live && q == 0) {
        if (bias) acc += bias[k];
        y[e] = relu_if(acc, s.relu);
    }
}

// gradWeight: one 1024-thread block per (output channel k, input channel c)
// pair, all KS*KS taps in registers; threads stride over the N*Ho*Wo pixels
// (about one each at the target sizes), then each tap's sum goes through a
// fixed-order tree (wave butterfly, the 16 waves in index order).
constexpr int kSmallWgradBlock = 1024;
template <int KS>
__global__ void __launch_bounds__(kSmallWgradBlock) direct_small_wgrad_kernel(Shape s, const float* __restrict__ x,
                                                                               const float* __restrict__ dy,
                                                                               float* __restrict__ dw)
{
    constexpr int T = KS * KS, NWV = kSmallWgradBlock / 64;
    __shared__ float part[NWV][T];
    const int kc = blockIdx.x;                 // k * Cg + c
    const int k = kc / s.Cg, c = kc - k * s.Cg;
    const int g = k / s.Kg;
    const int P = s.Ho * s.Wo;
    const int64_t HW = (int64_t)s.H * s.W;
    const int total = s.N * P;
    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.f;
    // Two pixels a pass, their loads issued together.
    for (int pix0 = threadIdx.x; pix0 < total; pix0 += 2 * kSmallWgradBlock) {
        float d[2], xv[2][T];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int pix = pix0 + u * kSmallWgradBlock;
            const bool pok = pix < total;
            const int n = pok ? pix / P : 0, p = pix - n * P;
            const int ho = p / s.Wo, wo = p - ho * s.Wo;
            d[u] = pok ? dy[((int64_t)n * s.K + k) * P + p] : 0.f;
            const float* xc = x + ((int64_t)n * s.C + (int64_t)g * s.Cg + c) * HW;
#pragma unroll
            for (int i = 0; i < KS; ++i) {
                const int h = ho * s.sh - s.ph + i * s.dh;
                const bool hok = pok && (unsigned)h < (unsigned)s.H;
#pragma unroll
                for (int j = 0; j < KS; ++j) {
                    const int ww = wo * s.sw - s.pw + j * s.dw;
                    xv[u][i * KS + j] = (hok && (unsigned)ww < (unsigned)s.W) ? xc[(int64_t)h * s.W + ww] : 0.f;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < T; ++t) acc[t] = fmaf(d[u], xv[u][t], acc[t]);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        float v = acc[t];
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) part[wave][t] = v;
    }
    __syncthreads();
    if (threadIdx.x < T) {
        const int t = threadIdx.x;
        float sum = part[0][t];
        for (int wv = 1; wv < NWV; ++wv) sum += part[wv][t];
        dw[(int64_t)kc * T + t] = sum;
    }
}

__global__ void __launch_bounds__(kBlock) fill_zero_kernel(float* p, int64_t count)
{
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < count;
         e += (int64_t)gridDim.x * kBlock)
        p[e] = 0.f;
}

unsigned grid_for(int64_t total)
{
    const int64_t blocks = (total + kBlock - 1) / kBlock;
    return (unsigned)(blocks < 65536 ? (blocks < 1 ? 1 : blocks) : 65536);
}

}  // namespace

// Small enough that latency, not bandwidth or arithmetic, sets the time: a
// few tens of thousands of outputs (the NNlib benchmark's grouped layer:
// 2 x 15 x 26 x 26), square 3x3 or 5x5 filters.
static bool small_fwd(const Shape& s)
{
    return s.kh == s.kw && (s.kh == 3 || s.kh == 5) && s.y_elems <= (1 << 16) && s.Cg >= 4;
}
static bool small_bwd_data(const Shape& s) { return s.x_elems <= (1 << 18) && s.Kg * s.kh * s.kw <= 64; }
static bool small_wgrad(const Shape& s)
{
    return s.kh == s.kw && (s.kh == 3 || s.kh == 5) && (int64_t)s.N * s.Ho * s.Wo <= 4096 &&
           (int64_t)s.K * s.Cg >= 128 && (int64_t)s.K * s.Cg < (1 << 30);
}

void direct_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y,
                hipStream_t st)
{
    if (s.y_elems == 0) return;
    if (small_fwd(s)) {
        const unsigned blocks = (unsigned)((s.y_elems * 8 + kBlock - 1) / kBlock);
        if (s.kh == 3) hipLaunchKernelGGL((direct_small_fwd_kernel<3>), dim3(blocks), dim3(kBlock), 0, st, s, x, w, bias, y);
        else hipLaunchKernelGGL((direct_small_fwd_kernel<5>), dim3(blocks), dim3(kBlock), 0, st, s, x, w, bias, y);
        return;
    }
    if (direct_tile_fwd(s, x, w, bias, y, st)) return;
    hipLaunchKernelGGL(direct_fwd_kernel, dim3(grid_for(s.y_elems)), dim3(kBlock), 0, st, s, x,
                       w, bias, y);
}

void direct_bwd_data(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st)
{
    if (s.x_elems == 0) return;
    if (!small_bwd_data(s) && direct_tile_bwd_data(s, dy, w, dx, st)) return;
    hipLaunchKernelGGL(direct_bwd_data_kernel, dim3(grid_for(s.x_elems)), dim3(kBlock), 0, st, s,
                       dy, w, dx);
}

size_t direct_bwd_filter_workspace(const Shape& s)
{
    return small_wgrad(s) ? 0 : direct_tile_bwd_filter_workspace(s);
}

void direct_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws,
                       hipStream_t st)
{
    if (small_wgrad(s)) {
        if (s.N == 0) {
            fill_zero(dw, s.w_elems, st);
            return;
        }
        const unsigned blocks = (unsigned)((int64_t)s.K * s.Cg);
        if (s.kh == 3) hipLaunchKernelGGL((direct_small_wgrad_kernel<3>), dim3(blocks), dim3(kSmallWgradBlock), 0, st, s, x, dy, dw);
        else hipLaunchKernelGGL((direct_small_wgrad_kernel<5>), dim3(blocks), dim3(kSmallWgradBlock), 0, st, s, x, dy, dw);
        return;
    }
    if (direct_tile_bwd_filter(s, x, dy, dw, ws, st)) return;
    const int64_t blocks = s.w_elems < (1 << 20) ? s.w_elems : (1 << 20);
    hipLaunchKernelGGL(direct_bwd_filter_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, s,
                       x, dy, dw);
}

void fill_zero(float* p, int64_t count, hipStream_t st)
{
    if (count == 0) return;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(count)), dim3(kBlock), 0, st, p, count);
}

}  // namespace gconv
