// direct_tile.hip -- LDS-tiled direct convolution for groups with up to 32
// output channels that the MFMA families do not take (a handful of outputs
// against many inputs, e.g. 20 in / 3 out per group), any stride, padding and
// dilation on the forward pass; gradInput at stride 1 as the forward of dy
// with the transposed, tap-reversed filter (the adjoint of a stride-1
// correlation is the correlation with the reversed kernel).
//
// A block owns 64 consecutive output pixels of one (image, group) plane; its
// four waves take every fourth input channel of those pixels (shorter serial
// chains, four times the blocks) and their sums are added in a fixed order at
// the end. For each chunk of input channels the input rows the pixels read
// (halo and zero padding included) and the chunk's filters go to LDS; each
// thread keeps all of its pixel's output channels in registers, so an input
// value read once from LDS feeds KG multiply-adds and the filter reads are
// wave-wide broadcasts. One launch covers every group
// ("[Feature request] Groups support for SpatialConvolutionMM": offsets per
// group, one kernel over all groups).
#include <algorithm>

#include "device_util.h"
#include "gconv_internal.h"

namespace gconv {
namespace {

struct TileArgs {
    const float* in;
    const float* wgt;
    const float* bias;
    float* out;
    int N, G, Cin_tot, Cin_g, Hin, Win, Cout_tot, Cout_g, Hout, Wout;
    int kh, kw, sh, sw, dh, dw, ph, pw;
    int w_so, w_sr, w_gstride;
    int tiles;          // tiles of 256 output pixels per plane
    int relu;           // forward epilogue: max(v, 0)
    int LW, LR, CC;     // LDS tile: row width, rows, input channels per chunk
    bool flip;
};

template <int KG>
__global__ void __launch_bounds__(256) direct_tile_kernel(TileArgs a)
{
    // [CC][LR][LW] input rows, then [CC][T][KG] filters; at the end the four
    // channel groups' partial sums [4][KG][64] reuse the space.
    extern __shared__ float lds[];
    const int T = a.kh * a.kw;
    float* xs = lds;
    float* wl = lds + a.CC * a.LR * a.LW;
    const int tid = threadIdx.x;
    const int px = tid & 63;                                    // pixel of the tile
    const int cg = __builtin_amdgcn_readfirstlane(tid >> 6);    // channel group = wave

    int bid = blockIdx.x;
    const int tile = bid % a.tiles;
    bid /= a.tiles;
    const int g = bid % a.G;
    const int n = bid / a.G;
    const int P = a.Hout * a.Wout;
    const int p0 = tile * 64;
    const int pl = min(p0 + 64, P) - 1;
    const int ho_first = p0 / a.Wout;
    const int rows = (pl / a.Wout - ho_first) * a.sh + (a.kh - 1) * a.dh + 1;  // <= LR
    const int hbase = ho_first * a.sh - a.ph;
    const int p = p0 + px;
    const int pc = min(p, pl);
    const int ho = pc / a.Wout, wo = pc - (pc / a.Wout) * a.Wout;
    const int xpix = (ho - ho_first) * a.sh * a.LW + wo * a.sw;

    const float* in_g = a.in + ((size_t)n * a.Cin_tot + (size_t)g * a.Cin_g) * a.Hin * a.Win;
    const float* w_g = a.wgt + (size_t)g * a.w_gstride;
    const int plane = rows * a.LW;

    float acc[KG];
#pragma unroll
    for (int k = 0; k < KG; ++k) acc[k] = 0.f;

    for (int c0 = 0; c0 < a.Cin_g; c0 += a.CC) {
        const int cc = min(a.CC, a.Cin_g - c0);
        __syncthreads();  // every thread is done with the previous chunk
        for (int e = tid; e < cc * plane; e += 256) {
            const int c = e / plane, rem = e - (e / plane) * plane;
            const int r = rem / a.LW, col = rem - (rem / a.LW) * a.LW;
            const int h = hbase + r, w = col - a.pw;
            const bool ok = (unsigned)h < (unsigned)a.Hin && (unsigned)w < (unsigned)a.Win;
            xs[(c * a.LR + r) * a.LW + col] =
                ok ? in_g[((size_t)(c0 + c) * a.Hin + h) * a.Win + w] : 0.f;
        }
        for (int e = tid; e < cc * T * KG; e += 256) {
            const int k = e % KG, ct = e / KG, c = ct / T, t = ct - (ct / T) * T;
            wl[e] = k < a.Cout_g
                        ? w_g[(size_t)k * a.w_so + (size_t)(c0 + c) * a.w_sr + (a.flip ? T - 1 - t : t)]
                        : 0.f;
        }
        __syncthreads();
        // This wave's channels of the chunk: cg, cg + 4, ...
        for (int c = cg; c < cc; c += 4) {
            const float* xc = xs + c * a.LR * a.LW + xpix;
            const float* wc = wl + c * T * KG;
            for (int i = 0; i < a.kh; ++i)
                for (int j = 0; j < a.kw; ++j) {
                    const float xv = xc[i * a.dh * a.LW + j * a.dw];
                    const float* wt = wc + (i * a.kw + j) * KG;
#pragma unroll
                    for (int k = 0; k < KG; ++k) acc[k] = fmaf(wt[k], xv, acc[k]);
                }
        }
    }
    // Add the four channel groups' sums in order: red[cg][k][px].
    __syncthreads();
    float* red = lds;
#pragma unroll
    for (int k = 0; k < KG; ++k) red[(cg * KG + k) * 64 + px] = acc[k];
    __syncthreads();
    if (cg != 0 || p >= P) return;
    float* out = a.out + ((size_t)n * a.Cout_tot + (size_t)g * a.Cout_g) * P + p;
#pragma unroll
    for (int k = 0; k < KG; ++k)
        if (k < a.Cout_g) {
            const float v = ((red[k * 64 + px] + red[(KG + k) * 64 + px]) + red[(2 * KG + k) * 64 + px]) +
                            red[(3 * KG + k) * 64 + px];
            out[(size_t)k * P] = relu_if(v + (a.bias ? a.bias[g * a.Cout_g + k] : 0.f), a.relu);
        }
}

constexpr int kTileFloats = 12288;  // 48 KiB of LDS per block

bool plan(TileArgs& a, size_t* lds)
{
    if (a.Cout_g > 32 || a.Cin_g < 1 || a.N < 1) return false;
    const int64_t P = (int64_t)a.Hout * a.Wout;
    if (P >= (1 << 30) || (int64_t)a.Hin * a.Win >= (1 << 30)) return false;
    const int KG = a.Cout_g <= 4 ? 4 : a.Cout_g <= 8 ? 8 : a.Cout_g <= 16 ? 16 : 32;
    const int T = a.kh * a.kw;
    const int64_t R = std::min<int64_t>(a.Hout, 63 / a.Wout + 2);  // output rows a tile touches
    const int64_t LR = (R - 1) * a.sh + (int64_t)(a.kh - 1) * a.dh + 1;
    const int64_t LW = (int64_t)(a.Wout - 1) * a.sw + (int64_t)(a.kw - 1) * a.dw + 1;
    const int64_t per_c = LR * LW + (int64_t)T * KG;
    if (per_c > kTileFloats) return false;
    a.CC = (int)std::min<int64_t>(a.Cin_g, kTileFloats / per_c);
    a.LR = (int)LR;
    a.LW = (int)LW;
    a.tiles = (int)((P + 63) / 64);
    if ((int64_t)a.N * a.G * a.tiles >= (int64_t(1) << 31)) return false;
    *lds = std::max((size_t)a.CC * per_c, (size_t)4 * KG * 64) * sizeof(float);
    return true;
}

bool run(TileArgs& a, hipStream_t st)
{
    size_t lds;
    if (!plan(a, &lds)) return false;
    const int blocks = a.N * a.G * a.tiles;
    if (a.Cout_g <= 4) hipLaunchKernelGGL(direct_tile_kernel<4>, dim3(blocks), dim3(256), lds, st, a);
    else if (a.Cout_g <= 8) hipLaunchKernelGGL(direct_tile_kernel<8>, dim3(blocks), dim3(256), lds, st, a);
    else if (a.Cout_g <= 16) hipLaunchKernelGGL(direct_tile_kernel<16>, dim3(blocks), dim3(256), lds, st, a);
    else hipLaunchKernelGGL(direct_tile_kernel<32>, dim3(blocks), dim3(256), lds, st, a);
    return true;
}

TileArgs fwd_args(const Shape& s, const float* x, const float* w, const float* bias, float* y)
{
    TileArgs a{};
    a.in = x; a.wgt = w; a.bias = bias; a.out = y;
    a.relu = s.relu;
    a.N = s.N; a.G = s.G; a.Cin_tot = s.C; a.Cin_g = s.Cg; a.Hin = s.H; a.Win = s.W;
    a.Cout_tot = s.K; a.Cout_g = s.Kg; a.Hout = s.Ho; a.Wout = s.Wo;
    a.kh = s.kh; a.kw = s.kw; a.sh = s.sh; a.sw = s.sw; a.dh = s.dh; a.dw = s.dw;
    a.ph = s.ph; a.pw = s.pw;
    const int T = s.kh * s.kw;
    a.w_so = s.Cg * T; a.w_sr = T; a.w_gstride = s.Kg * s.Cg * T;
    a.flip = false;
    return a;
}

// gradInput at stride 1: the forward correlation of dy with the transposed,
// tap-reversed filter and padding (k-1)*d - p (which must not be negative).
TileArgs bwd_data_args(const Shape& s, const float* dy, const float* w, float* dx)
{
    TileArgs a{};
    a.in = dy; a.wgt = w; a.bias = nullptr; a.out = dx;
    a.relu = 0;
    a.N = s.N; a.G = s.G; a.Cin_tot = s.K; a.Cin_g = s.Kg; a.Hin = s.Ho; a.Win = s.Wo;
    a.Cout_tot = s.C; a.Cout_g = s.Cg; a.Hout = s.H; a.Wout = s.W;
    a.kh = s.kh; a.kw = s.kw; a.sh = 1; a.sw = 1; a.dh = s.dh; a.dw = s.dw;
    a.ph = (s.kh - 1) * s.dh - s.ph;
    a.pw = (s.kw - 1) * s.dw - s.pw;
    const int T = s.kh * s.kw;
    a.w_so = T; a.w_sr = s.Cg * T; a.w_gstride = s.Kg * s.Cg * T;
    a.flip = true;
    return a;
}

// gradWeight for 3x3 and 5x5 filters with at most KG output channels per group:
// a block owns one (group, input channel) and one slice of the N*Ho*Wo pixels
// and computes its share of dw[g*Kg + k][c][tap] for all k and taps. Threads
// stride over the slice, each keeping KG x KS*KS sums; the block then adds
// them in a fixed order (a butterfly within each wave, then the four waves in
// index order). With one slice the block writes dw; with several, each writes
// its partial to the workspace and direct_wgrad_reduce adds the slices in
// order (depthwise layers have few (group, channel) pairs and long pixel
// reductions: the slices keep every CU busy).
struct WgradArgs {
    Shape s;
    const float* x;
    const float* dy;
    float* out;       // dw, or the workspace [nslice][w_elems]
    int nslice, slice;  // slices per (group, channel) and pixels per slice
};

template <int KG, int KS>
__global__ void __launch_bounds__(256) direct_wgrad_kernel(WgradArgs wa)
{
    constexpr int T = KS * KS;
    __shared__ float red[4][KG * T];
    const Shape& s = wa.s;
    const int pairs = s.G * s.Cg;
    const int gc = blockIdx.x % pairs, ks = blockIdx.x / pairs;
    const int g = gc / s.Cg, c = gc - (gc / s.Cg) * s.Cg;
    const int P = s.Ho * s.Wo;
    const int total = s.N * P;
    const int e0 = ks * wa.slice, e1 = min(total, e0 + wa.slice);
    const size_t HW = (size_t)s.H * s.W;
    float acc[KG * T];
#pragma unroll
    for (int e = 0; e < KG * T; ++e) acc[e] = 0.f;
    for (int e = e0 + threadIdx.x; e < e1; e += 256) {
        const int n = e / P, p = e - (e / P) * P;
        const int ho = p / s.Wo, wo = p - (p / s.Wo) * s.Wo;
        const float* dyp = wa.dy + ((size_t)n * s.K + (size_t)g * s.Kg) * P + p;
        float dv[KG];
#pragma unroll
        for (int k = 0; k < KG; ++k) dv[k] = k < s.Kg ? dyp[(size_t)k * P] : 0.f;
        const float* xc = wa.x + ((size_t)n * s.C + (size_t)g * s.Cg + c) * HW;
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            const int h = ho * s.sh - s.ph + i * s.dh;
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                const int w = wo * s.sw - s.pw + j * s.dw;
                const bool ok = (unsigned)h < (unsigned)s.H && (unsigned)w < (unsigned)s.W;
                const float xv = ok ? xc[(size_t)h * s.W + w] : 0.f;
#pragma unroll
                for (int k = 0; k < KG; ++k)
                    acc[k * T + i * KS + j] = fmaf(dv[k], xv, acc[k * T + i * KS + j]);
            }
        }
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int e = 0; e < KG * T; ++e) {
        float v = acc[e];
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) red[wave][e] = v;
    }
    __syncthreads();
    float* out = wa.out + (size_t)ks * s.w_elems;
    for (int e = threadIdx.x; e < s.Kg * T; e += 256) {
        const int k = e / T, t = e - (e / T) * T;
        out[(((size_t)g * s.Kg + k) * s.Cg + c) * T + t] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
    }
}

// dw[e] = sum of the slices' partials, in slice order.
__global__ void __launch_bounds__(256) direct_wgrad_reduce(const float* __restrict__ ws, float* __restrict__ dw,
                                                           int64_t E, int nslice)
{
    for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < E; e += (int64_t)gridDim.x * 256) {
        float sum = ws[e];
        for (int k = 1; k < nslice; ++k) sum += ws[k * E + e];
        dw[e] = sum;
    }
}

template <int KG, int KS>
void launch_wgrad(const WgradArgs& wa, int blocks, hipStream_t st)
{
    hipLaunchKernelGGL((direct_wgrad_kernel<KG, KS>), dim3(blocks), dim3(256), 0, st, wa);
}

// Slices per (group, input channel): about 2048 blocks in all, each slice at
// least 2048 pixels long.
void wgrad_slices(const Shape& s, int* nslice, int* slice)
{
    const int64_t total = (int64_t)s.N * s.Ho * s.Wo;
    const int64_t pairs = (int64_t)s.G * s.Cg;
    int64_t n = std::min<int64_t>((2048 + pairs - 1) / pairs, std::max<int64_t>(1, total / 2048));
    n = std::max<int64_t>(1, n);
    const int64_t len = (total + n - 1) / n;
    *slice = (int)len;
    *nslice = (int)((total + len - 1) / len);
}

bool wgrad_shape_ok(const Shape& s)
{
    const bool k3 = s.kh == 3 && s.kw == 3, k5 = s.kh == 5 && s.kw == 5;
    if (!(k3 || k5) || s.Kg > (k3 ? 8 : 4) || s.N < 1) return false;
    return (int64_t)s.N * s.Ho * s.Wo < (int64_t(1) << 31) && (int64_t)s.G * s.Cg < (1 << 24);
}

}  // namespace

bool direct_tile_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y,
                     hipStream_t st)
{
    TileArgs a = fwd_args(s, x, w, bias, y);
    return run(a, st);
}

bool direct_tile_bwd_data(const Shape& s, const float* dy, const float* w, float* dx,
                          hipStream_t st)
{
    if (s.sh != 1 || s.sw != 1) return false;
    TileArgs a = bwd_data_args(s, dy, w, dx);
    if (a.ph < 0 || a.pw < 0) return false;
    return run(a, st);
}

size_t direct_tile_bwd_filter_workspace(const Shape& s)
{
    if (!wgrad_shape_ok(s)) return 0;
    int nslice, slice;
    wgrad_slices(s, &nslice, &slice);
    return nslice > 1 ? (size_t)nslice * (size_t)s.w_elems * 4 : 0;
}

bool direct_tile_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws,
                            hipStream_t st)
{
    if (!wgrad_shape_ok(s)) return false;
    WgradArgs wa;
    wa.s = s; wa.x = x; wa.dy = dy;
    wgrad_slices(s, &wa.nslice, &wa.slice);
    if (wa.nslice > 1 && !ws) return false;
    wa.out = wa.nslice > 1 ? ws : dw;
    const int blocks = s.G * s.Cg * wa.nslice;
    const int kg = s.Kg <= 1 ? 1 : s.Kg <= 2 ? 2 : s.Kg <= 4 ? 4 : 8;
    if (s.kh == 3) {
        if (kg == 1) launch_wgrad<1, 3>(wa, blocks, st);
        else if (kg == 2) launch_wgrad<2, 3>(wa, blocks, st);
        else if (kg == 4) launch_wgrad<4, 3>(wa, blocks, st);
        else launch_wgrad<8, 3>(wa, blocks, st);
    } else {
        if (kg == 1) launch_wgrad<1, 5>(wa, blocks, st);
        else if (kg == 2) launch_wgrad<2, 5>(wa, blocks, st);
        else launch_wgrad<4, 5>(wa, blocks, st);
    }
    if (wa.nslice > 1) {
        const int64_t E = s.w_elems;
        const int rb = (int)std::min<int64_t>(1024, (E + 255) / 256);
        hipLaunchKernelGGL(direct_wgrad_reduce, dim3(rb), dim3(256), 0, st, ws, dw, E, wa.nslice);
    }
    return true;
}

}  // namespace gconv
