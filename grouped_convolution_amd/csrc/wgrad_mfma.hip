// wgrad_mfma.hip -- fp32-MFMA gradWeight for grouped 2-D convolution, NCHW.
//
//   dw[g*Kg + k, c, i, j] = sum_{n, ho, wo} dy[n, g*Kg + k, ho, wo]
//                               * x[n, g*Cg + c, ho*sh - ph + i*dh, wo*sw - pw + j*dw]
//
// For every tap (i, j) this is a GEMM over output pixels: rows = the Cg input
// channels, columns = the Kg output channels, reduction = N*Ho*Wo pixels.
// Each wave keeps one 16x16 accumulator per tap and per output-channel
// fragment, so an input value read once from LDS feeds every tap's MFMAs and
// a dy value feeds every tap.
//
//   v_mfma_f32_16x16x4f32: A = 16 input channels x 4 pixels (x at the tap's
//   shifted position), B = 4 pixels x 16 output channels (dy), D: lane l holds
//   dw[c = 4*(l/16)+v][k = l%16].
//
// Block = 4 waves arranged WC (input-channel fragments) x 4/WC, each wave
// 16 input channels x 16*WK output channels x all taps (for the wide 9-tap
// tile, four such sets of 4 waves split each chunk's pixels and add their sums
// at the end, in a fixed order). The pixel reduction
// is split: the N*Ho output rows are cut into chunks of R rows of one image,
// and each block reduces a contiguous run of chunks for one (group, input tile,
// output tile). Blocks write partial tiles to the workspace in accumulator
// order; a second kernel sums the splits in a fixed order and scatters into
// dw, so results are deterministic (no atomics). Tiles are staged global ->
// LDS directly (buffer loads with an LDS destination; out-of-range offsets
// write 0, which is the zero padding), double-buffered so the next chunk
// streams in while this one is multiplied.
#include <algorithm>

#include "device_util.h"
#include "fastdiv.h"
#include "gconv_internal.h"

namespace gconv {
namespace {

constexpr int kMaxSegX = 8;   // 64-float segments of one input-channel plane
constexpr int kMaxSegD = 4;   // ... of one dy plane

struct WgradArgs {
    const float* x;
    const float* dy;
    float* ws;
    int N, C, H, W, K, Ho, Wo, G, Cg, Kg;
    int sh, sw, dh, dw, ph, pw;
    int n_ctiles, n_ktiles, splits;
    int chunks_per_image, chunks_total, chunks_per_split;
    int LW, LR, XS, nsx;    // x tile: row width, rows, plane stride, 64-float segments per plane
    int WoP, DS, nsd;       // dy tile: padded row width, plane stride, segments per plane
    FastDiv div_LW, div_WoP, div_cpi;
};

// Channels-last tiles (INH): x is [N][H][W][C] and dy [N][Ho][Wo][K]. The LDS
// tile of x holds one plane per quad of 4 channels, [pixel][4] (XS floats
// apart, == 8 mod 32), and likewise dy (DS apart); one 16-byte DMA lane brings
// a pixel's quad, so a 64-lane instruction fills 64 pixels of one quad plane
// (nsx, nsd: such segments per quad plane). A half-wave's operand reads (16
// channels as 4 quads x 4, at 2 pixels) then fall in 32 distinct banks.

// The NH wave sets of a block hold sums over disjoint pixels of the same
// tile. They are added down a fixed tree through LDS (the tile buffers are
// free after the chunk loop's last barrier): set h + half hands its sums to
// set h, for half = NH/2, NH/4, .., 1, so set 0 ends with
// ((s0 + s2) + (s1 + s3)) for four sets. Every wave takes part in the
// barriers; returns whether this wave holds the block's total (set 0).
template <int T, int WK, int NH>
__device__ __forceinline__ bool sum_wave_sets(f4 (&acc)[T][WK], float* lds, int wq, int h, int lane)
{
    static_assert(NH == 1 || NH == 2 || NH == 4, "wave sets: 1, 2 or 4");
    constexpr int SLOT = T * WK * 256;  // floats of one wave's sums
#pragma unroll
    for (int half = NH / 2; half >= 1; half /= 2) {
        if (h >= half && h < 2 * half) {
            float* xch = lds + (size_t)((h - half) * 4 + wq) * SLOT + lane;
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int m = 0; m < WK; ++m)
#pragma unroll
                    for (int v = 0; v < 4; ++v) xch[(t * WK + m) * 256 + v * 64] = acc[t][m][v];
        }
        __syncthreads();
        if (h < half) {
            const float* xch = lds + (size_t)(h * 4 + wq) * SLOT + lane;
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int m = 0; m < WK; ++m)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[t][m][v] += xch[(t * WK + m) * 256 + v * 64];
        }
        if (half > 1) __syncthreads();  // the next round's writers reuse the slots
    }
    return h == 0;
}

template <int KH, int KW, int WC, int WK, int R, int NH>
__device__ __forceinline__ void wgrad_nhwc_body(const WgradArgs& a, int kt, int ct, int g, int s, int ch_begin,
                                                int ch_end, int wave, int lane)
{
    constexpr int T = KH * KW;
    constexpr int CT = 16 * WC;
    constexpr int KT = 16 * WK * (4 / WC);
    constexpr int NW = 4 * NH;
    constexpr int CQ = CT / 4, KQ = KT / 4;  // channel quads of the two tiles
    extern __shared__ float lds[];
    const int buf_floats = CQ * a.XS + KQ * a.DS;
    const int l16 = lane & 15, q = lane >> 4;
    const int wq = wave & 3, h = wave >> 2;
    const int wc = wq % WC, wk = wq / WC;
    const int c0 = ct * CT, k0 = kt * KT;
    const int cq_ok = min(CQ, (a.Cg - c0) / 4), kq_ok = min(KQ, (a.Kg - k0) / 4);  // quads inside the group

    // Per-lane pixel parts of the loads: segment sg covers tile pixels
    // 64*sg .. 64*sg + 63 (x: row-major LR x LW; dy: R x WoP).
    int xrow[kMaxSegX], xpix[kMaxSegX];
    bool xok[kMaxSegX];
#pragma unroll
    for (int sg = 0; sg < kMaxSegX; ++sg) {
        const int e = sg * 64 + lane;
        const int r = (int)fastdiv((uint32_t)e, a.div_LW);
        const int w = e - r * a.LW - a.pw;
        xrow[sg] = r;
        xpix[sg] = r * a.W + w;
        xok[sg] = sg < a.nsx && e < a.LR * a.LW && (unsigned)w < (unsigned)a.W;
    }
    int drow[kMaxSegD], dpix[kMaxSegD];
    bool dok[kMaxSegD];
#pragma unroll
    for (int sg = 0; sg < kMaxSegD; ++sg) {
        const int e = sg * 64 + lane;
        const int r = (int)fastdiv((uint32_t)e, a.div_WoP);
        const int col = e - r * a.WoP;
        drow[sg] = r;
        dpix[sg] = r * a.Wo + col;
        dok[sg] = sg < a.nsd && e < R * a.WoP && col < a.Wo;
    }
    const uint32_t ximg = (uint32_t)a.H * a.W * a.C * 4u, dimg = (uint32_t)a.Ho * a.Wo * a.K * 4u;

    // Chunk ch into buffer b: instruction i of the x tile is quad i % CQ,
    // segment i / CQ; this wave takes i = wave, wave + NW, ... (likewise dy).
    auto issue = [&](int ch, int b) {
        float* xs = lds + b * buf_floats;
        float* ds = xs + CQ * a.XS;
        const int n = (int)fastdiv((uint32_t)ch, a.div_cpi);
        const int ho0 = (ch - n * a.chunks_per_image) * R;
        const float* xg = a.x + (size_t)n * a.H * a.W * a.C + (size_t)g * a.Cg + c0;
        const float* dyg = a.dy + (size_t)n * a.Ho * a.Wo * a.K + (size_t)g * a.Kg + k0;
        // (the resources end at the image's last pixel: quads of a pixel past
        // the group's channels are masked below, never read)
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(xg, ximg - (uint32_t)(g * a.Cg + c0) * 4u);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(dyg, dimg - (uint32_t)(g * a.Kg + k0) * 4u);
        const int hb = ho0 * a.sh - a.ph;
        const int row_lo = -hb, row_hi = a.H - hb;
        const int drow_hi = a.Ho - ho0;
        const int xbase = hb * a.W;  // pixels
        const int dbase = ho0 * a.Wo;
        for (int i = wave; i < CQ * a.nsx; i += NW) {
            const int cq = i % CQ, sg = i / CQ;
            uint32_t off = kOOB;
#pragma unroll
            for (int u = 0; u < kMaxSegX; ++u)
                if (u == sg) {
                    const bool ok = cq < cq_ok && xok[u] && xrow[u] >= row_lo && xrow[u] < row_hi;
                    off = ok ? (uint32_t)((xbase + xpix[u]) * a.C + 4 * cq) * 4u : kOOB;
                }
            load_lds256(rx, xs + cq * a.XS + sg * 256, off);
        }
        for (int i = wave; i < KQ * a.nsd; i += NW) {
            const int kq = i % KQ, sg = i / KQ;
            uint32_t off = kOOB;
#pragma unroll
            for (int u = 0; u < kMaxSegD; ++u)
                if (u == sg) {
                    const bool ok = kq < kq_ok && dok[u] && drow[u] < drow_hi;
                    off = ok ? (uint32_t)((dbase + dpix[u]) * a.K + 4 * kq) * 4u : kOOB;
                }
            load_lds256(rd, ds + kq * a.DS + sg * 256, off);
        }
    };

    f4 acc[T][WK];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < WK; ++m) acc[t][m] = f4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = a.WoP / 4;
    // Lane (l16, q): A = x of channel wc*16 + l16 (quad plane, component) at
    // the step's pixel q; B = dy of output channel wk*16*WK + m*16 + l16.
    const int xlane = (wc * 4 + (l16 >> 2)) * a.XS + (l16 & 3) + q * a.sw * 4;
    const int dlane = ((wk * 16 * WK + l16) >> 2) * a.DS + (l16 & 3) + q * 4;
    if (ch_begin < ch_end) issue(ch_begin, 0);
    for (int ch = ch_begin; ch < ch_end; ++ch) {
        const int b = (ch - ch_begin) & 1;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (ch + 1 < ch_end) issue(ch + 1, b ^ 1);
        const float* xs = lds + b * buf_floats;
        const float* ds = xs + CQ * a.XS;
        const int n = (int)fastdiv((uint32_t)ch, a.div_cpi);
        const int ho0 = (ch - n * a.chunks_per_image) * R;
        const int total = min(R, a.Ho - ho0) * nsteps;
        const float* xl = xs + xlane;
        const float* dl = ds + dlane;
        float av[2][T], bv[2][WK];
        auto fetch = [&](int slot, int rr, int ss) {
            const float* xr = xl + (rr * a.sh * a.LW + ss * 4 * a.sw) * 4;
            const float* dr = dl + (rr * a.WoP + ss * 4) * 4;
#pragma unroll
            for (int i = 0; i < KH; ++i) {
                const float* xri = xr + i * a.dh * a.LW * 4;
#pragma unroll
                for (int j = 0; j < KW; ++j) av[slot][i * KW + j] = xri[j * a.dw * 4];
            }
#pragma unroll
            for (int m = 0; m < WK; ++m) bv[slot][m] = dr[m * 4 * a.DS];
        };
        auto mfmas = [&](int slot) {
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int m = 0; m < WK; ++m)
                    acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[slot][t], bv[slot][m],
                                                                     acc[t][m], 0, 0, 0);
        };
        const int u0 = h * total / NH, u1 = (h + 1) * total / NH;
        if (u0 < u1) {
            int fr = u0 / nsteps, fs = u0 - (u0 / nsteps) * nsteps;
            auto advance = [&]() {
                if (++fs == nsteps) {
                    fs = 0;
                    ++fr;
                }
            };
            const int last_r = (u1 - 1) / nsteps, last_s = (u1 - 1) - last_r * nsteps;
            constexpr int NRD = T + WK, NMF = T * WK;
            fetch(0, fr, fs);
            int u = u0;
            for (; u + 1 < u1; u += 2) {
                advance();
                fetch(1, fr, fs);
                mfmas(0);
                __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
                __builtin_amdgcn_sched_barrier(0);
                advance();
                const bool more = u + 2 < u1;
                fetch(0, more ? fr : last_r, more ? fs : last_s);
                mfmas(1);
                __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (u < u1) mfmas(0);
        }
        __syncthreads();
    }

    if (!sum_wave_sets<T, WK, NH>(acc, lds, wq, h, lane)) return;
    const int tile = (g * a.n_ctiles + ct) * a.n_ktiles + kt;
    const int n_tiles = a.G * a.n_ctiles * a.n_ktiles;
    float* out = a.ws + (((size_t)s * n_tiles + tile) * 4 + wq) * (size_t)(T * WK * 256);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < WK; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) out[(t * WK + m) * 256 + v * 64 + lane] = acc[t][m][v];
}

template <int KH, int KW, int WC, int WK, int R, int NH, bool INH = false>
__global__ void __launch_bounds__(256 * NH) wgrad_mfma_kernel(WgradArgs a)
{
    constexpr int T = KH * KW;
    constexpr int CT = 16 * WC;
    constexpr int KT = 16 * WK * (4 / WC);

    extern __shared__ float lds[];
    const int buf_floats = CT * a.XS + KT * a.DS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int l16 = lane & 15, q = lane >> 4;
    // Waves wq = wave % 4 own the output sub-tiles; with NH > 1 further sets
    // of four (h = 1 .. NH - 1) share them, each taking its slice of every
    // chunk's pixels, so NH waves per SIMD hide each other's stalls.
    const int wq = wave & 3, h = wave >> 2;
    const int wc = wq % WC, wk = wq / WC;

    int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int kt = bid % a.n_ktiles;
    bid /= a.n_ktiles;
    const int ct = bid % a.n_ctiles;
    bid /= a.n_ctiles;
    const int g = bid % a.G;
    const int s = bid / a.G;
    const int c0 = ct * CT, k0 = kt * KT;

    const int ch_begin = s * a.chunks_per_split;
    const int ch_end = min(a.chunks_total, ch_begin + a.chunks_per_split);

    if constexpr (INH) {
        wgrad_nhwc_body<KH, KW, WC, WK, R, NH>(a, kt, ct, g, s, ch_begin, ch_end, wave, lane);
        return;
    }
    // Per-lane parts of the tile loads, fixed for the whole kernel: for the
    // segment sg of a plane, this lane's (row, column) inside the tile.
    int xrow[kMaxSegX], xoff[kMaxSegX];
    bool xok[kMaxSegX];
#pragma unroll
    for (int sg = 0; sg < kMaxSegX; ++sg) {
        const int e = sg * 64 + lane;
        const int r = (int)fastdiv((uint32_t)e, a.div_LW);
        const int w = e - r * a.LW - a.pw;
        xrow[sg] = r;
        xoff[sg] = r * a.W + w;
        xok[sg] = sg < a.nsx && e < a.LR * a.LW && (unsigned)w < (unsigned)a.W;
    }
    int drow[kMaxSegD], doff[kMaxSegD];
    bool dok[kMaxSegD];
#pragma unroll
    for (int sg = 0; sg < kMaxSegD; ++sg) {
        const int e = sg * 64 + lane;
        const int r = (int)fastdiv((uint32_t)e, a.div_WoP);
        const int col = e - r * a.WoP;
        drow[sg] = r;
        doff[sg] = r * a.Wo + col;
        dok[sg] = sg < a.nsd && e < R * a.WoP && col < a.Wo;
    }
    const uint32_t xplane = (uint32_t)a.H * a.W * 4u, dplane = (uint32_t)a.Ho * a.Wo * 4u;

    // Issue the loads of chunk `ch` into LDS buffer `b`: plane p of the tile is
    // loaded by wave p % 4, one 64-float segment per instruction.
    // Channels (of x) and output channels (of dy) this wave loads per segment.
    constexpr int CPW = CT / (4 * NH), KPW = KT / (4 * NH);
    auto issue = [&](int ch, int b) {
        float* xs = lds + b * buf_floats;
        float* ds = xs + CT * a.XS;
        const int n = (int)fastdiv((uint32_t)ch, a.div_cpi);
        const int ho0 = (ch - n * a.chunks_per_image) * R;
        const float* xg = a.x + ((size_t)n * a.C + (size_t)g * a.Cg + c0) * a.H * a.W;
        const float* dyg = a.dy + ((size_t)n * a.K + (size_t)g * a.Kg + k0) * a.Ho * a.Wo;
        // Channels past the group end fall outside these resources and read 0.
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(xg, (uint32_t)max(0, min(CT, a.Cg - c0)) * xplane);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(dyg, (uint32_t)max(0, min(KT, a.Kg - k0)) * dplane);
        const int hb = ho0 * a.sh - a.ph;
        const int row_lo = -hb, row_hi = a.H - hb;     // tile rows r with 0 <= hb + r < H
        const int drow_hi = a.Ho - ho0;                // dy rows r with ho0 + r < Ho
        const int xbase = hb * a.W * 4;
        // One select per segment; each of the wave's planes then adds a uniform
        // plane offset (an out-of-range offset stays out of range: the planes
        // a tile spans stay far below 2^31 bytes).
#pragma unroll
        for (int sg = 0; sg < kMaxSegX; ++sg) {
            if (sg >= a.nsx) break;
            const bool ok = xok[sg] && xrow[sg] >= row_lo && xrow[sg] < row_hi;
            const uint32_t v = ok ? (uint32_t)(xbase + xoff[sg] * 4) + (uint32_t)wave * xplane : kOOB;
            float* dst = xs + wave * a.XS + sg * 64;
#pragma unroll
            for (int ci = 0; ci < CPW; ++ci)
                load_lds64(rx, dst + ci * (4 * NH) * a.XS, v + (uint32_t)(ci * 4 * NH) * xplane);
        }
        const int dbase = ho0 * a.Wo * 4;
#pragma unroll
        for (int sg = 0; sg < kMaxSegD; ++sg) {
            if (sg >= a.nsd) break;
            const bool ok = dok[sg] && drow[sg] < drow_hi;
            const uint32_t v = ok ? (uint32_t)(dbase + doff[sg] * 4) + (uint32_t)wave * dplane : kOOB;
            float* dst = ds + wave * a.DS + sg * 64;
#pragma unroll
            for (int ki = 0; ki < KPW; ++ki)
                load_lds64(rd, dst + ki * (4 * NH) * a.DS, v + (uint32_t)(ki * 4 * NH) * dplane);
        }
    };

    f4 acc[T][WK];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < WK; ++m) acc[t][m] = f4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = a.WoP / 4;
    if (ch_begin < ch_end) issue(ch_begin, 0);
    for (int ch = ch_begin; ch < ch_end; ++ch) {
        const int b = (ch - ch_begin) & 1;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of chunk ch landed
        __syncthreads();                                    // ... and every other wave's
        if (ch + 1 < ch_end) issue(ch + 1, b ^ 1);          // next chunk streams in meanwhile
        const float* xs = lds + b * buf_floats;
        const float* ds = xs + CT * a.XS;
        const int n = (int)fastdiv((uint32_t)ch, a.div_cpi);
        const int ho0 = (ch - n * a.chunks_per_image) * R;
        const int total = min(R, a.Ho - ho0) * nsteps;  // (row, 4-pixel step) pairs
        const float* xl = xs + (wc * 16 + l16) * a.XS + q * a.sw;
        const float* dl = ds + (wk * 16 * WK + l16) * a.DS + q;
        // Operands of step u+1 are fetched while the MFMAs of step u run. The
        // fetches are unconditional (the last one re-reads the final step), so
        // the LDS wait before each step covers only that step's operands.
        float av[2][T], bv[2][WK];
        auto fetch = [&](int slot, int rr, int ss) {
            const float* xr = xl + rr * a.sh * a.LW + ss * 4 * a.sw;
            const float* dr = dl + rr * a.WoP + ss * 4;
            if (a.dw == 1) {
                // Unit column dilation: a filter row's taps at immediate offsets.
#pragma unroll
                for (int i = 0; i < KH; ++i) {
                    const float* xri = xr + i * a.dh * a.LW;
#pragma unroll
                    for (int j = 0; j < KW; ++j) av[slot][i * KW + j] = xri[j];
                }
            } else {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int i = t / KW, j = t % KW;
                    av[slot][t] = xr[i * a.dh * a.LW + j * a.dw];
                }
            }
#pragma unroll
            for (int m = 0; m < WK; ++m) bv[slot][m] = dr[m * 16 * a.DS];
        };
        auto mfmas = [&](int slot) {
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int m = 0; m < WK; ++m)
                    acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[slot][t], bv[slot][m],
                                                                     acc[t][m], 0, 0, 0);
        };
        // This wave's steps of the chunk: [u0, u1).
        const int u0 = h * total / NH, u1 = (h + 1) * total / NH;
        if (u0 < u1) {
            // (row, step) of the next fetch, advanced one step at a time.
            int fr = u0 / nsteps, fs = u0 - (u0 / nsteps) * nsteps;
            auto advance = [&]() {
                if (++fs == nsteps) {
                    fs = 0;
                    ++fr;
                }
            };
            const int last_r = (u1 - 1) / nsteps, last_s = (u1 - 1) - last_r * nsteps;
            // Scheduling groups pin the order: the next step's LDS reads, then
            // this step's MFMAs (the compiler would otherwise interleave them and
            // wait on freshly issued reads).
            constexpr int NRD = T + WK, NMF = T * WK;
            fetch(0, fr, fs);
            int u = u0;
            for (; u + 1 < u1; u += 2) {
                advance();
                fetch(1, fr, fs);  // step u+1 (exists)
                mfmas(0);          // step u
                __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
                __builtin_amdgcn_sched_barrier(0);
                advance();
                const bool more = u + 2 < u1;
                fetch(0, more ? fr : last_r, more ? fs : last_s);
                mfmas(1);          // step u+1
                __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (u < u1) mfmas(0);
        }
        __syncthreads();  // every wave is done with buffer b before it is refilled
    }

    if (!sum_wave_sets<T, WK, NH>(acc, lds, wq, h, lane)) return;

    // Partial tile in accumulator order: [split][tile][wave][t][m][v][lane].
    const int tile = (g * a.n_ctiles + ct) * a.n_ktiles + kt;
    const int n_tiles = a.G * a.n_ctiles * a.n_ktiles;
    float* out = a.ws + (((size_t)s * n_tiles + tile) * 4 + wq) * (size_t)(T * WK * 256);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < WK; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) out[(t * WK + m) * 256 + v * 64 + lane] = acc[t][m][v];
}

// dw from the partial tiles. Block = 16 quads of consecutive elements x 16
// split groups: thread (quad, sg) sums splits sg, sg+16, ... in order with
// 16-byte loads; the 16 group sums are then added in order, so the result
// does not depend on scheduling. (per_split is a multiple of 256.)
template <int T, int WC, int WK>
__global__ void __launch_bounds__(256) wgrad_reduce_kernel(const float* __restrict__ ws,
                                                           float* __restrict__ dw, int splits,
                                                           int n_ctiles, int n_ktiles, int Cg,
                                                           int Kg, int per_split)
{
    constexpr int CT = 16 * WC;
    constexpr int KT = 16 * WK * (4 / WC);
    __shared__ f4 part[16][17];
    const int qd = threadIdx.x & 15, sg = threadIdx.x >> 4;
    const int j4 = blockIdx.x * 16 + qd;  // quad index
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
    if (j4 * 4 < per_split) {
        const f4* src = reinterpret_cast<const f4*>(ws) + j4;
        const size_t stride4 = (size_t)per_split / 4;
#pragma unroll 8
        for (int s = sg; s < splits; s += 16) acc += src[(size_t)s * stride4];
    }
    part[sg][qd] = acc;
    __syncthreads();
    if (threadIdx.x >= 64) return;
    // Thread e of the first 64 finishes element 4*qd + e%4 of the block's quads.
    const int q2 = threadIdx.x >> 2, comp = threadIdx.x & 3;
    const int j = (blockIdx.x * 16 + q2) * 4 + comp;
    if (j >= per_split) return;
    float sum = part[0][q2][comp];
#pragma unroll
    for (int i = 1; i < 16; ++i) sum += part[i][q2][comp];
    // j = ((tile*4 + wave)*T + t)*WK*256 + m*256 + v*64 + lane
    const int lane = j & 63, v = (j >> 6) & 3;
    int rest = j >> 8;
    const int m = rest % WK;
    rest /= WK;
    const int t = rest % T;
    rest /= T;
    const int wave = rest & 3;
    const int tile = rest >> 2;
    const int kt = tile % n_ktiles, ct = (tile / n_ktiles) % n_ctiles;
    const int g = tile / (n_ktiles * n_ctiles);
    const int wc = wave % WC, wk = wave / WC;
    const int c = ct * CT + wc * 16 + 4 * (lane >> 4) + v;
    const int k = kt * KT + wk * 16 * WK + m * 16 + (lane & 15);
    if (c < Cg && k < Kg) dw[(((size_t)g * Kg + k) * Cg + c) * T + t] = sum;
}

// ---- host side ----------------------------------------------------------------

struct Config {
    int WC, WK, R, NH;
};

// Plane stride: a multiple of 64 plus 2, so that the 16 channels x 2 pixels a
// half-wave reads in one instruction fall in 32 distinct banks.
int plane_stride(int nseg) { return nseg * 64 + 2; }

struct Plan {
    bool ok;
    Config cfg;
    WgradArgs a;
    int blocks;
    size_t lds_bytes, ws_floats;
    int per_split;
};

Plan make_plan(const Shape& s, bool nhwc = false)
{
    Plan p{};
    p.ok = false;
    // Channels-last tiles move whole quads of a group's channels.
    if (nhwc && ((s.Cg & 3) != 0 || (s.Kg & 3) != 0)) return p;
    const bool k3 = s.kh == 3 && s.kw == 3, k5 = s.kh == 5 && s.kw == 5;
    if (!k3 && !k5) return p;
    if (s.N < 1) return p;
    const int T = s.kh * s.kw;
    Config cfg;
    // Wide tiles (2x2 waves of 16 channels x 32 outputs) where the group has
    // >= 32 input and >= 64 output channels; otherwise one input tile of 16
    // with four waves along the outputs. 25-tap filters keep one input tile
    // per block (their per-wave accumulators already fill 200 registers).
#ifndef GCONV_WGRAD_WIDE
#define GCONV_WGRAD_WIDE 0
#endif
// Wave sets of the wide 9-tap tile: four (16 waves, four a SIMD) measured
// 87.6-88.8 against 90.0-90.3 us on dense3x3's gradWeight with two.
#ifndef GCONV_WGRAD_NH
#define GCONV_WGRAD_NH 4
#endif
    // 9-tap tiles with >= 32 input and output channels per group: two wave
    // sets per block (8 waves) on a 32 x 32 tile whose LDS stays under 80 KiB,
    // so two blocks share a CU and one block's barriers and loads overlap the
    // other's MFMAs.
    int lds_cap = 160 * 1024;
    if (GCONV_WGRAD_WIDE >= 1 && T <= 9 && s.Cg >= 32 && s.Kg >= 32) {
        cfg = {2, 1, 0, 2};
        if (GCONV_WGRAD_WIDE == 1) lds_cap = 80 * 1024;
    } else if (T <= 9 && s.Cg >= 32 && s.Kg >= 64) cfg = {2, 2, 0, GCONV_WGRAD_NH};
    else if (T > 9 && s.Kg >= 128) cfg = {1, 2, 0, 1};
    else cfg = {1, 1, 0, 1};
    const int CT = 16 * cfg.WC, KT = 16 * cfg.WK * (4 / cfg.WC);
    WgradArgs& a = p.a;
    a.WoP = (s.Wo + 3) / 4 * 4;
    a.LW = (s.Wo - 1) * s.sw + (s.kw - 1) * s.dw + 1;
    // Rows per chunk: about 64-112 output pixels, as many as the double-buffered
    // tiles allow in LDS.
    int R = std::max(1, std::min(4, 112 / std::max(1, s.Wo)));
    if (R > s.Ho) R = s.Ho;
    for (;; --R) {
        if (R < 1) return p;
        a.LR = (R - 1) * s.sh + (s.kh - 1) * s.dh + 1;
        // The last quad of a row may reach up to 3 columns (times the stride)
        // past the row end: keep those reads inside the loaded (zero-filled) span.
        const int xspan = a.LR * a.LW + 4 * s.sw;
        a.nsx = (xspan + 63) / 64;
        a.nsd = (R * a.WoP + 63) / 64;
        if (nhwc) {
            // quad planes of 64-pixel segments, 8 floats (mod 32) apart
            a.XS = a.nsx * 256 + 8;
            a.DS = a.nsd * 256 + 8;
            p.lds_bytes = 2 * ((size_t)(CT / 4) * a.XS + (size_t)(KT / 4) * a.DS) * 4;
        } else {
            a.XS = plane_stride(a.nsx);
            a.DS = plane_stride(a.nsd);
            p.lds_bytes = 2 * ((size_t)CT * a.XS + (size_t)KT * a.DS) * 4;
        }
        // The second wave set's sums pass through LDS at the end.
        // The wave sets' sums pass through LDS at the end: NH / 2 sets at once.
        if (cfg.NH > 1) p.lds_bytes = std::max(p.lds_bytes, (size_t)(cfg.NH / 2) * 4 * T * cfg.WK * 256 * 4);
        if (a.nsx <= kMaxSegX && a.nsd <= kMaxSegD && p.lds_bytes <= (size_t)lds_cap) break;
    }
    cfg.R = R;
    a.N = s.N; a.C = s.C; a.H = s.H; a.W = s.W; a.K = s.K; a.Ho = s.Ho; a.Wo = s.Wo;
    a.G = s.G; a.Cg = s.Cg; a.Kg = s.Kg;
    a.sh = s.sh; a.sw = s.sw; a.dh = s.dh; a.dw = s.dw; a.ph = s.ph; a.pw = s.pw;
    a.n_ctiles = (s.Cg + CT - 1) / CT;
    a.n_ktiles = (s.Kg + KT - 1) / KT;
    a.chunks_per_image = (s.Ho + R - 1) / R;
    const int64_t chunks_total = (int64_t)s.N * a.chunks_per_image;
    if (chunks_total >= (1 << 30)) return p;
    a.chunks_total = (int)chunks_total;
    // Tiles are addressed with 32-bit byte offsets below 2^30, including the
    // channels a tile may reach past the end of its group.
    if ((int64_t)(s.Cg + CT) * s.H * s.W * 4 >= (int64_t(1) << 30)) return p;
    if ((int64_t)(s.Kg + KT) * s.Ho * s.Wo * 4 >= (int64_t(1) << 30)) return p;
    // channels-last: one image's pixels, all channels, from one resource
    if (nhwc && ((int64_t)s.H * s.W * s.C * 4 >= (int64_t(1) << 30) ||
                 (int64_t)s.Ho * s.Wo * s.K * 4 >= (int64_t(1) << 30)))
        return p;
    const int n_tiles = s.G * a.n_ctiles * a.n_ktiles;
    // Blocks per CU that fit in LDS, and about that many blocks per CU in total.
    const int per_cu = std::max(1, (int)((160 * 1024) / p.lds_bytes));
    int splits = std::max(1, (256 * std::min(per_cu, 2)) / n_tiles);
    splits = std::min(splits, a.chunks_total);
    a.chunks_per_split = (a.chunks_total + splits - 1) / splits;
    splits = (a.chunks_total + a.chunks_per_split - 1) / a.chunks_per_split;
    a.splits = splits;
    a.div_LW = make_fastdiv((uint32_t)a.LW);
    a.div_WoP = make_fastdiv((uint32_t)a.WoP);
    a.div_cpi = make_fastdiv((uint32_t)a.chunks_per_image);
    const int64_t blocks = (int64_t)n_tiles * splits;
    if (blocks >= (1 << 30)) return p;
    p.blocks = (int)blocks;
    p.per_split = n_tiles * 4 * T * cfg.WK * 256;
    p.ws_floats = (size_t)splits * p.per_split;
    p.cfg = cfg;
    p.ok = true;
    return p;
}

template <int KH, int KW, int WC, int WK, int R, int NH, bool INH = false>
void launch_main(const Plan& p, hipStream_t st)
{
    auto kern = wgrad_mfma_kernel<KH, KW, WC, WK, R, NH, INH>;
    // Allow dynamic LDS up to the CU's 160 KiB (once per kernel instance).
    static const bool attr_set = hipFuncSetAttribute((const void*)kern,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     160 * 1024) == hipSuccess;
    (void)attr_set;
    hipLaunchKernelGGL(kern, dim3(p.blocks), dim3(256 * NH), p.lds_bytes, st, p.a);
}

template <int KH, int KW, int WC, int WK, int NH, bool INH = false>
bool launch_r(const Plan& p, hipStream_t st)
{
    switch (p.cfg.R) {
        case 1: launch_main<KH, KW, WC, WK, 1, NH, INH>(p, st); return true;
        case 2: launch_main<KH, KW, WC, WK, 2, NH, INH>(p, st); return true;
        case 3: launch_main<KH, KW, WC, WK, 3, NH, INH>(p, st); return true;
        case 4: launch_main<KH, KW, WC, WK, 4, NH, INH>(p, st); return true;
        default: return false;
    }
}

template <int T, int WC, int WK>
void launch_reduce(const Plan& p, const Shape& s, float* ws, float* dw, hipStream_t st)
{
    const int blocks = (p.per_split + 63) / 64;
    hipLaunchKernelGGL((wgrad_reduce_kernel<T, WC, WK>), dim3(blocks), dim3(256), 0, st, ws, dw,
                       p.a.splits, p.a.n_ctiles, p.a.n_ktiles, s.Cg, s.Kg, p.per_split);
}

}  // namespace

bool igemm_bwd_filter_supported(const Shape& s) { return make_plan(s).ok; }

size_t igemm_bwd_filter_workspace(const Shape& s)
{
    const Plan p = make_plan(s);
    return p.ok ? p.ws_floats * sizeof(float) : 0;
}

template <bool INH>
static bool run_wgrad(Plan& p, const Shape& s, const float* x, const float* dy, float* dw, float* ws,
                      hipStream_t st)
{
    p.a.x = x;
    p.a.dy = dy;
    p.a.ws = ws;
    const Config c = p.cfg;
    if (s.kh == 3 && c.WC == 2 && c.WK == 2) {
        if (!launch_r<3, 3, 2, 2, GCONV_WGRAD_NH, INH>(p, st)) return false;
        launch_reduce<9, 2, 2>(p, s, ws, dw, st);
    } else if (s.kh == 3 && c.WC == 2 && c.WK == 1) {
        if (!launch_r<3, 3, 2, 1, 2, INH>(p, st)) return false;
        launch_reduce<9, 2, 1>(p, s, ws, dw, st);
    } else if (s.kh == 3 && c.WC == 1 && c.WK == 1) {
        if (!launch_r<3, 3, 1, 1, 1, INH>(p, st)) return false;
        launch_reduce<9, 1, 1>(p, s, ws, dw, st);
    } else if (s.kh == 5 && c.WC == 1 && c.WK == 2) {
        if (!launch_r<5, 5, 1, 2, 1, INH>(p, st)) return false;
        launch_reduce<25, 1, 2>(p, s, ws, dw, st);
    } else if (s.kh == 5 && c.WC == 1 && c.WK == 1) {
        if (!launch_r<5, 5, 1, 1, 1, INH>(p, st)) return false;
        launch_reduce<25, 1, 1>(p, s, ws, dw, st);
    } else {
        return false;
    }
    return true;
}

bool igemm_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws,
                      hipStream_t st)
{
    Plan p = make_plan(s);
    return p.ok && run_wgrad<false>(p, s, x, dy, dw, ws, st);
}

// Channels-last x and dy read in place (s is the NCHW shape of the layer).
bool igemm_bwd_filter_nhwc_supported(const Shape& s) { return make_plan(s, true).ok; }

size_t igemm_bwd_filter_nhwc_workspace(const Shape& s)
{
    const Plan p = make_plan(s, true);
    return p.ok ? p.ws_floats * sizeof(float) : 0;
}

bool igemm_bwd_filter_nhwc(const Shape& s, const float* x, const float* dy, float* dw, float* ws, hipStream_t st)
{
    if (((uintptr_t)x & 15) || ((uintptr_t)dy & 15)) return false;
    Plan p = make_plan(s, true);
    return p.ok && run_wgrad<true>(p, s, x, dy, dw, ws, st);
}

}  // namespace gconv
