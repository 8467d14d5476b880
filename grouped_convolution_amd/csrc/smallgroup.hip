// smallgroup.hip -- grouped 2-D convolution (NCHW fp32) when each group has only
// a few channels (ResNeXt-style 4-in / 4-out groups, depthwise-like shapes).
// Such a layer moves ~9 FLOP per byte, so it is HBM-bound; the point is to read
// x (or dy) once and write y (or dx) once with full-width coalesced accesses,
// while the arithmetic runs on v_mfma_f32_4x4x1f32 (sixteen independent 4x4
// outer products per instruction, the full fp32 matrix rate).
//
// Forward / gradInput (stride 1; gradInput is the forward correlation of dy
// with the transposed, tap-reversed filter):
//   lane l of a wave owns output pixel p0 + l; MFMA block b = l/4 holds pixels
//   4b..4b+3. Per (input channel, tap): A = the filter value of output channel
//   4*oq + l%4 (kept in registers for the whole kernel), B = the input value at
//   the lane's pixel shifted by the tap (LDS), and lane l ends up holding its
//   pixel's four output channels (acc[v] = channel 4*oq + v). One block = 256
//   consecutive output pixels of one (image, group); the input rows they touch
//   (with halo and zero padding) are staged in LDS.
//
// gradWeight: dw[k, c, tap] = sum_pixels dy[k, p] * x[c, p + tap]. MFMA block b
//   takes pixel P + b of a 16-pixel step: A = dy of channel l%4 at that pixel
//   (read straight from memory, reused by all taps), B = x of channel l%4 at the
//   pixel shifted by the tap (LDS). Each block accumulates its own pixels; at
//   the end the 16 blocks are summed across lanes, then the 4 waves through LDS,
//   in a fixed order. One workgroup per (image, group) writes a partial to the
//   workspace and a second kernel sums the images in order.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "fastdiv.h"
#include "device_util.h"
#include "gconv_internal.h"

namespace gconv {
namespace {

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// forward / gradInput
// ---------------------------------------------------------------------------

struct SgArgs {
    const float* in;
    const float* wgt;
    const float* bias;
    float* out;
    int N, G;
    int Cin_tot, Cin_g, Hin, Win;
    int Cout_tot, Cout_g, Hout, Wout;
    int sh, sw, dh, dw, ph, pw;
    int w_so, w_sr, w_gstride;
    int R, nbands;              // output rows per workgroup, bands per plane
    int LW, LR, plane;          // LDS input tile: row width, rows, plane floats
    // Input upsampling (strided gradInput): Hin x Win is the virtual input, in
    // which only rows and columns divisible by uh, uw hold values, row h/uh and
    // column w/uw of the stored Hr x Wr planes; 1, 1 otherwise.
    int uh, uw, Hr, Wr;
    int relu;                   // forward epilogue: max(v, 0)
    FastDiv div_plane, div_LW, div_Wout;
};

// One workgroup = R output rows of one (image, group) plane. Its input rows
// (with halo; zero padding from out-of-range loads) are copied global -> LDS
// directly, so no registers hold staged data and many workgroups per CU keep
// their loads in flight; the filters of this group sit in registers.
template <int KH, int KW, int CIN, int OQ, bool FLIP>
__global__ void __launch_bounds__(256) sg_conv_kernel(SgArgs a)
{
    constexpr int T = KH * KW;
    constexpr int NW = CIN * T * 4 * OQ;     // staged filter values
    extern __shared__ float lds[];           // [CIN][plane] (64-float aligned end), filters
    const int xfloats = (CIN * a.plane + 63) / 64 * 64;
    float* wl = lds + xfloats;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int band = bid % a.nbands;
    bid /= a.nbands;
    const int g = bid % a.G;
    const int n = bid / a.G;
    const int ho0 = band * a.R;
    const int rows = min(a.R, a.Hout - ho0);
    const int hbase = ho0 * a.sh - a.ph;

    const float* in_g = a.in + ((size_t)n * a.Cin_tot + (size_t)g * a.Cin_g) * a.Hr * a.Wr;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(in_g, (uint32_t)a.Cin_g * a.Hr * a.Wr * 4u);
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(a.wgt + (size_t)g * a.w_gstride, (uint32_t)a.w_gstride * 4u);

    // Input tile: element e = c*plane + r*LW + col, 64 per instruction.
    const bool up = a.uh != 1 || a.uw != 1;
    for (int i = wave; i < xfloats / 64; i += 4) {
        const int e = i * 64 + lane;
        const int c = (int)fastdiv((uint32_t)e, a.div_plane);
        const int rem = e - c * a.plane;
        const int r = (int)fastdiv((uint32_t)rem, a.div_LW);
        const int w = rem - r * a.LW - a.pw;
        const int h = hbase + r;
        bool ok = c < CIN && (unsigned)h < (unsigned)a.Hin && (unsigned)w < (unsigned)a.Win;
        int hr = h, wr = w;
        if (up) {   // upsampled input: the other positions are 0
            hr = h / a.uh;
            wr = w / a.uw;
            ok = ok && hr * a.uh == h && wr * a.uw == w;
        }
        load_lds64(rx, lds + i * 64, ok ? (uint32_t)((c * a.Hr + hr) * a.Wr + wr) * 4u : kOOB);
    }
    // Filters -> LDS as [(c*T + t)][o] (zeros past the group's channels).
    for (int e = tid; e < NW; e += 256) {
        const int o = e % (4 * OQ), ct = e / (4 * OQ), c = ct / T, t = ct % T;
        const bool ok = o < a.Cout_g && c < a.Cin_g;
        wl[e] = load_f32(rw, ok ? (uint32_t)(o * a.w_so + c * a.w_sr + (FLIP ? T - 1 - t : t)) * 4u : kOOB);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    float wv[CIN][T][OQ];
#pragma unroll
    for (int c = 0; c < CIN; ++c)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int oq = 0; oq < OQ; ++oq) wv[c][t][oq] = wl[(c * T + t) * 4 * OQ + oq * 4 + (lane & 3)];
    float bv[OQ][4];
#pragma unroll
    for (int oq = 0; oq < OQ; ++oq)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int o = oq * 4 + v;
            bv[oq][v] = (a.bias && o < a.Cout_g) ? a.bias[g * a.Cout_g + o] : 0.f;
        }

    const int P = a.Hout * a.Wout;
    float* out_g = a.out + ((size_t)n * a.Cout_tot + (size_t)g * a.Cout_g) * P + (size_t)ho0 * a.Wout;
    const int npix = rows * a.Wout;
    for (int s = wave * 64; s < npix; s += 256) {
        const int pl = s + lane;
        const int pc = min(pl, npix - 1);
        const int r = (int)fastdiv((uint32_t)pc, a.div_Wout);
        const int base = r * a.sh * a.LW + (pc - r * a.Wout) * a.sw;
        f4 acc[OQ];
#pragma unroll
        for (int oq = 0; oq < OQ; ++oq) acc[oq] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < CIN; ++c)
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int i = t / KW, j = t % KW;
                const float xv = lds[c * a.plane + base + i * a.dh * a.LW + j * a.dw];
#pragma unroll
                for (int oq = 0; oq < OQ; ++oq) acc[oq] = mfma4(wv[c][t][oq], xv, acc[oq]);
            }
        if (pl < npix) {
#pragma unroll
            for (int oq = 0; oq < OQ; ++oq)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int o = oq * 4 + v;
                    if (o < a.Cout_g) out_g[(size_t)o * P + pl] = relu_if(acc[oq][v] + bv[oq][v], a.relu);
                }
        }
    }
}

// Unit stride and dilation, padded rows of at most 64 floats (the common 3x3
// case): the LDS tile keeps one 64-float row per input row, so one DMA
// instruction copies one row (lane = column, a uniform row offset plus the
// lane's column) and every tap read is an LDS load at an immediate offset from
// the pixel's address. The address arithmetic of the general kernel above is
// what limits it at these shapes, not the memory system.
template <int CIN, int OQ, bool FLIP>
__global__ void __launch_bounds__(256) sg_conv_row64_kernel(SgArgs a)
{
    constexpr int T = 9;
    constexpr int NW = CIN * T * 4 * OQ;     // staged filter values
    extern __shared__ float lds[];           // [CIN][LR][64] input rows, then filters
    const int plane = a.LR * 64;
    float* wl = lds + CIN * plane;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int band = bid % a.nbands;
    bid /= a.nbands;
    const int g = bid % a.G;
    const int n = bid / a.G;
    const int ho0 = band * a.R;
    const int rows = min(a.R, a.Hout - ho0);
    const int hbase = ho0 - a.ph;

    const float* in_g = a.in + ((size_t)n * a.Cin_tot + (size_t)g * a.Cin_g) * a.Hin * a.Win;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(in_g, (uint32_t)a.Cin_g * a.Hin * a.Win * 4u);
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(a.wgt + (size_t)g * a.w_gstride, (uint32_t)a.w_gstride * 4u);

    // Tile column `lane` holds input column lane - pw (zero outside the image).
    const int wcol = lane - a.pw;
    const bool colok = (unsigned)wcol < (unsigned)a.Win;
#pragma unroll
    for (int c = 0; c < CIN; ++c)
        for (int r = wave; r < a.LR; r += 4) {
            const int h = hbase + r;
            const bool ok = colok && c < a.Cin_g && (unsigned)h < (unsigned)a.Hin;
            load_lds64(rx, lds + c * plane + r * 64,
                       ok ? (uint32_t)((c * a.Hin + h) * a.Win + wcol) * 4u : kOOB);
        }
    // Filters -> LDS as [(c*T + t)][o] (zeros past the group's channels).
    for (int e = tid; e < NW; e += 256) {
        const int o = e % (4 * OQ), ct = e / (4 * OQ), c = ct / T, t = ct % T;
        const bool ok = o < a.Cout_g && c < a.Cin_g;
        wl[e] = load_f32(rw, ok ? (uint32_t)(o * a.w_so + c * a.w_sr + (FLIP ? T - 1 - t : t)) * 4u : kOOB);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    float wv[CIN][T][OQ];
#pragma unroll
    for (int c = 0; c < CIN; ++c)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int oq = 0; oq < OQ; ++oq) wv[c][t][oq] = wl[(c * T + t) * 4 * OQ + oq * 4 + (lane & 3)];
    float bv[OQ][4];
#pragma unroll
    for (int oq = 0; oq < OQ; ++oq)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int o = oq * 4 + v;
            bv[oq][v] = (a.bias && o < a.Cout_g) ? a.bias[g * a.Cout_g + o] : 0.f;
        }

    const int P = a.Hout * a.Wout;
    float* out_g = a.out + ((size_t)n * a.Cout_tot + (size_t)g * a.Cout_g) * P + (size_t)ho0 * a.Wout;
    const int npix = rows * a.Wout;
    for (int s = wave * 64; s < npix; s += 256) {
        const int pl = s + lane;
        const int pc = min(pl, npix - 1);
        const int r = (int)fastdiv((uint32_t)pc, a.div_Wout);
        const float* xb = lds + r * 64 + (pc - r * a.Wout);
        f4 acc[OQ];
#pragma unroll
        for (int oq = 0; oq < OQ; ++oq) acc[oq] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < CIN; ++c) {
            const float* xc = xb + c * plane;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const float xv = xc[(t / 3) * 64 + t % 3];
#pragma unroll
                for (int oq = 0; oq < OQ; ++oq) acc[oq] = mfma4(wv[c][t][oq], xv, acc[oq]);
            }
        }
        if (pl < npix) {
#pragma unroll
            for (int oq = 0; oq < OQ; ++oq)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int o = oq * 4 + v;
                    // Streaming stores: the output is not read again here, so it
                    // should not displace the input rows neighbouring bands reuse.
                    if (o < a.Cout_g)
                        __builtin_nontemporal_store(relu_if(acc[oq][v] + bv[oq][v], a.relu),
                                                    out_g + (size_t)o * P + pl);
                }
        }
    }
}

// Waits until at most N vector memory instructions of this wave are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until this wave's LDS reads have returned their data. A buffer load
// into LDS writes by another path than the wave's LDS instructions, so a slot
// that was just read is only free for a new DMA after this.
__device__ __forceinline__ void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Depthwise form (one input channel per group, up to 8 outputs): a workgroup
// takes kDwGroups consecutive groups of one band, so that the tiles stay large
// although each group has a single input plane, and every output is a plain
// 9-tap FMA chain on the vector ALUs (the 4x4 MFMA blocks would be at most a
// quarter used here). Same tile as above: one 64-float LDS row per input row,
// lane = pixel, taps at immediate offsets from the pixel's address.
//   S = 2: forward stride 2; output (r, wo) reads LDS rows 2r.., columns 2wo..
//   a.uh, a.uw > 1 (unit stride only): the input is the virtually upsampled
//     dy of a strided gradInput; its rows and columns that are not multiples
//     of the factor are loaded as zeros (out-of-range DMA, no memory traffic).
constexpr int kDwGroups = 4;

template <int MQ, bool FLIP, int S>
__global__ void __launch_bounds__(256) sg_dw_row64_kernel(SgArgs a)
{
    constexpr int T = 9, GB = kDwGroups;
    extern __shared__ float lds[];           // [GB][LR][64] input rows, then [GB][MQ][T] filters
    const int plane = a.LR * 64;
    float* wl = lds + GB * plane;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int band = bid % a.nbands;
    bid /= a.nbands;
    const int ngb = (a.G + GB - 1) / GB;
    const int gb = bid % ngb;
    const int n = bid / ngb;
    const int g0 = gb * GB, ng = min(GB, a.G - g0);
    const int ho0 = band * a.R;
    const int rows = min(a.R, a.Hout - ho0);
    const int hbase = ho0 * S - a.ph;

    // The groups' input planes are consecutive channels of image n (stored
    // planes of Hr x Wr; equal to Hin x Win unless upsampled).
    const int HWr = a.Hr * a.Wr;
    const float* in_n = a.in + ((size_t)n * a.Cin_tot + g0) * HWr;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(in_n, (uint32_t)ng * HWr * 4u);
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(a.wgt + (size_t)g0 * a.w_gstride, (uint32_t)ng * a.w_gstride * 4u);
    // Only gradInput reads an upsampled input.
    const bool up = FLIP && (a.uh != 1 || a.uw != 1);
    const int wcol = lane - a.pw;
    bool colok = (unsigned)wcol < (unsigned)a.Win;
    int wsrc = wcol;
    if (up) {
        wsrc = colok ? wcol / a.uw : 0;
        colok = colok && wsrc * a.uw == wcol;
    }
    const int lrows = (rows - 1) * S + 3;
#pragma unroll
    for (int gi = 0; gi < GB; ++gi)
        for (int r = wave; r < lrows; r += 4) {
            const int h = hbase + r;
            bool ok = colok && gi < ng && (unsigned)h < (unsigned)a.Hin;
            int hs = h;
            if (up) {
                hs = ok ? h / a.uh : 0;
                ok = ok && hs * a.uh == h;
            }
            load_lds64(rx, lds + gi * plane + r * 64,
                       ok ? (uint32_t)((gi * a.Hr + hs) * a.Wr + wsrc) * 4u : kOOB);
        }
    for (int e = tid; e < GB * MQ * T; e += 256) {
        const int gi = e / (MQ * T), o = (e / T) % MQ, t = e % T;
        const bool ok = gi < ng && o < a.Cout_g;
        wl[e] = load_f32(rw, ok ? (uint32_t)(gi * a.w_gstride + o * a.w_so + (FLIP ? T - 1 - t : t)) * 4u : kOOB);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    const size_t P = (size_t)a.Hout * a.Wout;
    const int npix = rows * a.Wout;
    for (int gi = 0; gi < ng; ++gi) {
        float wv[MQ][T], bv[MQ];
#pragma unroll
        for (int o = 0; o < MQ; ++o) {
#pragma unroll
            for (int t = 0; t < T; ++t) wv[o][t] = wl[(gi * MQ + o) * T + t];
            bv[o] = (a.bias && o < a.Cout_g) ? a.bias[(g0 + gi) * a.Cout_g + o] : 0.f;
        }
        float* out_g = a.out + ((size_t)n * a.Cout_tot + (size_t)(g0 + gi) * a.Cout_g) * P + (size_t)ho0 * a.Wout;
        for (int s0 = wave * 64; s0 < npix; s0 += 256) {
            const int pl = s0 + lane;
            const int pc = min(pl, npix - 1);
            const int r = (int)fastdiv((uint32_t)pc, a.div_Wout);
            const float* xb = lds + gi * plane + r * (S * 64) + (pc - r * a.Wout) * S;
            float xv[T];
#pragma unroll
            for (int t = 0; t < T; ++t) xv[t] = xb[(t / 3) * 64 + t % 3];
            if (pl < npix) {
#pragma unroll
                for (int o = 0; o < MQ; ++o) {
                    float acc = 0.f;
#pragma unroll
                    for (int t = 0; t < T; ++t) acc = fmaf(wv[o][t], xv[t], acc);
                    // Write-back stores: non-temporal ones (which skip the
                    // L2's merging of partial lines) measured slower here.
                    if (o < a.Cout_g)
                        out_g[(size_t)o * P + pl] = relu_if(acc + bv[o], a.relu);
                }
            }
        }
    }
}

// Depthwise 3x3 with multiplier 1 at unit stride and dilation, walking down
// the rows: a wave owns 64 / lpw planes side by side (lane = output column of
// plane lane / lpw; lpw = 32 or 16 where rows have at most 30 or 14 outputs)
// and a band of output rows, and streams the band's input rows once each, PF
// rows ahead.
// Input row t of the band adds its tap row i to output row t - i, whose sum
// sits in a ring of three accumulators; output row t - 2 is stored after step
// t. gradInput is the forward of dy with the reversed taps (FLIP). Loads and
// stores are buffer operations whose out-of-range offsets (rows outside the
// image or past the band, columns outside the row, idle lanes) read 0 or are
// dropped, so a band's steps are one straight run of code (the band height is
// a compile-time constant) and the compiler's waits count exactly the rows in
// flight.
struct SgDwWalkArgs {
    const float* in;     // x or dy, planes of Hin x Win
    const float* wgt;    // [C][3][3]
    const float* bias;   // forward only, may be null
    float* out;          // planes of Hout x Wout
    int C, Hin, Win, Hout, Wout, ph, pw, relu;
    int planes;          // N * C
    int lpw_log2;        // lanes per plane: 64, 32 or 16
    int nbands, waves;   // bands of RB output rows per plane
};

// f(integral_constant<int, I>) for each I of the sequence, in order (a loop
// unrolled with the index usable as a constant expression).
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}

template <bool FLIP, int PF, int RB>
__global__ void __launch_bounds__(256) sg_dw_walk_kernel(SgDwWalkArgs a)
{
    constexpr int T = 9;
    constexpr int NS = RB + 2;                   // input rows a band reads
    constexpr int NB = PF + 1;                   // input-row buffers
    // A lane's column offset past its planes (reads 0, stores dropped), and a
    // row offset past everything; their sum stays below 2^32.
    constexpr uint32_t kColOOB = 0x40000000u, kRowOOB = 0x80000000u;
    const int lane = threadIdx.x & 63;
    const int gw = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (gw >= a.waves) return;
    const int band = gw % a.nbands;
    const int pg = gw / a.nbands;
    const int ppw = 64 >> a.lpw_log2;
    const int p0 = pg * ppw;
    const int np = min(ppw, a.planes - p0);
    const int slot = lane >> a.lpw_log2;
    const int wo = lane - (slot << a.lpw_log2);
    const bool live = slot < np && wo < a.Wout;
    const int c = (p0 + min(slot, np - 1)) % a.C;

    float wv[T];
#pragma unroll
    for (int t = 0; t < T; ++t) wv[t] = a.wgt[(size_t)c * T + (FLIP ? T - 1 - t : t)];
    const float b0 = a.bias ? a.bias[c] : 0.f;

    const uint32_t HWi = (uint32_t)a.Hin * a.Win, HWo = (uint32_t)a.Hout * a.Wout;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.in + (size_t)p0 * HWi, (uint32_t)np * HWi * 4u);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.out + (size_t)p0 * HWo, (uint32_t)np * HWo * 4u);
    const int r0 = band * RB;
    const int rows = min(RB, a.Hout - r0);
    const int hb = r0 - a.ph;
    // Lane wo loads input column wo - pw (tap column 0 of its output); tap
    // columns 1 and 2 are the values of lanes wo + 1 and wo + 2, moved down
    // the wave by DPP (lanes past a plane's last output feed only idle ones).
    const int cc = wo - a.pw;
    const uint32_t xcol = slot < np && (unsigned)cc < (unsigned)a.Win ? (uint32_t)(slot * HWi + cc) * 4u : kColOOB;
    const uint32_t ycol = live ? (uint32_t)(slot * HWo + r0 * a.Wout + wo) * 4u : kColOOB;

    // Rows outside the image and past the (last, shorter) band read 0.
    auto load = [&](int t) {
        const int h = hb + t;
        const uint32_t hs = t < rows + 2 && (unsigned)h < (unsigned)a.Hin ? (uint32_t)h * a.Win * 4u : kRowOOB;
        return load_f32(rx, xcol + hs);
    };
    auto down1 = [](float v) {  // lane L takes lane L + 1's value
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x130, 0xF, 0xF, false));
    };

    float acc[3] = {b0, b0, b0};
    float win[NB];
#pragma unroll
    for (int k = 0; k < PF; ++k) win[k] = load(k);
    // Step t: issue row t + PF, add row t's taps, store output row t - 2. The
    // band is unrolled whole (straight-line code: the compiler's waits count
    // exactly the PF rows in flight).
    unroll_seq(
        [&](auto sc) {
            constexpr int t = decltype(sc)::value;
            if constexpr (t + PF < NS) win[(t + PF) % NB] = load(t + PF);
            float v[3];
            v[0] = win[t % NB];
            v[1] = down1(v[0]);
            v[2] = down1(v[1]);
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                float& o = acc[(t - i + 3) % 3];
#pragma unroll
                for (int j = 0; j < 3; ++j) o = fmaf(wv[i * 3 + j], v[j], o);
            }
            // Slot (t + 1) mod 3 is complete (output t - 2), or before step 2
            // holds only the taps of rows above the band's first output.
            float& done = acc[(t + 1) % 3];
            if constexpr (t >= 2)
                store_f32(ry, ycol + (t - 2 < rows ? (uint32_t)(t - 2) * a.Wout * 4u : kRowOOB), relu_if(done, a.relu));
            done = b0;
        },
        std::make_integer_sequence<int, NS>{});
}

// The walk at a forward stride of 2 (3x3, multiplier 1, unit dilation): lane
// L of a plane loads input column L - pw of each input row, and output wo sits
// on lane 2 wo with its tap columns on lanes 2 wo, 2 wo + 1, 2 wo + 2 (DPP
// moves them down). A band of RB output rows reads 2 RB + 1 input rows; input
// row t adds tap row i to output (t - i) / 2 where that divides, so an even
// step starts one output (tap row 0) and ends the one before (tap row 2).
template <int PF, int RB>
__global__ void __launch_bounds__(256) sg_dw_walk_s2_kernel(SgDwWalkArgs a)
{
    constexpr int T = 9;
    constexpr int NS = 2 * RB + 1;
    constexpr int NB = PF + 1;
    constexpr uint32_t kColOOB = 0x40000000u, kRowOOB = 0x80000000u;
    const int lane = threadIdx.x & 63;
    const int gw = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (gw >= a.waves) return;
    const int band = gw % a.nbands;
    const int pg = gw / a.nbands;
    const int ppw = 64 >> a.lpw_log2;
    const int p0 = pg * ppw;
    const int np = min(ppw, a.planes - p0);
    const int slot = lane >> a.lpw_log2;
    const int L = lane - (slot << a.lpw_log2);
    const int wo = L >> 1;
    const bool live = slot < np && (L & 1) == 0 && wo < a.Wout;
    const int c = (p0 + min(slot, np - 1)) % a.C;

    float wv[T];
#pragma unroll
    for (int t = 0; t < T; ++t) wv[t] = a.wgt[(size_t)c * T + t];
    const float b0 = a.bias ? a.bias[c] : 0.f;

    const uint32_t HWi = (uint32_t)a.Hin * a.Win, HWo = (uint32_t)a.Hout * a.Wout;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.in + (size_t)p0 * HWi, (uint32_t)np * HWi * 4u);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.out + (size_t)p0 * HWo, (uint32_t)np * HWo * 4u);
    const int r0 = band * RB;
    const int rows = min(RB, a.Hout - r0);
    const int nin = 2 * rows + 1;
    const int hb = 2 * r0 - a.ph;
    const int cc = L - a.pw;
    const uint32_t xcol = slot < np && (unsigned)cc < (unsigned)a.Win ? (uint32_t)(slot * HWi + cc) * 4u : kColOOB;
    const uint32_t ycol = live ? (uint32_t)(slot * HWo + r0 * a.Wout + wo) * 4u : kColOOB;

    auto load = [&](int t) {
        const int h = hb + t;
        const uint32_t hs = t < nin && (unsigned)h < (unsigned)a.Hin ? (uint32_t)h * a.Win * 4u : kRowOOB;
        return load_f32(rx, xcol + hs);
    };
    auto down1 = [](float v) {  // lane L takes lane L + 1's value
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x130, 0xF, 0xF, false));
    };

    float acc[2] = {b0, b0};
    float win[NB];
#pragma unroll
    for (int k = 0; k < PF; ++k) win[k] = load(k);
    unroll_seq(
        [&](auto sc) {
            constexpr int t = decltype(sc)::value;
            if constexpr (t + PF < NS) win[(t + PF) % NB] = load(t + PF);
            float v[3];
            v[0] = win[t % NB];
            v[1] = down1(v[0]);
            v[2] = down1(v[1]);
            if constexpr (t % 2 == 0) {
                float& o0 = acc[(t / 2) % 2];       // output t / 2, tap row 0
                float& o2 = acc[(t / 2 + 1) % 2];   // output t / 2 - 1, tap row 2
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    o0 = fmaf(wv[j], v[j], o0);
                    o2 = fmaf(wv[6 + j], v[j], o2);
                }
                if constexpr (t >= 2)
                    store_f32(ry, ycol + (t / 2 - 1 < rows ? (uint32_t)(t / 2 - 1) * a.Wout * 4u : kRowOOB),
                              relu_if(o2, a.relu));
                o2 = b0;
            } else {
                float& o1 = acc[(t / 2) % 2];       // output (t - 1) / 2, tap row 1
#pragma unroll
                for (int j = 0; j < 3; ++j) o1 = fmaf(wv[3 + j], v[j], o1);
            }
        },
        std::make_integer_sequence<int, NS>{});
}

// Depthwise gradInput at stride 2 (3x3, multiplier 1, unit dilation) walking
// down dy: lane L of a plane is dx column w = L - 2 and loads dy column
// b = floor((w + pw) / 2) of each dy row; dy column b - 1 is lane L - 2's
// value (DPP moves it up). Tap columns: w + pw even takes j = 0 on column b
// and j = 2 on b - 1, odd takes j = 1 on column b, so with (A_i, B_i) =
// (w_i0, w_i2) or (w_i1, 0), tap row i of dy row r gives
// X_i = A_i d(b) + B_i d(b - 1), and dy row r completes dx rows 2r - ph
// (X_0 plus X_2 of row r - 1) and 2r - ph + 1 (X_1); its X_2 carries to the
// next step. A band of RB dy-row steps starts from the carry of the row
// before it.
struct SgDwWalkDArgs {
    const float* dy;     // planes of Ho x Wo
    const float* wgt;    // [C][3][3]
    float* dx;           // planes of H x W
    int C, H, W, Ho, Wo, ph, pw;
    int planes, lpw_log2;
    int r_lo;            // first dy-row step (dx rows 2 r_lo - ph, + 1)
    int nsteps;          // dy-row steps over all bands
    int nbands, waves;
};

template <int PF, int RB>
__global__ void __launch_bounds__(256) sg_dw_walk_dgrad_s2_kernel(SgDwWalkDArgs a)
{
    constexpr int NS = RB + 1;                  // the carry row, then RB steps
    constexpr int NB = PF + 1;
    constexpr uint32_t kColOOB = 0x40000000u, kRowOOB = 0x80000000u;
    const int lane = threadIdx.x & 63;
    const int gw = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (gw >= a.waves) return;
    const int band = gw % a.nbands;
    const int pg = gw / a.nbands;
    const int ppw = 64 >> a.lpw_log2;
    const int p0 = pg * ppw;
    const int np = min(ppw, a.planes - p0);
    const int slot = lane >> a.lpw_log2;
    const int w = lane - (slot << a.lpw_log2) - 2;
    const bool live = slot < np && w >= 0 && w < a.W;
    const int c = (p0 + min(slot, np - 1)) % a.C;
    const int par = (w + a.pw) & 1;
    const int bcol = (w + a.pw) >> 1;           // arithmetic shift: floor

    float A[3], B[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const float* wr = a.wgt + (size_t)c * 9 + i * 3;
        A[i] = par ? wr[1] : wr[0];
        B[i] = par ? 0.f : wr[2];
    }

    const uint32_t HWi = (uint32_t)a.Ho * a.Wo, HWo = (uint32_t)a.H * a.W;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dy + (size_t)p0 * HWi, (uint32_t)np * HWi * 4u);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.dx + (size_t)p0 * HWo, (uint32_t)np * HWo * 4u);
    const int s0 = band * RB;                   // first step of the band
    const int nst = min(RB, a.nsteps - s0);
    const int rb = a.r_lo + s0;                 // its first dy row
    const uint32_t dcol = slot < np && bcol >= 0 && bcol < a.Wo ? (uint32_t)(slot * HWi + bcol) * 4u : kColOOB;
    const uint32_t xcol = live ? (uint32_t)(slot * HWo + w) * 4u : kColOOB;

    // Step k reads dy row rb - 1 + k (k = 0: the carry row).
    auto load = [&](int k) {
        const int r = rb - 1 + k;
        const uint32_t rs = k <= nst && (unsigned)r < (unsigned)a.Ho ? (uint32_t)r * a.Wo * 4u : kRowOOB;
        return load_f32(rd, dcol + rs);
    };
    auto up2 = [](float v) {  // lane L takes lane L - 2's value
        const int x = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x138, 0xF, 0xF, false);
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x138, 0xF, 0xF, false));
    };
    auto row_store = [&](int h, float v) {
        const uint32_t hs = (unsigned)h < (unsigned)a.H ? (uint32_t)h * a.W * 4u : kRowOOB;
        store_f32(rx, xcol + hs, v);
    };

    float carry = 0.f;
    float win[NB];
#pragma unroll
    for (int k = 0; k < PF; ++k) win[k] = load(k);
    unroll_seq(
        [&](auto sc) {
            constexpr int k = decltype(sc)::value;
            if constexpr (k + PF < NS) win[(k + PF) % NB] = load(k + PF);
            const float d0 = win[k % NB];
            const float d1 = up2(d0);
            const float x2 = fmaf(B[2], d1, A[2] * d0);
            if constexpr (k > 0) {
                const int r = rb - 1 + k;
                const bool in_band = k <= nst;
                const float x0 = fmaf(B[0], d1, fmaf(A[0], d0, carry));
                const float x1 = fmaf(B[1], d1, A[1] * d0);
                row_store(in_band ? 2 * r - a.ph : -1, x0);
                row_store(in_band ? 2 * r - a.ph + 1 : -1, x1);
            }
            carry = x2;
        },
        std::make_integer_sequence<int, NS>{});
}

// Depthwise gradInput at stride 2 (3x3, dilation 1, one input and one output
// channel per group), split by output phase. With h + ph = 2a + u and
// w + pw = 2b + v (u, v in {0, 1}), dx[h][w] takes dy rows a (tap row u) and,
// for u = 0, a - 1 (tap row 2); columns likewise. So the four dx of (a, b)
//   (0,0): w00 D(a,b) + w02 D(a,b-1) + w20 D(a-1,b) + w22 D(a-1,b-1)
//   (0,1): w01 D(a,b) + w21 D(a-1,b)
//   (1,0): w10 D(a,b) + w12 D(a,b-1)
//   (1,1): w11 D(a,b)
// where D is dy, 0 outside it. A lane owns dx column w of phase row a and
// writes its two dx rows (stores stay contiguous across lanes): with
// (A, B) = (w_i0, w_i2) for v = 0 and (w_i1, 0) for v = 1, tap row i gives
// A D(., b) + B D(., b-1). A workgroup takes kDwGroups consecutive groups of
// one band of a; LDS row k of a group holds dy row a_lo - 1 + k with dy
// column m at position m + 1 (position 0, and rows and columns outside dy,
// hold 0).
struct SgDw2Args {
    const float* dy;
    const float* wgt;
    float* dx;
    int N, G, H, W, Ho, Wo, ph, pw;
    int a_min, na;              // phase rows a covering dx
    int RA, nbands;             // values of a per workgroup, bands per plane
    FastDiv div_W;
};

__global__ void __launch_bounds__(256) sg_dw_dgrad_s2_kernel(SgDw2Args a)
{
    constexpr int GB = kDwGroups;
    extern __shared__ float lds[];  // [GB][RA + 1][64] dy rows, then [GB][9] filters
    const int plane = (a.RA + 1) * 64;
    float* wl = lds + GB * plane;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int band = bid % a.nbands;
    bid /= a.nbands;
    const int ngb = (a.G + GB - 1) / GB;
    const int gb = bid % ngb;
    const int n = bid / ngb;
    const int g0 = gb * GB, ng = min(GB, a.G - g0);
    const int a_lo = a.a_min + band * a.RA;
    const int ra = min(a.RA, a.a_min + a.na - a_lo);

    const int HWo = a.Ho * a.Wo;
    const float* dy_n = a.dy + ((size_t)n * a.G + g0) * HWo;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dy_n, (uint32_t)ng * HWo * 4u);
    const int m = lane - 1;  // dy column of LDS position `lane`
    const bool colok = (unsigned)m < (unsigned)a.Wo;
#pragma unroll
    for (int gi = 0; gi < GB; ++gi)
        for (int k = wave; k <= ra; k += 4) {
            const int hd = a_lo - 1 + k;
            const bool ok = colok && gi < ng && (unsigned)hd < (unsigned)a.Ho;
            load_lds64(rd, lds + gi * plane + k * 64, ok ? (uint32_t)((gi * a.Ho + hd) * a.Wo + m) * 4u : kOOB);
        }
    if (tid < GB * 9) {
        const int gi = tid / 9;
        wl[tid] = gi < ng ? a.wgt[(size_t)(g0 + gi) * 9 + tid % 9] : 0.f;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    const size_t HW = (size_t)a.H * a.W;
    const int npos = ra * a.W;
    // The (group, 64-position chunk) pairs are dealt to the waves in turn, so
    // that the four waves get equal shares of the workgroup's chunks.
    const int nch = (npos + 63) >> 6;
    for (int c = wave; c < ng * nch; c += 4) {
        const int gi = c / nch;
        float wv[9];
#pragma unroll
        for (int t = 0; t < 9; ++t) wv[t] = wl[gi * 9 + t];
        float* dx_g = a.dx + ((size_t)n * a.G + g0 + gi) * HW;
        {
            const int pl = (c - gi * nch) * 64 + lane;
            const int pc = min(pl, npos - 1);
            const int r = (int)fastdiv((uint32_t)pc, a.div_W);
            const int w = pc - r * a.W;
            const int b = (w + a.pw) >> 1;
            const bool odd = (w + a.pw) & 1;
            // Tap columns: (A, B) act on dy columns b and b - 1.
            const float A0 = odd ? wv[1] : wv[0], B0 = odd ? 0.f : wv[2];
            const float A1 = odd ? wv[4] : wv[3], B1 = odd ? 0.f : wv[5];
            const float A2 = odd ? wv[7] : wv[6], B2 = odd ? 0.f : wv[8];
            // Row r + 1 is dy row a = a_lo + r, row r is a - 1; position b + 1
            // is dy column b, position b is b - 1.
            const float* L = lds + gi * plane + r * 64 + b;
            const float d11 = L[64 + 1], d10 = L[64], d01 = L[1], d00 = L[0];
            const float y0 = fmaf(B2, d00, fmaf(A2, d01, fmaf(B0, d10, A0 * d11)));
            const float y1 = fmaf(B1, d10, A1 * d11);
            if (pl < npos) {
                const int h0 = 2 * (a_lo + r) - a.ph;
                float* o = dx_g + (size_t)h0 * a.W + w;
                if ((unsigned)h0 < (unsigned)a.H) __builtin_nontemporal_store(y0, o);
                if ((unsigned)(h0 + 1) < (unsigned)a.H) __builtin_nontemporal_store(y1, o + a.W);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// gradWeight
// ---------------------------------------------------------------------------

struct SgWArgs {
    const float* x;
    const float* dy;
    float* ws;
    int N, C, H, W, K, Ho, Wo, G, Cg, Kg;
    int sh, sw, dh, dw, ph, pw;
    int R, nbands, LW, LR, plane;   // input band
    int dplane;                     // dy band plane stride (== 8 mod 32)
    int run, nruns;                 // row-per-DMA kernel: images per workgroup, workgroups per group
    FastDiv div_plane, div_LW, div_Wo, div_dband;
};

// One workgroup per (image, group, band of R output rows): the band's input
// rows and dy rows are copied global -> LDS directly; 16-pixel MFMA steps are
// spread over the four waves. Partial sums go to the workspace per band.
template <int KH, int KW>
__global__ void __launch_bounds__(256) sg_wgrad_kernel(SgWArgs a)
{
    constexpr int T = KH * KW;
    extern __shared__ float lds[];  // [4][plane] input, [4][dplane] dy; later [4][T*16] sums
    const int xfloats = (4 * a.plane + 63) / 64 * 64;
    float* ds = lds + xfloats;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c4 = lane & 3, blk = lane >> 2;  // this lane's channel (c and k), MFMA block

    int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int band = bid % a.nbands;
    bid /= a.nbands;
    const int g = bid % a.G;
    const int n = bid / a.G;
    const int ho0 = band * a.R;
    const int rows = min(a.R, a.Ho - ho0);
    const int hb = ho0 * a.sh - a.ph;
    const int npix = rows * a.Wo;

    const float* xg = a.x + ((size_t)n * a.C + (size_t)g * a.Cg) * a.H * a.W;
    const float* dyg = a.dy + ((size_t)n * a.K + (size_t)g * a.Kg) * a.Ho * a.Wo + (size_t)ho0 * a.Wo;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xg, (uint32_t)a.Cg * a.H * a.W * 4u);
    // dy rows of this band, channel stride Ho*Wo; the resource ends after the
    // group's last channel so channels past Kg read 0.
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc(dyg, (uint32_t)(((a.Kg - 1) * a.Ho + (a.Ho - ho0)) * a.Wo) * 4u);

    for (int i = wave; i < xfloats / 64; i += 4) {
        const int e = i * 64 + lane;
        const int c = (int)fastdiv((uint32_t)e, a.div_plane);
        const int rem = e - c * a.plane;
        const int r = (int)fastdiv((uint32_t)rem, a.div_LW);
        const int w = rem - r * a.LW - a.pw;
        const int h = hb + r;
        const bool ok = c < 4 && (unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W;
        load_lds64(rx, lds + i * 64, ok ? (uint32_t)((c * a.H + h) * a.W + w) * 4u : kOOB);
    }
    // dy band: per channel, R*Wo contiguous floats into a plane of dplane.
    const int nseg = (a.dplane - 8) / 64;  // dplane = 64*nseg + 8: segments stay in the plane
    for (int i = wave; i < 4 * nseg; i += 4) {
        const int k = i / nseg, sg = i - k * nseg;
        const int e = sg * 64 + lane;
        const bool ok = k < a.Kg && e < npix;
        load_lds64(rd, ds + k * a.dplane + sg * 64,
                   ok ? (uint32_t)(k * a.Ho * a.Wo + e) * 4u : kOOB);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    f4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
    for (int s = wave * 16; s < npix; s += 64) {
        const int pl = min(s + blk, npix - 1);
        const float dv = (s + blk < npix) ? ds[c4 * a.dplane + pl] : 0.f;
        const int r = (int)fastdiv((uint32_t)pl, a.div_Wo);
        const int base = c4 * a.plane + r * a.sh * a.LW + (pl - r * a.Wo) * a.sw;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int ii = t / KW, jj = t % KW;
            acc[t] = mfma4(dv, lds[base + ii * a.dh * a.LW + jj * a.dw], acc[t]);
        }
    }

    // acc[t][v] of lane l = sum over its block's pixels of dy[k = v] * x[c = l%4].
    // Sum the 16 blocks (lanes with equal l%4), in a fixed butterfly order.
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float sum = acc[t][v];
            sum += __shfl_xor(sum, 4, 64);
            sum += __shfl_xor(sum, 8, 64);
            sum += __shfl_xor(sum, 16, 64);
            sum += __shfl_xor(sum, 32, 64);
            acc[t][v] = sum;
        }
    __syncthreads();  // LDS reuse for the cross-wave sum
    float* red = lds;  // [wave][t][k(4)][c(4)]
    if (lane < 4) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[(wave * T + t) * 16 + v * 4 + lane] = acc[t][v];
    }
    __syncthreads();
    // Partial of this (image, band, group): [(n*nbands + band)][g][k][c][t].
    float* out = a.ws + (((size_t)n * a.nbands + band) * a.G + g) * (16 * T);
    for (int e = tid; e < 16 * T; e += 256) {
        const int t = e % T, kc = e / T;  // kc = k*4 + c
        const float sum = ((red[(0 * T + t) * 16 + kc] + red[(1 * T + t) * 16 + kc]) +
                           red[(2 * T + t) * 16 + kc]) +
                          red[(3 * T + t) * 16 + kc];
        out[kc * T + t] = sum;
    }
}

// Unit stride and dilation, padded rows of at most 64 floats. A workgroup owns
// one group and a run of images (a.R images from image n0), loops over their
// bands and keeps its sums in registers, so the cross-lane reduction runs
// once per workgroup. Bands of x and dy are staged one row per DMA
// instruction ([4][rows][64] planes, padded to 8 mod 32 so the 4 channels x 8
// pixels of a half-wave hit distinct banks). Each wave walks whole output
// rows in 16-pixel steps (MFMA block b = pixel b of the step; columns past the
// image width hold dy = 0), so a step costs one dy read, nine x reads at
// immediate offsets and nine MFMAs. At most 128 registers a lane (74 in
// practice, no spills), so that the 1024 workgroups of a ResNeXt 32x4d layer
// (four per CU) are resident at once: at 148 registers three fitted, and the
// fourth workgroup of each CU ran alone in a second round (61.3 -> 59.8 us).
// (Double-buffered bands, two workgroups per CU at 62 KB of LDS each,
// measured 67.9 us: four resident workgroups hide each other's copies better.)
template <int NSTEP>
__global__ void __launch_bounds__(256, 4) sg_wgrad_row64_kernel(SgWArgs a)
{
    constexpr int T = 9;
    extern __shared__ float lds[];  // [4][plane] x rows, [4][dplane] dy rows; later [4][T*16] sums
    float* ds = lds + 4 * a.plane;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c4 = lane & 3, blk = lane >> 2;  // this lane's channel (c and k), MFMA block

    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int g = bid % a.G;
    const int chunk = bid / a.G;               // image run
    const int n_begin = chunk * a.run;
    const int n_end = min(a.N, n_begin + a.run);

    const int wcol = lane - a.pw;
    const bool colok = (unsigned)wcol < (unsigned)a.W;
    // Lanes past the image width may read up to two floats beyond the last x
    // row of a plane (times dy = 0): keep the pad after each plane zero.
    if (tid < 32) lds[(tid >> 3) * a.plane + (a.R + 2) * 64 + (tid & 7)] = 0.f;

    f4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
    const float* xl = lds + c4 * a.plane + blk;
    const float* dl = ds + c4 * a.dplane + blk;

    for (int n = n_begin; n < n_end; ++n) {
        const float* xg = a.x + ((size_t)n * a.C + (size_t)g * a.Cg) * a.H * a.W;
        const float* dyg = a.dy + ((size_t)n * a.K + (size_t)g * a.Kg) * a.Ho * a.Wo;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(xg, (uint32_t)a.Cg * a.H * a.W * 4u);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(dyg, (uint32_t)a.Kg * a.Ho * a.Wo * 4u);
        for (int ho0 = 0; ho0 < a.Ho; ho0 += a.R) {
            const int rows = min(a.R, a.Ho - ho0);
            const int hb = ho0 - a.ph;
            const int LR = rows + 2;
            __syncthreads();  // every wave is done with the previous band
#pragma unroll
            for (int c = 0; c < 4; ++c)
                for (int r = wave; r < LR; r += 4) {
                    const int h = hb + r;
                    const bool ok = colok && c < a.Cg && (unsigned)h < (unsigned)a.H;
                    load_lds64(rx, lds + c * a.plane + r * 64,
                               ok ? (uint32_t)((c * a.H + h) * a.W + wcol) * 4u : kOOB);
                }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                for (int r = wave; r < rows; r += 4) {
                    // Rows of the band only; channels past Kg fall outside the resource.
                    load_lds64(rd, ds + k * a.dplane + r * 64,
                               lane < a.Wo ? (uint32_t)((k * a.Ho + ho0 + r) * a.Wo + lane) * 4u : kOOB);
                }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            for (int r = wave; r < rows; r += 4) {
                const float* xr = xl + r * 64;
                const float* dr = dl + r * 64;
#pragma unroll
                for (int st = 0; st < NSTEP; ++st) {
                    const float dv = dr[st * 16];
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        acc[t] = mfma4(dv, xr[st * 16 + (t / 3) * 64 + t % 3], acc[t]);
                }
            }
        }
    }

    // acc[t][v] of lane l = sum over its block's pixels of dy[k = v] * x[c = l%4].
    // Sum the 16 blocks (lanes with equal l%4), in a fixed butterfly order.
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float sum = acc[t][v];
            sum += __shfl_xor(sum, 4, 64);
            sum += __shfl_xor(sum, 8, 64);
            sum += __shfl_xor(sum, 16, 64);
            sum += __shfl_xor(sum, 32, 64);
            acc[t][v] = sum;
        }
    __syncthreads();  // LDS reuse for the cross-wave sum
    float* red = lds;  // [wave][t][k(4)][c(4)]
    if (lane < 4) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[(wave * T + t) * 16 + v * 4 + lane] = acc[t][v];
    }
    __syncthreads();
    // Partial of this (image run, group): [chunk][g][k][c][t].
    float* out = a.ws + ((size_t)chunk * a.G + g) * (16 * T);
    for (int e = tid; e < 16 * T; e += 256) {
        const int t = e % T, kc = e / T;  // kc = k*4 + c
        out[e] = ((red[(0 * T + t) * 16 + kc] + red[(1 * T + t) * 16 + kc]) +
                  red[(2 * T + t) * 16 + kc]) +
                 red[(3 * T + t) * 16 + kc];
    }
}

// Streaming form of the gradWeight kernel above, for 3x3 filters at stride 1
// or 2 with up to 8 input and 8 output channels per group (CQ and KQ quads of
// 4: each (k quad, c quad) pair is a 4x4 block of the 4x4x1 MFMA, kept in its
// own accumulators). A workgroup owns one group; its four waves stream units
// (one band of one image each) independently, each through rings in its own
// LDS slice: input rows and dy rows, 72 floats per channel (== 8 mod 32, so
// the 4 channels x 8 pixels of a half-wave read distinct banks at stride 1).
// Stream step j loads input rows S*j .. S*j + S - 1 and dy row j - D, D the
// steps until an output row's three input rows are all in (2 at stride 1, 1
// at stride 2). Step i + D + PF + 1 is issued when output row i is done, into
// the slots that row no longer needs, so PF steps stay in flight behind the
// row being summed and no barrier ties the waves together until the final
// cross-wave sum. Every step past the first D issues the same DMA rows (past
// the band: out-of-range zeros into freed slots), so the wait for a step
// counts exactly the PF steps after it.
struct SgWStreamArgs {
    const float* x;
    const float* dy;
    float* ws;
    int N, C, H, W, K, Ho, Wo, G, Cg, Kg;
    int ph, pw;
    int R, nbands;              // output rows per band, bands per image
    int upw, nchunks;           // units (image, band) per wave, workgroups per group
};

// (8 x 8 channels: 144 accumulators a lane; at most 256 registers keep two
// workgroups per CU.)
template <int NSTEP, int PF, int S, int CQ, int KQ>
__global__ void __launch_bounds__(256, (CQ * KQ > 1 ? 2 : 1)) sg_wgrad_stream_kernel(SgWStreamArgs a)
{
    constexpr int T = 9;
    constexpr int D = S == 1 ? 2 : 1;
    constexpr int RX = S * (D + 1 + PF), RD = PF + 1;  // input-row and dy-row slots
    constexpr int CS = 72;                              // channel stride of a slot
    constexpr int XSLOT = 4 * CQ * CS, DSLOT = 4 * KQ * CS;
    constexpr int WLDS = RX * XSLOT + RD * DSLOT;
    constexpr int NDMA = S * 4 * CQ + 4 * KQ;          // DMA rows per step
    extern __shared__ float lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c4 = lane & 3, blk = lane >> 2;  // this lane's channel in a quad (c and k), MFMA block
    float* xring = lds + wave * WLDS;
    float* dring = xring + RX * XSLOT;

    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int g = bid % a.G;
    const int chunk = bid / a.G;
    const int units = a.N * a.nbands;

    // Columns 64..71 of the input slots are never loaded: zero them once
    // (lanes past the output width read up to column 64 + S - 1, times dy = 0).
    for (int e = lane; e < RX * 4 * CQ * 8; e += 64) xring[(e >> 3) * CS + 64 + (e & 7)] = 0.f;

    const int wcol = lane - a.pw;
    const bool colok = (unsigned)wcol < (unsigned)a.W;
    f4 acc[KQ][CQ][T];
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
        for (int cq = 0; cq < CQ; ++cq)
#pragma unroll
            for (int t = 0; t < T; ++t) acc[kq][cq][t] = f4{0.f, 0.f, 0.f, 0.f};

    for (int k = 0; k < a.upw; ++k) {
        const int u = (chunk * a.upw + k) * 4 + wave;
        if (u >= units) break;
        const int n = u / a.nbands, band = u - n * a.nbands;
        const int r0 = band * a.R;
        const int rows = min(a.R, a.Ho - r0);
        const int nin = S * (rows - 1) + 3;   // input rows of the band
        const int hfirst = S * r0 - a.ph;
        const float* xg = a.x + ((size_t)n * a.C + (size_t)g * a.Cg) * a.H * a.W;
        const float* dyg = a.dy + ((size_t)n * a.K + (size_t)g * a.Kg) * a.Ho * a.Wo;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(xg, (uint32_t)a.Cg * a.H * a.W * 4u);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(dyg, (uint32_t)a.Kg * a.Ho * a.Wo * 4u);
        // Step j: input rows S*j .. into slots sx, sx + 1 (S = 2: sx is even,
        // RX too, so no wrap), dy row j - D into slot sd. One lane offset per
        // row; the channel's plane offset rides in the scalar offset, and
        // channels past the group fall outside the resource (read 0).
        const uint32_t xplane = (uint32_t)a.H * a.W * 4u, dplane = (uint32_t)a.Ho * a.Wo * 4u;
        auto issue_step = [&](int j, int sx, int sd, bool with_dy) {
#pragma unroll
            for (int r = 0; r < S; ++r) {
                const int jj = S * j + r, h = hfirst + jj;
                const bool okx = colok && jj < nin && (unsigned)h < (unsigned)a.H;
                const uint32_t off = okx ? (uint32_t)(h * a.W + wcol) * 4u : kOOB;
#pragma unroll
                for (int c = 0; c < 4 * CQ; ++c) load_lds64s(rx, xring + (sx + r) * XSLOT + c * CS, off, c * xplane);
            }
            if (with_dy) {
                const int d = j - D;
                const uint32_t off = (lane < a.Wo && d < rows) ? (uint32_t)((r0 + d) * a.Wo + lane) * 4u : kOOB;
#pragma unroll
                for (int kk = 0; kk < 4 * KQ; ++kk) load_lds64s(rd, dring + sd * DSLOT + kk * CS, off, kk * dplane);
            }
        };
        // Steps 0 .. D - 1 carry no dy row; steps D .. D + PF carry dy rows 0 .. PF.
#pragma unroll
        for (int j = 0; j < D; ++j) issue_step(j, S * j, 0, false);
#pragma unroll
        for (int j = D; j <= D + PF; ++j) issue_step(j, S * j, j - D, true);

        int sx0 = 0, sd0 = 0;  // slots of input row S*i and dy row i
        for (int i = 0; i < rows; ++i) {
            wait_vmcnt<PF * NDMA>();  // step i + D landed: PF steps follow it
            int sx[3];
#pragma unroll
            for (int ti = 0; ti < 3; ++ti) sx[ti] = sx0 + ti >= RX ? sx0 + ti - RX : sx0 + ti;
#pragma unroll
            for (int st = 0; st < NSTEP; ++st) {
                float dv[KQ];
#pragma unroll
                for (int kq = 0; kq < KQ; ++kq) dv[kq] = dring[sd0 * DSLOT + (kq * 4 + c4) * CS + st * 16 + blk];
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    float xv[CQ];
#pragma unroll
                    for (int cq = 0; cq < CQ; ++cq)
                        xv[cq] = xring[sx[t / 3] * XSLOT + (cq * 4 + c4) * CS + S * (st * 16 + blk) + t % 3];
#pragma unroll
                    for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
                        for (int cq = 0; cq < CQ; ++cq) acc[kq][cq][t] = mfma4(dv[kq], xv[cq], acc[kq][cq][t]);
                }
            }
            // Input rows S*i .. S*i + S - 1 and dy row i are no longer read:
            // step i + D + PF + 1 reuses their slots. Their LDS reads must
            // have returned first: a DMA whose rows are out of range writes
            // its zeros without a memory access, soon enough to land ahead of
            // a read still queued at the LDS.
            lds_reads_done();
            issue_step(i + D + PF + 1, sx0, sd0, true);
            sx0 = sx0 + S >= RX ? sx0 + S - RX : sx0 + S;
            sd0 = sd0 + 1 == RD ? 0 : sd0 + 1;
        }
    }

    // acc[kq][cq][t][v] of lane l = sum over its block's pixels of
    // dy[k = 4 kq + v] * x[c = 4 cq + l%4]. Sum the 16 blocks (lanes with
    // equal l%4), in a fixed butterfly order, each sum going straight to this
    // wave's own LDS slice (its rings are idle once the tail's zero rows have
    // landed), so the accumulators die one by one.
    constexpr int KC = 16 * KQ * CQ;  // (k, c) pairs of the partial
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    float* red = xring;               // [k][c][t] of this wave
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
        for (int cq = 0; cq < CQ; ++cq)
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float sum = acc[kq][cq][t][v];
                    sum += __shfl_xor(sum, 4, 64);
                    sum += __shfl_xor(sum, 8, 64);
                    sum += __shfl_xor(sum, 16, 64);
                    sum += __shfl_xor(sum, 32, 64);
                    if (lane < 4) red[((kq * 4 + v) * (4 * CQ) + cq * 4 + lane) * T + t] = sum;
                }
    __syncthreads();
    // Partial of this (unit run, group): [chunk][g][k][c][t], the waves added in order.
    float* out = a.ws + ((size_t)chunk * a.G + g) * (KC * T);
    for (int e = tid; e < KC * T; e += 256)
        out[e] = ((lds[e] + lds[WLDS + e]) + lds[2 * WLDS + e]) + lds[3 * WLDS + e];
}

// Depthwise form of the streaming gradWeight (one input and MQ <= 2 output
// channels per group, 3x3, stride 1 or 2): the same per-wave rings and exact
// waits, with the 9 x MQ sums of a lane (lane = output column) on the vector
// ALUs, since 4x4 MFMA blocks would be a sixteenth used with one channel. A
// workgroup owns one group; its waves stream units (one band of one image)
// independently through rings of 72-float rows: input rows and the group's
// MQ dy rows. At stride 2 lanes past the output width read the last output's
// x (their dy is 0).
template <int S, int MQ, int PF>
__global__ void __launch_bounds__(256) sg_dw_wgrad_stream_kernel(SgWStreamArgs a)
{
    constexpr int T = 9;
    constexpr int D = S == 1 ? 2 : 1;
    constexpr int RX = S * (D + 1 + PF), RD = PF + 1;  // input-row and dy-row slots
    constexpr int CS = 72;
    constexpr int WLDS = RX * CS + RD * MQ * CS;
    constexpr int NDMA = S + MQ;                        // DMA rows per step
    extern __shared__ float lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    float* xring = lds + wave * WLDS;
    float* dring = xring + RX * CS;

    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int g = bid % a.G;
    const int chunk = bid / a.G;
    const int units = a.N * a.nbands;

    // Columns 64..71 of the input slots are never loaded (stride-1 lanes past
    // the output width read up to column 65, times dy = 0).
    for (int e = lane; e < RX * 8; e += 64) xring[(e >> 3) * CS + 64 + (e & 7)] = 0.f;

    const int wcol = lane - a.pw;
    const bool colok = (unsigned)wcol < (unsigned)a.W;
    const int xcol = S == 1 ? lane : min(lane, a.Wo - 1) * S;
    const uint32_t dplane = (uint32_t)a.Ho * a.Wo * 4u;
    float acc[MQ][T];
#pragma unroll
    for (int m = 0; m < MQ; ++m)
#pragma unroll
        for (int t = 0; t < T; ++t) acc[m][t] = 0.f;

    for (int k = 0; k < a.upw; ++k) {
        const int u = (chunk * a.upw + k) * 4 + wave;
        if (u >= units) break;
        const int n = u / a.nbands, band = u - n * a.nbands;
        const int r0 = band * a.R;
        const int rows = min(a.R, a.Ho - r0);
        const int nin = S * (rows - 1) + 3;
        const int hfirst = S * r0 - a.ph;
        const float* xg = a.x + ((size_t)n * a.C + g) * a.H * a.W;
        const float* dyg = a.dy + ((size_t)n * a.K + (size_t)g * a.Kg) * a.Ho * a.Wo;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(xg, (uint32_t)a.H * a.W * 4u);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(dyg, (uint32_t)a.Kg * a.Ho * a.Wo * 4u);
        auto issue_step = [&](int j, int sx, int sd, bool with_dy) {
#pragma unroll
            for (int r = 0; r < S; ++r) {
                const int jj = S * j + r, h = hfirst + jj;
                const bool okx = colok && jj < nin && (unsigned)h < (unsigned)a.H;
                load_lds64(rx, xring + (sx + r) * CS, okx ? (uint32_t)(h * a.W + wcol) * 4u : kOOB);
            }
            if (with_dy) {
                const int d = j - D;
                const uint32_t off = (lane < a.Wo && d < rows) ? (uint32_t)((r0 + d) * a.Wo + lane) * 4u : kOOB;
#pragma unroll
                for (int m = 0; m < MQ; ++m) load_lds64s(rd, dring + (sd * MQ + m) * CS, off, m * dplane);
            }
        };
#pragma unroll
        for (int j = 0; j < D; ++j) issue_step(j, S * j, 0, false);
#pragma unroll
        for (int j = D; j <= D + PF; ++j) issue_step(j, S * j, j - D, true);

        int sx0 = 0, sd0 = 0;
        for (int i = 0; i < rows; ++i) {
            wait_vmcnt<PF * NDMA>();
            float dv[MQ];
#pragma unroll
            for (int m = 0; m < MQ; ++m) dv[m] = dring[(sd0 * MQ + m) * CS + lane];
#pragma unroll
            for (int ti = 0; ti < 3; ++ti) {
                const int sv = sx0 + ti >= RX ? sx0 + ti - RX : sx0 + ti;
                const float* xr = xring + sv * CS + xcol;
#pragma unroll
                for (int tj = 0; tj < 3; ++tj) {
                    const float xv = xr[tj];
#pragma unroll
                    for (int m = 0; m < MQ; ++m) acc[m][ti * 3 + tj] = fmaf(dv[m], xv, acc[m][ti * 3 + tj]);
                }
            }
            lds_reads_done();  // (the slots' reads returned before the DMA reuses them)
            issue_step(i + D + PF + 1, sx0, sd0, true);
            sx0 = sx0 + S >= RX ? sx0 + S - RX : sx0 + S;
            sd0 = sd0 + 1 == RD ? 0 : sd0 + 1;
        }
    }

    // Sum the 64 lanes (a fixed butterfly) into this wave's own slice, then
    // the four waves in order.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int m = 0; m < MQ; ++m)
#pragma unroll
        for (int t = 0; t < T; ++t) {
            float v = acc[m][t];
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
            if (lane == 0) xring[m * T + t] = v;
        }
    __syncthreads();
    if (tid < MQ * T)
        a.ws[((size_t)chunk * a.G + g) * (MQ * T) + tid] =
            ((lds[tid] + lds[WLDS + tid]) + lds[2 * WLDS + tid]) + lds[3 * WLDS + tid];
}

// dw[g*Kg + k, c, t] = sum over the (image, band) partial sets. Block = 16
// outputs x 16 set groups: thread (e, sg) sums sets sg, sg+16, ... in order,
// then the 16 group sums are added in order.
// Depthwise gradWeight (one input channel per group, up to 2 outputs): the
// row tile of the kernel above for kDwwGroups consecutive groups at a time,
// accumulated on the vector ALUs (lane = output column, 9 taps x MQ sums per
// group and lane), so no arithmetic goes to absent channels. A workgroup owns
// a group block and a run of images, walks their bands, and writes one
// partial [o][tap] per group; sg_dw_wgrad_reduce adds the runs in order.
// S = 2 (stride 2): output (r, wo) pairs with LDS x rows 2r.., columns 2wo..;
// lanes past the output width read the last output's x (their dy is 0).
constexpr int kDwwGroups = 4;

struct SgDwWArgs {
    const float* x;
    const float* dy;
    float* ws;
    int N, C, H, W, K, Ho, Wo, G, Kg, ph, pw;
    int S;                  // stride (both axes)
    int R, run, nruns;      // band rows, images per workgroup, workgroups per group block
    int plane, dplane;      // x plane (((R-1)*S+3)*64 + 8) and dy plane (R*64 + 8), floats
};

template <int MQ, int S>
__global__ void __launch_bounds__(256) sg_dw_wgrad_kernel(SgDwWArgs a)
{
    constexpr int T = 9, GB = kDwwGroups;
    extern __shared__ float lds[];  // [GB][plane] x rows, [GB*MQ][dplane] dy rows; later sums
    float* ds = lds + GB * a.plane;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int ngb = (a.G + GB - 1) / GB;
    const int gb = bid % ngb, chunk = bid / ngb;
    const int g0 = gb * GB, ng = min(GB, a.G - g0);
    const int n_begin = chunk * a.run, n_end = min(a.N, n_begin + a.run);

    const int wcol = lane - a.pw;
    const bool colok = (unsigned)wcol < (unsigned)a.W;
    // Lanes past the image width read up to two floats beyond the last x row of
    // a plane (times dy = 0): keep the pad after each plane zero.
    if (S == 1 && tid < GB * 8) lds[(tid >> 3) * a.plane + (a.R + 2) * 64 + (tid & 7)] = 0.f;
    const int xcol = S == 1 ? lane : min(lane, a.Wo - 1) * S;

    float acc[GB][MQ][T];
#pragma unroll
    for (int gi = 0; gi < GB; ++gi)
#pragma unroll
        for (int o = 0; o < MQ; ++o)
#pragma unroll
            for (int t = 0; t < T; ++t) acc[gi][o][t] = 0.f;

    for (int n = n_begin; n < n_end; ++n) {
        const float* xg = a.x + ((size_t)n * a.C + g0) * a.H * a.W;
        const float* dyg = a.dy + ((size_t)n * a.K + (size_t)g0 * a.Kg) * a.Ho * a.Wo;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(xg, (uint32_t)ng * a.H * a.W * 4u);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(dyg, (uint32_t)ng * a.Kg * a.Ho * a.Wo * 4u);
        for (int ho0 = 0; ho0 < a.Ho; ho0 += a.R) {
            const int rows = min(a.R, a.Ho - ho0);
            const int hb = ho0 * S - a.ph;
            const int lrows = (rows - 1) * S + 3;
            __syncthreads();  // every wave is done with the previous band
#pragma unroll
            for (int gi = 0; gi < GB; ++gi)
                for (int r = wave; r < lrows; r += 4) {
                    const int h = hb + r;
                    const bool ok = colok && gi < ng && (unsigned)h < (unsigned)a.H;
                    load_lds64(rx, lds + gi * a.plane + r * 64,
                               ok ? (uint32_t)((gi * a.H + h) * a.W + wcol) * 4u : kOOB);
                }
#pragma unroll
            for (int j = 0; j < GB * MQ; ++j)
                for (int r = wave; r < rows; r += 4) {
                    const int gi = j / MQ, o = j % MQ;
                    const bool ok = lane < a.Wo && gi < ng && o < a.Kg;
                    load_lds64(rd, ds + j * a.dplane + r * 64,
                               ok ? (uint32_t)(((gi * a.Kg + o) * a.Ho + ho0 + r) * a.Wo + lane) * 4u : kOOB);
                }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            for (int r = wave; r < rows; r += 4) {
#pragma unroll
                for (int gi = 0; gi < GB; ++gi) {
                    const float* xr = lds + gi * a.plane + r * (S * 64) + xcol;
                    float xv[T];
#pragma unroll
                    for (int t = 0; t < T; ++t) xv[t] = xr[(t / 3) * 64 + t % 3];
#pragma unroll
                    for (int o = 0; o < MQ; ++o) {
                        const float dv = ds[(gi * MQ + o) * a.dplane + r * 64 + lane];
#pragma unroll
                        for (int t = 0; t < T; ++t) acc[gi][o][t] = fmaf(dv, xv[t], acc[gi][o][t]);
                    }
                }
            }
        }
    }

    // Sum the 64 lanes (a fixed butterfly), then the four waves in order.
    __syncthreads();  // LDS reuse
    float* red = lds;  // [wave][GB*MQ*T]
#pragma unroll
    for (int gi = 0; gi < GB; ++gi)
#pragma unroll
        for (int o = 0; o < MQ; ++o)
#pragma unroll
            for (int t = 0; t < T; ++t) {
                float v = acc[gi][o][t];
                for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
                if (lane == 0) red[wave * (GB * MQ * T) + (gi * MQ + o) * T + t] = v;
            }
    __syncthreads();
    // Partial of this (image run, group block): ws[chunk][g][o][t].
    for (int e = tid; e < GB * MQ * T; e += 256) {
        const int gi = e / (MQ * T);
        if (gi >= ng) continue;
        constexpr int NS = GB * MQ * T;
        const float v = ((red[e] + red[NS + e]) + red[2 * NS + e]) + red[3 * NS + e];
        a.ws[((size_t)chunk * a.G + g0) * (MQ * T) + e] = v;
    }
}

// Depthwise gradWeight (3x3, multiplier 1, unit dilation, stride S = 1 or 2)
// walking down the rows: a wave owns 64 / lpw planes side by side and a band
// of RB output rows. Lane L of a plane loads input column L - pw of each input
// row (tap columns 1 and 2 are lanes L + 1 and L + 2, moved down by DPP) and
// dy column L / S of the output rows (lanes that hold no output read 0). Input
// row t pairs tap row i with output row (t - i) / S where that divides; each
// lane keeps the 9 tap sums of its column, and at the band's end the lanes of
// a plane are added by a fixed butterfly into the band's partial [n, band][c][9]
// (sg_dw_wgrad_reduce adds the partials in order).
struct SgDwWalkWArgs {
    const float* x;      // planes of H x W
    const float* dy;     // planes of Ho x Wo
    float* ws;           // [N * nbands][C][9]
    int C, H, W, Ho, Wo, ph, pw;
    int planes, lpw_log2, nbands, waves;
    int rb;              // dy rows per band (the kernel's RB)
};

template <int S, int PF, int RB>
__global__ void __launch_bounds__(256) sg_dw_wgrad_walk_kernel(SgDwWalkWArgs a)
{
    constexpr int NS = S * (RB - 1) + 3;        // input rows a band reads
    constexpr int NB = PF + 1;                  // input-row buffers
    constexpr int PFD = (PF + S - 1) / S;       // dy rows loaded ahead
    constexpr int NBD = PFD + 3;                // dy rows held: in flight, and the three being paired
    constexpr uint32_t kColOOB = 0x40000000u, kRowOOB = 0x80000000u;
    const int lane = threadIdx.x & 63;
    const int gw = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (gw >= a.waves) return;
    const int band = gw % a.nbands;
    const int pg = gw / a.nbands;
    const int ppw = 64 >> a.lpw_log2;
    const int p0 = pg * ppw;
    const int np = min(ppw, a.planes - p0);
    const int slot = lane >> a.lpw_log2;
    const int L = lane - (slot << a.lpw_log2);
    const int wo = S == 1 ? L : L >> 1;
    const bool has_dy = slot < np && (S == 1 || (L & 1) == 0) && wo < a.Wo;

    const uint32_t HWi = (uint32_t)a.H * a.W, HWo = (uint32_t)a.Ho * a.Wo;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x + (size_t)p0 * HWi, (uint32_t)np * HWi * 4u);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dy + (size_t)p0 * HWo, (uint32_t)np * HWo * 4u);
    const int r0 = band * RB;
    const int rows = min(RB, a.Ho - r0);
    const int nin = S * (rows - 1) + 3;
    const int hb = S * r0 - a.ph;
    const int cc = L - a.pw;
    const uint32_t xcol = slot < np && (unsigned)cc < (unsigned)a.W ? (uint32_t)(slot * HWi + cc) * 4u : kColOOB;
    const uint32_t dcol = has_dy ? (uint32_t)(slot * HWo + r0 * a.Wo + wo) * 4u : kColOOB;

    auto loadx = [&](int t) {
        const int h = hb + t;
        const uint32_t hs = t < nin && (unsigned)h < (unsigned)a.H ? (uint32_t)h * a.W * 4u : kRowOOB;
        return load_f32(rx, xcol + hs);
    };
    auto loadd = [&](int q) { return load_f32(rd, dcol + (q < rows ? (uint32_t)q * a.Wo * 4u : kRowOOB)); };
    auto down1 = [](float v) {  // lane L takes lane L + 1's value
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x130, 0xF, 0xF, false));
    };

    float acc[9];
#pragma unroll
    for (int e = 0; e < 9; ++e) acc[e] = 0.f;
    float xw[NB], dw[NBD];
#pragma unroll
    for (int k = 0; k < PF; ++k) xw[k] = loadx(k);
#pragma unroll
    for (int q = 0; q < PFD && q < RB; ++q) dw[q] = loadd(q);
    unroll_seq(
        [&](auto sc) {
            constexpr int t = decltype(sc)::value;
            // Steps stay in order: hoisting later rows' loads (the code
            // generator would issue most of them first) holds them all in
            // registers and cuts the waves a SIMD keeps ...
            asm volatile("" ::: "memory");
            if constexpr (t + PF < NS) xw[(t + PF) % NB] = loadx(t + PF);
            // dy row q + PFD is loaded at the first step that pairs with row q.
            if constexpr (t % S == 0 && t / S + PFD < RB) dw[(t / S + PFD) % NBD] = loadd(t / S + PFD);
            float v[3];
            v[0] = xw[t % NB];
            v[1] = down1(v[0]);
            v[2] = down1(v[1]);
            unroll_seq(
                [&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    if constexpr ((t - i) % S == 0 && t >= i && (t - i) / S < RB) {
                        const float d = dw[((t - i) / S) % NBD];
#pragma unroll
                        for (int j = 0; j < 3; ++j) acc[i * 3 + j] = fmaf(d, v[j], acc[i * 3 + j]);
                    }
                },
                std::make_integer_sequence<int, 3>{});
            // ... and this step's sums are formed before the next step's
            // loads (else the FMAs sink below them).
            asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
                         "+v"(acc[6]), "+v"(acc[7]), "+v"(acc[8]));
        },
        std::make_integer_sequence<int, NS>{});

    // The lanes of each plane, by a fixed butterfly (xor offsets below lpw stay
    // within the plane), then lane 0 of the plane writes the band's partial.
    const int lpw = 1 << a.lpw_log2;
#pragma unroll
    for (int e = 0; e < 9; ++e)
        for (int off = lpw >> 1; off > 0; off >>= 1) acc[e] += __shfl_xor(acc[e], off, 64);
    if (L == 0 && slot < np) {
        const int p = p0 + slot, n = p / a.C, c = p - n * a.C;
        float* out = a.ws + (((size_t)n * a.nbands + band) * a.C + c) * 9;
#pragma unroll
        for (int e = 0; e < 9; ++e) out[e] = acc[e];
    }
}

// dw[g*Kg + o][0][t] = sum over image runs of ws[run][g][o][t] in a fixed
// order. Block = 16 outputs x 16 run groups: thread (e, rg) sums runs rg,
// rg + 16, ... in order, then the 16 group sums are added in order (a serial
// loop over all runs per output left each thread waiting on one load at a time).
__global__ void __launch_bounds__(256) sg_dw_wgrad_reduce(const float* __restrict__ ws, float* __restrict__ dw,
                                                          int nruns, int G, int Kg, int MQ)
{
    __shared__ float part[16][17];
    const int el = threadIdx.x & 15, rg = threadIdx.x >> 4;
    const int e = blockIdx.x * 16 + el;  // over G * Kg * 9
    const int E = G * Kg * 9;
    float sum = 0.f;
    if (e < E) {
        const int t = e % 9, go = e / 9, g = go / Kg, o = go - g * Kg;
        const size_t per = (size_t)G * MQ * 9;
        const size_t idx = ((size_t)g * MQ + o) * 9 + t;
        for (int r = rg; r < nruns; r += 16) sum += ws[(size_t)r * per + idx];
    }
    part[rg][el] = sum;
    __syncthreads();
    if (rg != 0 || e >= E) return;
    sum = part[0][el];
#pragma unroll
    for (int i = 1; i < 16; ++i) sum += part[i][el];
    dw[e] = sum;
}

__global__ void __launch_bounds__(256) sg_wgrad_reduce(const float* __restrict__ ws,
                                                       float* __restrict__ dw, int nsets, int G,
                                                       int Kg, int Cg, int T, int K4, int C4)
{
    __shared__ float part[16][17];
    const int el = threadIdx.x & 15, sg = threadIdx.x >> 4;
    const int e = blockIdx.x * 16 + el;  // over G * K4 * C4 * T (partials of K4 x C4 channel pairs)
    const int per_set = G * K4 * C4 * T;
    float sum = 0.f;
    if (e < per_set)
        for (int s = sg; s < nsets; s += 16) sum += ws[(size_t)s * per_set + e];
    part[sg][el] = sum;
    __syncthreads();
    if (sg != 0 || e >= per_set) return;
    sum = part[0][el];
#pragma unroll
    for (int i = 1; i < 16; ++i) sum += part[i][el];
    const int t = e % T, kc = (e / T) % (K4 * C4), g = e / (K4 * C4 * T);
    const int k = kc / C4, c = kc - k * C4;
    if (k >= Kg || c >= Cg) return;
    dw[(((size_t)g * Kg + k) * Cg + c) * T + t] = sum;
}

// ---- host side --------------------------------------------------------------

struct SgProblem {
    const float *in, *wgt, *bias;
    float* out;
    int N, G, Cin_tot, Cin_g, Hin, Win, Cout_tot, Cout_g, Hout, Wout;
    int kh, kw, sh, sw, dh, dw, ph, pw;
    int w_so, w_sr, w_gstride;
    bool flip;
    int uh = 1, uw = 1, Hr = 0, Wr = 0;  // input upsampling (general kernel only), stored plane size
    int relu = 0;                        // forward epilogue
};

// LDS tile budget per workgroup (28 KiB): five workgroups share a CU, so the
// loads of some overlap the arithmetic of others.
constexpr int kSgTileFloats = 7168;

int sg_cinq(int cin) { return cin <= 1 ? 1 : cin <= 2 ? 2 : 4; }
int ceil64(int v) { return (v + 63) / 64 * 64; }

// Rows per workgroup: the most whose input tile fits the budget.
int sg_rows(const SgProblem& p, int cinq, int* LW, int* LR)
{
    *LW = (p.Wout - 1) * p.sw + (p.kw - 1) * p.dw + 1;
    int R = p.Hout;
    for (; R >= 1; --R) {
        *LR = (R - 1) * p.sh + (p.kh - 1) * p.dh + 1;
        if ((int64_t)cinq * *LR * *LW <= kSgTileFloats) break;
    }
    return R;
}

bool sg_problem_ok(const SgProblem& p)
{
    // 3x3, or 5x5 with at most two input channels per group (depthwise with a
    // channel multiplier up to 8): the filters of a group sit in registers.
    if (!((p.kh == 3 && p.kw == 3) || (p.kh == 5 && p.kw == 5 && p.Cin_g <= 2))) return false;
    if (p.Cin_g > 4 || p.Cout_g > 8 || p.N < 1) return false;
    int LW, LR;
    if (sg_rows(p, sg_cinq(p.Cin_g), &LW, &LR) < 1) return false;
    if ((int64_t)(p.Cin_g + 4) * p.Hr * p.Wr * 4 >= (int64_t(1) << 30)) return false;
    if ((int64_t)p.Hin * p.Win >= (1 << 30) || (int64_t)p.Hout * p.Wout >= (1 << 30)) return false;
    return true;
}

template <int KS, int CIN, int OQ, bool FLIP>
void sg_launch(const SgArgs& a, int blocks, size_t lds, hipStream_t st)
{
    hipLaunchKernelGGL((sg_conv_kernel<KS, KS, CIN, OQ, FLIP>), dim3(blocks), dim3(256), lds, st, a);
}

// The row-per-DMA fast path: 3x3 at unit stride and dilation, padded rows of
// at most 64 floats. Bands of about 16 rows keep the tile near 17 KiB, so
// eight workgroups share a CU.
bool sg_row64_ok(const SgProblem& p)
{
    return p.kh == 3 && p.kw == 3 && p.sh == 1 && p.sw == 1 && p.dh == 1 && p.dw == 1 &&
           p.uh == 1 && p.uw == 1 &&
           p.Wout + 2 <= 64 && p.ph >= 0 && p.pw >= 0 && p.pw <= 2;
}

template <int CIN, int OQ, bool FLIP>
void sg_row64_launch(const SgArgs& a, int blocks, size_t lds, hipStream_t st)
{
    hipLaunchKernelGGL((sg_conv_row64_kernel<CIN, OQ, FLIP>), dim3(blocks), dim3(256), lds, st, a);
}

bool sg_run_row64(const SgProblem& p, hipStream_t st)
{
    const int CINq = sg_cinq(p.Cin_g);
    const int OQ = p.Cout_g <= 4 ? 1 : 2;
    SgArgs a;
    a.in = p.in; a.wgt = p.wgt; a.bias = p.bias; a.out = p.out;
    a.relu = p.relu;
    a.N = p.N; a.G = p.G;
    a.Cin_tot = p.Cin_tot; a.Cin_g = p.Cin_g; a.Hin = p.Hin; a.Win = p.Win;
    a.Cout_tot = p.Cout_tot; a.Cout_g = p.Cout_g; a.Hout = p.Hout; a.Wout = p.Wout;
    a.sh = 1; a.sw = 1; a.dh = 1; a.dw = 1; a.ph = p.ph; a.pw = p.pw;
    a.w_so = p.w_so; a.w_sr = p.w_sr; a.w_gstride = p.w_gstride;
    a.uh = 1; a.uw = 1; a.Hr = p.Hin; a.Wr = p.Win;
    const int nb = (p.Hout + 15) / 16;
    a.R = (p.Hout + nb - 1) / nb;
    a.nbands = (p.Hout + a.R - 1) / a.R;
    a.LR = a.R + 2;
    a.LW = 64;
    a.plane = a.LR * 64;
    a.div_plane = make_fastdiv((uint32_t)a.plane);
    a.div_LW = make_fastdiv(64u);
    a.div_Wout = make_fastdiv((uint32_t)p.Wout);
    const int64_t blocks = (int64_t)p.N * p.G * a.nbands;
    if (blocks >= (1 << 30)) return false;
    const size_t lds = ((size_t)CINq * a.plane + (size_t)CINq * 9 * 4 * OQ) * 4;
#define SG_CASE(cin, oq)                                                          \
    if (CINq == cin && OQ == oq) {                                                \
        if (p.flip) sg_row64_launch<cin, oq, true>(a, (int)blocks, lds, st);      \
        else sg_row64_launch<cin, oq, false>(a, (int)blocks, lds, st);            \
        return true;                                                              \
    }
    SG_CASE(1, 1) SG_CASE(2, 1) SG_CASE(4, 1) SG_CASE(1, 2) SG_CASE(2, 2) SG_CASE(4, 2)
#undef SG_CASE
    return false;
}

// The walking depthwise kernel: 3x3, multiplier 1, unit dilation and stride
// (forward, or gradInput as the forward of dy), rows of at most 62 outputs
// (a lane per output and two lanes past the last).
bool sg_dw_walk_ok(const SgProblem& p)
{
#ifdef GCONV_SG_NO_DW_WALK
    (void)p;
    return false;
#else
    if (!(p.kh == 3 && p.kw == 3 && p.dh == 1 && p.dw == 1 && p.Cin_g == 1 && p.Cout_g == 1)) return false;
    if (!(p.uh == 1 && p.uw == 1 && p.sh == 1 && p.sw == 1)) return false;
    if (p.Wout + 2 > 64 || p.N < 1 || (int64_t)p.N * p.G >= (1 << 30)) return false;
    // A wave's (up to four) planes stay below 2^30 bytes (the buffer offsets of the kernel).
    return (int64_t)p.Hin * p.Win * 16 < (int64_t(1) << 30) && (int64_t)p.Hout * p.Wout * 16 < (int64_t(1) << 30);
#endif
}

#ifndef GCONV_DW_WALK_PF
#define GCONV_DW_WALK_PF 8
#endif
#ifndef GCONV_DW_WALK_RB
#define GCONV_DW_WALK_RB 14
#endif
// Output rows per band (a band is one straight run of code).
constexpr int kDwWalkRows = GCONV_DW_WALK_RB;

bool sg_run_dw_walk(const SgProblem& p, hipStream_t st)
{
    SgDwWalkArgs a{};
    a.in = p.in; a.wgt = p.wgt; a.bias = p.bias; a.out = p.out;
    a.C = p.G; a.Hin = p.Hin; a.Win = p.Win; a.Hout = p.Hout; a.Wout = p.Wout;
    a.ph = p.ph; a.pw = p.pw; a.relu = p.relu;
    a.planes = p.N * p.G;
    a.lpw_log2 = p.Wout + 2 <= 16 ? 4 : p.Wout + 2 <= 32 ? 5 : 6;
    const int64_t groups = ((int64_t)a.planes + (64 >> a.lpw_log2) - 1) >> (6 - a.lpw_log2);
    a.nbands = (p.Hout + kDwWalkRows - 1) / kDwWalkRows;
    const int64_t waves = groups * a.nbands;
    if (waves >= (int64_t(1) << 30)) return false;
    a.waves = (int)waves;
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    if (p.flip) hipLaunchKernelGGL((sg_dw_walk_kernel<true, GCONV_DW_WALK_PF, kDwWalkRows>), dim3(blocks), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((sg_dw_walk_kernel<false, GCONV_DW_WALK_PF, kDwWalkRows>), dim3(blocks), dim3(256), 0, st, a);
    return true;
}

#ifndef GCONV_DW_WALK2_RB
#define GCONV_DW_WALK2_RB 7
#endif
#ifndef GCONV_DW_WALK2_PF
#define GCONV_DW_WALK2_PF 8
#endif
constexpr int kDwWalk2Rows = GCONV_DW_WALK2_RB;  // output rows per band, stride 2

// The stride-2 forward walk: 3x3, multiplier 1, unit dilation, 2 Wout + 1
// lanes a plane within the wave.
bool sg_dw_walk_s2_ok(const SgProblem& p)
{
#ifdef GCONV_SG_NO_DW_WALK2
    (void)p;
    return false;
#else
    if (!(p.kh == 3 && p.kw == 3 && p.dh == 1 && p.dw == 1 && p.Cin_g == 1 && p.Cout_g == 1)) return false;
    if (!(p.uh == 1 && p.uw == 1 && p.sh == 2 && p.sw == 2 && !p.flip)) return false;
    if (2 * p.Wout + 1 > 64 || p.N < 1 || (int64_t)p.N * p.G >= (1 << 30)) return false;
    return (int64_t)p.Hin * p.Win * 16 < (int64_t(1) << 30) && (int64_t)p.Hout * p.Wout * 16 < (int64_t(1) << 30);
#endif
}

bool sg_run_dw_walk_s2(const SgProblem& p, hipStream_t st)
{
    SgDwWalkArgs a{};
    a.in = p.in; a.wgt = p.wgt; a.bias = p.bias; a.out = p.out;
    a.C = p.G; a.Hin = p.Hin; a.Win = p.Win; a.Hout = p.Hout; a.Wout = p.Wout;
    a.ph = p.ph; a.pw = p.pw; a.relu = p.relu;
    a.planes = p.N * p.G;
    a.lpw_log2 = 2 * p.Wout + 1 <= 16 ? 4 : 2 * p.Wout + 1 <= 32 ? 5 : 6;
    const int64_t groups = ((int64_t)a.planes + (64 >> a.lpw_log2) - 1) >> (6 - a.lpw_log2);
    a.nbands = (p.Hout + kDwWalk2Rows - 1) / kDwWalk2Rows;
    const int64_t waves = groups * a.nbands;
    if (waves >= (int64_t(1) << 30)) return false;
    a.waves = (int)waves;
    hipLaunchKernelGGL((sg_dw_walk_s2_kernel<GCONV_DW_WALK2_PF, kDwWalk2Rows>), dim3((unsigned)((waves + 3) / 4)),
                       dim3(256), 0, st, a);
    return true;
}

template <int MQ, bool FLIP, int S>
void sg_dw_launch(const SgArgs& a, int blocks, size_t lds, hipStream_t st)
{
    hipLaunchKernelGGL((sg_dw_row64_kernel<MQ, FLIP, S>), dim3(blocks), dim3(256), lds, st, a);
}

// The depthwise row tile: 3x3, dilation 1, one input channel per group;
// stride 1 (also over a virtually upsampled input: strided gradInput) or a
// forward stride of 2; every column the outputs read lies in the 64-float
// LDS row that starts pw columns left of the input.
bool sg_dw_ok(const SgProblem& p)
{
    if (!(p.kh == 3 && p.kw == 3 && p.dh == 1 && p.dw == 1 && p.Cin_g == 1)) return false;
    if (!(p.sh == p.sw && (p.sh == 1 || (p.sh == 2 && p.uh == 1 && p.uw == 1)))) return false;
    if (p.uh < 1 || p.uw < 1) return false;
    return (p.Wout - 1) * p.sw + 2 <= 63 && p.ph >= 0 && p.pw >= 0 && p.pw <= 2;
}

// One input channel per group (depthwise forward; depthwise gradInput with a
// multiplier of 1) on the row-per-DMA tile, kDwGroups groups per workgroup.
bool sg_run_dw(const SgProblem& p, hipStream_t st)
{
    const int MQ = p.Cout_g <= 1 ? 1 : p.Cout_g <= 2 ? 2 : p.Cout_g <= 4 ? 4 : 8;
    const int S = p.sh;
    SgArgs a;
    a.in = p.in; a.wgt = p.wgt; a.bias = p.bias; a.out = p.out;
    a.relu = p.relu;
    a.N = p.N; a.G = p.G;
    a.Cin_tot = p.Cin_tot; a.Cin_g = p.Cin_g; a.Hin = p.Hin; a.Win = p.Win;
    a.Cout_tot = p.Cout_tot; a.Cout_g = p.Cout_g; a.Hout = p.Hout; a.Wout = p.Wout;
    a.sh = S; a.sw = S; a.dh = 1; a.dw = 1; a.ph = p.ph; a.pw = p.pw;
    a.w_so = p.w_so; a.w_sr = p.w_sr; a.w_gstride = p.w_gstride;
    a.uh = p.uh; a.uw = p.uw; a.Hr = p.Hr; a.Wr = p.Wr;
    // Bands of about 16 input rows.
#ifndef GCONV_DW_S2_RMAX
#define GCONV_DW_S2_RMAX 14
#endif
    const int rmax = S == 1 ? 16 : GCONV_DW_S2_RMAX;
    const int nb = (p.Hout + rmax - 1) / rmax;
    a.R = (p.Hout + nb - 1) / nb;
    a.nbands = (p.Hout + a.R - 1) / a.R;
    a.LR = (a.R - 1) * S + 3;
    a.LW = 64;
    a.plane = a.LR * 64;
    a.div_plane = make_fastdiv((uint32_t)a.plane);
    a.div_LW = make_fastdiv(64u);
    a.div_Wout = make_fastdiv((uint32_t)p.Wout);
    const int64_t blocks = (int64_t)p.N * ((p.G + kDwGroups - 1) / kDwGroups) * a.nbands;
    if (blocks >= (1 << 30)) return false;
    if ((int64_t)kDwGroups * p.w_gstride * 4 >= (int64_t(1) << 30)) return false;
    const size_t lds = ((size_t)kDwGroups * a.plane + (size_t)kDwGroups * MQ * 9) * 4;
#define SG_CASE(mq)                                                             \
    if (MQ == mq) {                                                             \
        if (S == 2) sg_dw_launch<mq, false, 2>(a, (int)blocks, lds, st);        \
        else if (p.flip) sg_dw_launch<mq, true, 1>(a, (int)blocks, lds, st);    \
        else sg_dw_launch<mq, false, 1>(a, (int)blocks, lds, st);               \
        return true;                                                            \
    }
    SG_CASE(1) SG_CASE(2) SG_CASE(4) SG_CASE(8)
#undef SG_CASE
    return false;
}

bool sg_run(const SgProblem& p, hipStream_t st)
{
    if (!sg_problem_ok(p)) return false;
    if (sg_dw_walk_ok(p)) return sg_run_dw_walk(p, st);
    if (sg_dw_walk_s2_ok(p)) return sg_run_dw_walk_s2(p, st);
#ifndef GCONV_SG_NO_DW
#ifdef GCONV_SG_NO_DW_S2
    if (sg_dw_ok(p) && p.sh == 1) return sg_run_dw(p, st);
#else
    if (sg_dw_ok(p) && !(p.flip && p.sh != 1)) return sg_run_dw(p, st);
#endif
#endif
#ifndef GCONV_SG_NO_ROW64
    if (sg_row64_ok(p)) return sg_run_row64(p, st);
#endif
    const int CINq = sg_cinq(p.Cin_g);
    const int OQ = p.Cout_g <= 4 ? 1 : 2;
    SgArgs a;
    a.in = p.in; a.wgt = p.wgt; a.bias = p.bias; a.out = p.out;
    a.relu = p.relu;
    a.N = p.N; a.G = p.G;
    a.Cin_tot = p.Cin_tot; a.Cin_g = p.Cin_g; a.Hin = p.Hin; a.Win = p.Win;
    a.Cout_tot = p.Cout_tot; a.Cout_g = p.Cout_g; a.Hout = p.Hout; a.Wout = p.Wout;
    a.sh = p.sh; a.sw = p.sw; a.dh = p.dh; a.dw = p.dw; a.ph = p.ph; a.pw = p.pw;
    a.w_so = p.w_so; a.w_sr = p.w_sr; a.w_gstride = p.w_gstride;
    a.uh = p.uh; a.uw = p.uw; a.Hr = p.Hr; a.Wr = p.Wr;
    a.R = sg_rows(p, CINq, &a.LW, &a.LR);
    a.nbands = (p.Hout + a.R - 1) / a.R;
    a.plane = a.LR * a.LW;
    a.div_plane = make_fastdiv((uint32_t)a.plane);
    a.div_LW = make_fastdiv((uint32_t)a.LW);
    a.div_Wout = make_fastdiv((uint32_t)p.Wout);
    const int64_t blocks = (int64_t)p.N * p.G * a.nbands;
    if (blocks >= (1 << 30)) return false;
    const size_t lds = ((size_t)ceil64(CINq * a.plane) + (size_t)CINq * p.kh * p.kw * 4 * OQ) * 4;
#define SG_CASE(ks, cin, oq)                                                       \
    if (p.kh == ks && CINq == cin && OQ == oq) {                                   \
        if (p.flip) sg_launch<ks, cin, oq, true>(a, (int)blocks, lds, st);         \
        else sg_launch<ks, cin, oq, false>(a, (int)blocks, lds, st);               \
        return true;                                                               \
    }
    SG_CASE(3, 1, 1) SG_CASE(3, 2, 1) SG_CASE(3, 4, 1) SG_CASE(3, 1, 2) SG_CASE(3, 2, 2) SG_CASE(3, 4, 2)
    SG_CASE(5, 1, 1) SG_CASE(5, 2, 1) SG_CASE(5, 1, 2) SG_CASE(5, 2, 2)
#undef SG_CASE
    return false;
}

SgProblem sg_fwd_problem(const Shape& s, const float* x, const float* w, const float* bias, float* y)
{
    SgProblem p;
    p.in = x; p.wgt = w; p.bias = bias; p.out = y;
    p.N = s.N; p.G = s.G; p.Cin_tot = s.C; p.Cin_g = s.Cg; p.Hin = s.H; p.Win = s.W;
    p.Cout_tot = s.K; p.Cout_g = s.Kg; p.Hout = s.Ho; p.Wout = s.Wo;
    p.kh = s.kh; p.kw = s.kw; p.sh = s.sh; p.sw = s.sw; p.dh = s.dh; p.dw = s.dw;
    p.ph = s.ph; p.pw = s.pw;
    const int T = s.kh * s.kw;
    p.w_so = s.Cg * T; p.w_sr = T; p.w_gstride = s.Kg * s.Cg * T;
    p.flip = false;
    p.Hr = s.H; p.Wr = s.W;
    p.relu = s.relu;
    return p;
}

SgProblem sg_bwd_data_problem(const Shape& s, const float* dy, const float* w, float* dx)
{
    SgProblem p;
    p.in = dy; p.wgt = w; p.bias = nullptr; p.out = dx;
    p.N = s.N; p.G = s.G; p.Cin_tot = s.K; p.Cin_g = s.Kg;
    // At stride s, dy is read as if upsampled by s (zeros between its values):
    // the adjoint of a strided correlation is the unit-stride correlation of
    // the upsampled dy with the tap-reversed filter.
    p.Hin = (s.Ho - 1) * s.sh + 1; p.Win = (s.Wo - 1) * s.sw + 1;
    p.uh = s.sh; p.uw = s.sw; p.Hr = s.Ho; p.Wr = s.Wo;
    p.Cout_tot = s.C; p.Cout_g = s.Cg; p.Hout = s.H; p.Wout = s.W;
    p.kh = s.kh; p.kw = s.kw; p.sh = 1; p.sw = 1; p.dh = s.dh; p.dw = s.dw;
    p.ph = (s.kh - 1) * s.dh - s.ph;
    p.pw = (s.kw - 1) * s.dw - s.pw;
    const int T = s.kh * s.kw;
    p.w_so = T; p.w_sr = s.Cg * T; p.w_gstride = s.Kg * s.Cg * T;
    p.flip = true;
    return p;
}

// Plane stride == 8 (mod 32): the 4 channels x 8 pixels of a half-wave read
// fall in distinct banks.
int pad8(int v) { return (v + 23) / 32 * 32 + 8; }

// The row-per-DMA gradWeight kernel: unit stride and dilation, padded rows of
// at most 64 floats; bands of about 16 rows.
bool sgw_row64_ok(const Shape& s)
{
    return s.kh == 3 && s.kw == 3 && s.sh == 1 && s.sw == 1 && s.dh == 1 && s.dw == 1 && s.Wo + 2 <= 64;
}

bool sgw_plan(const Shape& s, SgWArgs* out, bool* row64 = nullptr)
{
    // 3x3 only: a 5x5 workgroup would hold 25 accumulators per lane and run
    // at one wave per SIMD, slower than the direct kernel.
    if (!(s.kh == 3 && s.kw == 3)) return false;
    if (s.Cg > 4 || s.Kg > 4 || s.N < 1) return false;
    SgWArgs a{};
    a.N = s.N; a.C = s.C; a.H = s.H; a.W = s.W; a.K = s.K; a.Ho = s.Ho; a.Wo = s.Wo;
    a.G = s.G; a.Cg = s.Cg; a.Kg = s.Kg;
    a.sh = s.sh; a.sw = s.sw; a.dh = s.dh; a.dw = s.dw; a.ph = s.ph; a.pw = s.pw;
    if ((int64_t)(s.Cg + 4) * s.H * s.W * 4 >= (int64_t(1) << 30)) return false;
    if ((int64_t)(s.Kg + 4) * s.Ho * s.Wo * 4 >= (int64_t(1) << 30)) return false;
#ifndef GCONV_SG_NO_ROW64
    if (sgw_row64_ok(s)) {
        // Bands of about 16 rows; runs of images such that about 1024
        // workgroups (four per CU) cover all groups.
        const int nb = (s.Ho + 15) / 16;
        a.R = (s.Ho + nb - 1) / nb;
        const int runs = std::max(1, std::min(s.N, 1024 / std::max(1, s.G)));
        a.run = (s.N + runs - 1) / runs;
        a.nruns = (s.N + a.run - 1) / a.run;
        a.nbands = (s.Ho + a.R - 1) / a.R;
        a.LW = 64;
        a.LR = a.R + 2;
        a.plane = a.LR * 64 + 8;  // == 8 (mod 32)
        a.dplane = a.R * 64 + 8;
        if ((int64_t)a.nruns * s.G >= (1 << 30)) return false;
        if (out) *out = a;
        if (row64) *row64 = true;
        return true;
    }
#endif
    if (row64) *row64 = false;
    a.LW = (s.Wo - 1) * s.sw + (s.kw - 1) * s.dw + 1;
    // Rows per band: the most whose input and dy bands fit the LDS budget.
    int R = s.Ho;
    for (; R >= 1; --R) {
        a.LR = (R - 1) * s.sh + (s.kh - 1) * s.dh + 1;
        a.plane = pad8(a.LR * a.LW);
        a.dplane = ceil64(R * s.Wo) + 8;
        if (ceil64(4 * a.plane) + 4 * a.dplane <= kSgTileFloats) break;
    }
    if (R < 1) return false;
    a.R = R;
    a.nbands = (s.Ho + R - 1) / R;
    if ((int64_t)(s.Cg + 4) * s.H * s.W * 4 >= (int64_t(1) << 30)) return false;
    if ((int64_t)(s.Kg + 4) * s.Ho * s.Wo * 4 >= (int64_t(1) << 30)) return false;
    if ((int64_t)s.N * a.nbands * s.G >= (1 << 30)) return false;
    a.div_plane = make_fastdiv((uint32_t)a.plane);
    a.div_LW = make_fastdiv((uint32_t)a.LW);
    a.div_Wo = make_fastdiv((uint32_t)a.Wo);
    if (out) *out = a;
    return true;
}

// The streaming gradWeight kernel: 3x3, unit dilation, stride 1 or 2, up to 8
// input and 8 output channels per group, every input column the outputs read
// inside a 64-float row (rows of at most 62 outputs at stride 1, 31 at
// stride 2). Bands per image such that the waves of one round of resident
// workgroups have a unit each (ResNeXt 32x4d, 64 images of 56 x 56: 1024
// workgroups of 28 KiB, four per CU), bands of at least 8 rows; a wave takes
// several units where there are more than two rounds' worth. One step of
// prefetch: on ResNeXt 32x4d deeper rings cost resident workgroups and time
// (49.9 us at one step, 51.4 at two, 56.1 at three; the banded kernel 60.1).
#ifndef GCONV_SG_WSTREAM_PF
#define GCONV_SG_WSTREAM_PF 1
#endif
constexpr int kSgwStreamPF = GCONV_SG_WSTREAM_PF;

struct SgwStreamShape {
    int S, CQ, KQ, nstep;
    size_t lds;   // bytes per workgroup
};

bool sgw_stream_plan(const Shape& s, SgWStreamArgs* out, SgwStreamShape* shp = nullptr)
{
#ifdef GCONV_SG_NO_STREAM
    (void)s; (void)out; (void)shp;
    return false;
#else
    if (!(s.kh == 3 && s.kw == 3 && s.dh == 1 && s.dw == 1 && s.sh == s.sw && (s.sh == 1 || s.sh == 2))) return false;
    if (!(s.Cg <= 8 && s.Kg <= 8 && s.N >= 1 && s.ph >= 0 && s.pw >= 0)) return false;
    const int S = s.sh;
    if (S == 1 ? s.Wo + 2 > 64 : 2 * s.Wo > 63) return false;
    if ((int64_t)(s.Cg + 8) * s.H * s.W * 4 >= (int64_t(1) << 30)) return false;
    if ((int64_t)(s.Kg + 8) * s.Ho * s.Wo * 4 >= (int64_t(1) << 30)) return false;
    SgwStreamShape sh;
    sh.S = S;
    sh.CQ = s.Cg <= 4 ? 1 : 2;
    sh.KQ = s.Kg <= 4 ? 1 : 2;
    sh.nstep = (s.Wo + 15) / 16;
    constexpr int PF = kSgwStreamPF, CS = 72;
    const int D = S == 1 ? 2 : 1;
    const int RX = S * (D + 1 + PF), RD = PF + 1;
    sh.lds = (size_t)4 * (RX * 4 * sh.CQ + RD * 4 * sh.KQ) * CS * 4;
    const int per_cu = (int)std::min<size_t>(8, (160 * 1024) / sh.lds);
    const int64_t waves = (int64_t)256 * per_cu * 4;
    SgWStreamArgs a{};
    a.N = s.N; a.C = s.C; a.H = s.H; a.W = s.W; a.K = s.K; a.Ho = s.Ho; a.Wo = s.Wo;
    a.G = s.G; a.Cg = s.Cg; a.Kg = s.Kg; a.ph = s.ph; a.pw = s.pw;
    const int64_t planes = (int64_t)s.N * s.G;
    const int nb = (int)std::max<int64_t>(1, std::min<int64_t>(waves / planes, std::max(1, s.Ho / 8)));
    a.R = (s.Ho + nb - 1) / nb;
    a.nbands = (s.Ho + a.R - 1) / a.R;
    const int64_t units = (int64_t)s.N * a.nbands;  // per group
    a.upw = (int)std::max<int64_t>(1, (units * s.G + 2 * waves - 1) / (2 * waves));
    a.nchunks = (int)((units + 4 * a.upw - 1) / (4 * a.upw));
    if ((int64_t)a.nchunks * s.G >= (1 << 30)) return false;
    if (out) *out = a;
    if (shp) *shp = sh;
    return true;
#endif
}

template <int S, int CQ, int KQ>
void sgw_stream_launch(const SgWStreamArgs& a, const SgwStreamShape& sh, int blocks, hipStream_t st)
{
    constexpr int PF = kSgwStreamPF;
    switch (sh.nstep) {
        case 1: hipLaunchKernelGGL((sg_wgrad_stream_kernel<1, PF, S, CQ, KQ>), dim3(blocks), dim3(256), sh.lds, st, a); break;
        case 2: hipLaunchKernelGGL((sg_wgrad_stream_kernel<2, PF, S, CQ, KQ>), dim3(blocks), dim3(256), sh.lds, st, a); break;
        case 3:
            if constexpr (S == 1)
                hipLaunchKernelGGL((sg_wgrad_stream_kernel<3, PF, S, CQ, KQ>), dim3(blocks), dim3(256), sh.lds, st, a);
            break;
        default:
            if constexpr (S == 1)
                hipLaunchKernelGGL((sg_wgrad_stream_kernel<4, PF, S, CQ, KQ>), dim3(blocks), dim3(256), sh.lds, st, a);
            break;
    }
}

void sgw_stream_dispatch(const SgWStreamArgs& a, const SgwStreamShape& sh, int blocks, hipStream_t st)
{
#define SGW_CASE(s_, cq, kq) \
    if (sh.S == s_ && sh.CQ == cq && sh.KQ == kq) return sgw_stream_launch<s_, cq, kq>(a, sh, blocks, st);
    SGW_CASE(1, 1, 1) SGW_CASE(1, 1, 2) SGW_CASE(1, 2, 1) SGW_CASE(1, 2, 2)
    SGW_CASE(2, 1, 1) SGW_CASE(2, 1, 2) SGW_CASE(2, 2, 1) SGW_CASE(2, 2, 2)
#undef SGW_CASE
}

}  // namespace

// Depthwise gradWeight on the row tile: 3x3, dilation 1, stride 1 or 2, one
// input and at most 2 output channels per group; every x column the outputs
// read lies in the 64-float LDS row (rows of at most 62 outputs at stride 1,
// 31 at stride 2).
bool sg_dw_wgrad_plan(const Shape& s, SgDwWArgs* out, int* mq)
{
    if (!(s.kh == 3 && s.kw == 3 && s.dh == 1 && s.dw == 1)) return false;
    if (!(s.sh == s.sw && (s.sh == 1 || s.sh == 2))) return false;
    if (s.Cg != 1 || s.Kg > 2 || s.N < 1 || (s.Wo - 1) * s.sw + 2 > 63 || s.ph < 0 || s.pw < 0 ||
        s.pw > 2)
        return false;
    if ((int64_t)kDwwGroups * s.H * s.W * 4 >= (int64_t(1) << 30)) return false;
    if ((int64_t)kDwwGroups * s.Kg * s.Ho * s.Wo * 4 >= (int64_t(1) << 30)) return false;
    SgDwWArgs a{};
    a.N = s.N; a.C = s.C; a.H = s.H; a.W = s.W; a.K = s.K; a.Ho = s.Ho; a.Wo = s.Wo;
    a.G = s.G; a.Kg = s.Kg; a.ph = s.ph; a.pw = s.pw;
    a.S = s.sh;
    // Bands of about 16 x rows.
#ifndef GCONV_DWW_S2_RMAX
#define GCONV_DWW_S2_RMAX 8
#endif
#ifndef GCONV_DWW_WGS
#define GCONV_DWW_WGS 2048
#endif
    const int rmax = a.S == 1 ? 16 : GCONV_DWW_S2_RMAX;
    const int nb = (s.Ho + rmax - 1) / rmax;
    a.R = (s.Ho + nb - 1) / nb;
    const int ngb = (s.G + kDwwGroups - 1) / kDwwGroups;
    const int runs = std::max(1, std::min(s.N, GCONV_DWW_WGS / std::max(1, ngb)));
    a.run = (s.N + runs - 1) / runs;
    a.nruns = (s.N + a.run - 1) / a.run;
    a.plane = ((a.R - 1) * a.S + 3) * 64 + 8;
    a.dplane = a.R * 64 + 8;
    if ((int64_t)a.nruns * ngb >= (1 << 30)) return false;
    if (out) *out = a;
    if (mq) *mq = s.Kg <= 1 ? 1 : 2;
    return true;
}

// The streaming depthwise gradWeight: the shapes of sg_dw_wgrad_plan. Units
// (one image's rows, or bands of at least 8 rows where images are few) such
// that at most one round of resident waves (32 a CU) has them, a wave taking
// several units where there are more. Three steps of prefetch: mobilenet_dw
// 64.8 -> 63.1 us against the banded kernel, its stride-2 "same" layer 49.7
// -> 45.9 us; six steps measured the same, twelve slower (66.4, 62.1).
#ifndef GCONV_SG_DW_STREAM_PF
#define GCONV_SG_DW_STREAM_PF 3
#endif
constexpr int kSgDwStreamPF = GCONV_SG_DW_STREAM_PF;

bool sg_dw_stream_plan(const Shape& s, SgWStreamArgs* out, int* mq, size_t* lds)
{
#ifdef GCONV_SG_NO_DW_STREAM
    (void)s; (void)out; (void)mq; (void)lds;
    return false;
#else
    if (!sg_dw_wgrad_plan(s, nullptr, nullptr)) return false;
    const int S = s.sh, MQ = s.Kg <= 1 ? 1 : 2;
    constexpr int PF = kSgDwStreamPF, CS = 72;
    const int D = S == 1 ? 2 : 1;
    const size_t wg_lds = (size_t)4 * (S * (D + 1 + PF) + (PF + 1) * MQ) * CS * 4;
    const int per_cu = (int)std::min<size_t>(8, (160 * 1024) / wg_lds);
    const int64_t waves = (int64_t)256 * per_cu * 4;
    SgWStreamArgs a{};
    a.N = s.N; a.C = s.C; a.H = s.H; a.W = s.W; a.K = s.K; a.Ho = s.Ho; a.Wo = s.Wo;
    a.G = s.G; a.Cg = s.Cg; a.Kg = s.Kg; a.ph = s.ph; a.pw = s.pw;
    const int64_t planes = (int64_t)s.N * s.G;
    const int nb = (int)std::max<int64_t>(1, std::min<int64_t>(waves / planes, std::max(1, s.Ho / 8)));
    a.R = (s.Ho + nb - 1) / nb;
    a.nbands = (s.Ho + a.R - 1) / a.R;
    const int64_t units = (int64_t)s.N * a.nbands;  // per group
    a.upw = (int)std::max<int64_t>(1, (units * s.G + waves - 1) / waves);
    a.nchunks = (int)((units + 4 * a.upw - 1) / (4 * a.upw));
    if ((int64_t)a.nchunks * s.G >= (1 << 30)) return false;
    if (out) *out = a;
    if (mq) *mq = MQ;
    if (lds) *lds = wg_lds;
    return true;
#endif
}

#ifndef GCONV_DWW_WALK_PF
#define GCONV_DWW_WALK_PF 12
#endif
// dy rows per band: a long band where the planes are tall enough to fill it
// most of the way (fewer halo rows and partials), else a short one (its
// unrolled steps past the last row would still be issued).
#ifndef GCONV_DWW_WALK_RB1
#define GCONV_DWW_WALK_RB1 56
#endif
#ifndef GCONV_DWW_WALK_RB1S
#define GCONV_DWW_WALK_RB1S 28
#endif
#ifndef GCONV_DWW_WALK_RB2
#define GCONV_DWW_WALK_RB2 28
#endif
#ifndef GCONV_DWW_WALK_RB2S
#define GCONV_DWW_WALK_RB2S 14
#endif

// The walking depthwise gradWeight: 3x3, multiplier 1, unit dilation, stride
// 1 or 2, a plane's lanes within the wave (S = 1: Wo + 2 of them, S = 2:
// 2 Wo + 1).
bool sg_dw_wgrad_walk_plan(const Shape& s, SgDwWalkWArgs* out)
{
#ifdef GCONV_SG_NO_DWW_WALK
    (void)s; (void)out;
    return false;
#else
    if (!(s.kh == 3 && s.kw == 3 && s.dh == 1 && s.dw == 1 && s.sh == s.sw && (s.sh == 1 || s.sh == 2))) return false;
    if (s.Cg != 1 || s.Kg != 1 || s.N < 1 || s.ph < 0 || s.pw < 0) return false;
    const int lanes = s.sh == 1 ? s.Wo + 2 : 2 * s.Wo + 1;
    if (lanes > 64 || (int64_t)s.N * s.G >= (1 << 30)) return false;
    if ((int64_t)s.H * s.W * 16 >= (int64_t(1) << 30) || (int64_t)s.Ho * s.Wo * 16 >= (int64_t(1) << 30)) return false;
    SgDwWalkWArgs a{};
    a.C = s.G; a.H = s.H; a.W = s.W; a.Ho = s.Ho; a.Wo = s.Wo; a.ph = s.ph; a.pw = s.pw;
    a.planes = s.N * s.G;
    a.lpw_log2 = lanes <= 16 ? 4 : lanes <= 32 ? 5 : 6;
    const int RB = s.sh == 1 ? (s.Ho > GCONV_DWW_WALK_RB1S ? GCONV_DWW_WALK_RB1 : GCONV_DWW_WALK_RB1S)
                             : (s.Ho > GCONV_DWW_WALK_RB2S ? GCONV_DWW_WALK_RB2 : GCONV_DWW_WALK_RB2S);
    a.rb = RB;
    a.nbands = (s.Ho + RB - 1) / RB;
    const int64_t groups = ((int64_t)a.planes + (64 >> a.lpw_log2) - 1) >> (6 - a.lpw_log2);
    const int64_t waves = groups * a.nbands;
    if (waves >= (int64_t(1) << 30) || (int64_t)s.N * a.nbands * s.G * 9 >= (int64_t(1) << 31)) return false;
    a.waves = (int)waves;
    if (out) *out = a;
    return true;
#endif
}

bool smallgroup_dw_wgrad_ok(const Shape& s) { return sg_dw_wgrad_plan(s, nullptr, nullptr); }

bool smallgroup_fwd_supported(const Shape& s)
{
    return sg_problem_ok(sg_fwd_problem(s, nullptr, nullptr, nullptr, nullptr));
}

// Depthwise gradInput at stride 2 by output phase (sg_dw_dgrad_s2_kernel):
// 3x3, dilation 1, one input and one output channel per group; the phase
// columns b (and b - 1) fit the 64-float LDS row.
static bool sg_dw_dgrad_s2_plan(const Shape& s, SgDw2Args* out)
{
    if (!(s.kh == 3 && s.kw == 3 && s.sh == 2 && s.sw == 2 && s.dh == 1 && s.dw == 1)) return false;
    if (s.Cg != 1 || s.Kg != 1 || s.N < 1 || s.ph < 0 || s.pw < 0) return false;
    SgDw2Args a{};
    a.N = s.N; a.G = s.G; a.H = s.H; a.W = s.W; a.Ho = s.Ho; a.Wo = s.Wo; a.ph = s.ph; a.pw = s.pw;
    a.a_min = s.ph / 2;
    a.na = (s.H - 1 + s.ph) / 2 - a.a_min + 1;
    const int b_max = (s.W - 1 + s.pw) / 2;
    if (b_max + 1 > 63 || s.Wo + 1 > 64) return false;
    // Bands of about 8 phase rows (16 dx rows): more, smaller workgroups
    // measured faster than bands of 16 (4608 -> 9216 workgroups at 64 x 144
    // x 28 x 28 dy: 45 -> 40 us).
    const int nbands = (a.na + 7) / 8;
    a.RA = (a.na + nbands - 1) / nbands;
    a.nbands = (a.na + a.RA - 1) / a.RA;
    if ((int64_t)kDwGroups * s.Ho * s.Wo * 4 >= (int64_t(1) << 30)) return false;
    if ((int64_t)s.N * ((s.G + kDwGroups - 1) / kDwGroups) * a.nbands >= (1 << 30)) return false;
    a.div_W = make_fastdiv((uint32_t)s.W);
    if (out) *out = a;
    return true;
}

#ifndef GCONV_DW_WALKD_RB
#define GCONV_DW_WALKD_RB 14
#endif
#ifndef GCONV_DW_WALKD_PF
#define GCONV_DW_WALKD_PF 12
#endif
constexpr int kDwWalkDRows = GCONV_DW_WALKD_RB;  // dy-row steps per band

// The stride-2 gradInput walk: 3x3, multiplier 1, unit dilation, W + 2 lanes
// a plane within the wave.
static bool sg_dw_walk_dgrad_s2_plan(const Shape& s, SgDwWalkDArgs* out)
{
#ifdef GCONV_SG_NO_DW_WALKD
    (void)s; (void)out;
    return false;
#else
    if (!(s.kh == 3 && s.kw == 3 && s.sh == 2 && s.sw == 2 && s.dh == 1 && s.dw == 1)) return false;
    if (s.Cg != 1 || s.Kg != 1 || s.N < 1 || s.ph < 0 || s.pw < 0 || s.W + 2 > 64) return false;
    if ((int64_t)s.N * s.G >= (1 << 30)) return false;
    if ((int64_t)s.H * s.W * 16 >= (int64_t(1) << 30) || (int64_t)s.Ho * s.Wo * 16 >= (int64_t(1) << 30)) return false;
    SgDwWalkDArgs a{};
    a.C = s.G; a.H = s.H; a.W = s.W; a.Ho = s.Ho; a.Wo = s.Wo; a.ph = s.ph; a.pw = s.pw;
    a.planes = s.N * s.G;
    a.lpw_log2 = s.W + 2 <= 16 ? 4 : s.W + 2 <= 32 ? 5 : 6;
    // dy-row steps r_lo .. r_hi: dx rows 2r - ph and 2r - ph + 1 cover 0 .. H - 1.
    a.r_lo = s.ph / 2;
    const int r_hi = (s.H - 1 + s.ph) / 2;
    a.nsteps = r_hi - a.r_lo + 1;
    a.nbands = (a.nsteps + kDwWalkDRows - 1) / kDwWalkDRows;
    const int64_t groups = ((int64_t)a.planes + (64 >> a.lpw_log2) - 1) >> (6 - a.lpw_log2);
    const int64_t waves = groups * a.nbands;
    if (waves >= (int64_t(1) << 30)) return false;
    a.waves = (int)waves;
    if (out) *out = a;
    return true;
#endif
}

static bool sg_run_dw_walk_dgrad_s2(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st)
{
    SgDwWalkDArgs a;
    if (!sg_dw_walk_dgrad_s2_plan(s, &a)) return false;
    a.dy = dy; a.wgt = w; a.dx = dx;
    hipLaunchKernelGGL((sg_dw_walk_dgrad_s2_kernel<GCONV_DW_WALKD_PF, kDwWalkDRows>),
                       dim3((unsigned)((a.waves + 3) / 4)), dim3(256), 0, st, a);
    return true;
}

static bool sg_run_dw_dgrad_s2(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st)
{
    SgDw2Args a;
    if (!sg_dw_dgrad_s2_plan(s, &a)) return false;
    a.dy = dy; a.wgt = w; a.dx = dx;
    const int blocks = s.N * ((s.G + kDwGroups - 1) / kDwGroups) * a.nbands;
    const size_t lds = ((size_t)kDwGroups * (a.RA + 1) * 64 + (size_t)kDwGroups * 9) * 4;
    hipLaunchKernelGGL(sg_dw_dgrad_s2_kernel, dim3(blocks), dim3(256), lds, st, a);
    return true;
}

bool smallgroup_bwd_data_supported(const Shape& s)
{
    return sg_dw_walk_dgrad_s2_plan(s, nullptr) || sg_dw_dgrad_s2_plan(s, nullptr) ||
           sg_problem_ok(sg_bwd_data_problem(s, nullptr, nullptr, nullptr));
}

bool smallgroup_bwd_filter_supported(const Shape& s) { return sgw_stream_plan(s, nullptr) || sgw_plan(s, nullptr); }

size_t smallgroup_bwd_filter_workspace(const Shape& s)
{
    SgDwWArgs da;
    int mq;
    SgDwWalkWArgs wa;
    if (sg_dw_wgrad_walk_plan(s, &wa)) return (size_t)s.N * wa.nbands * s.G * 9 * sizeof(float);
    SgWStreamArgs dsa;
    size_t dlds;
    if (sg_dw_stream_plan(s, &dsa, &mq, &dlds)) return (size_t)dsa.nchunks * s.G * mq * 9 * sizeof(float);
    if (sg_dw_wgrad_plan(s, &da, &mq)) return (size_t)da.nruns * s.G * mq * 9 * sizeof(float);
    SgWStreamArgs sa;
    SgwStreamShape sh;
    if (sgw_stream_plan(s, &sa, &sh)) return (size_t)sa.nchunks * s.G * 16 * sh.CQ * sh.KQ * 9 * sizeof(float);
    SgWArgs a;
    bool row64 = false;
    if (!sgw_plan(s, &a, &row64)) return 0;
    const size_t sets = row64 ? (size_t)a.nruns : (size_t)s.N * a.nbands;
    return sets * s.G * 16 * s.kh * s.kw * sizeof(float);
}

bool smallgroup_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y,
                    hipStream_t st)
{
    return sg_run(sg_fwd_problem(s, x, w, bias, y), st);
}

bool smallgroup_bwd_data(const Shape& s, const float* dy, const float* w, float* dx,
                         hipStream_t st)
{
    if (sg_dw_walk_dgrad_s2_plan(s, nullptr)) return sg_run_dw_walk_dgrad_s2(s, dy, w, dx, st);
#ifndef GCONV_SG_NO_DW_S2_PHASE
    if (sg_dw_dgrad_s2_plan(s, nullptr)) return sg_run_dw_dgrad_s2(s, dy, w, dx, st);
#endif
    return sg_run(sg_bwd_data_problem(s, dy, w, dx), st);
}

bool smallgroup_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws,
                           hipStream_t st)
{
    SgDwWArgs da;
    int mq;
    {
        SgDwWalkWArgs wa;
        if (sg_dw_wgrad_walk_plan(s, &wa)) {
            wa.x = x; wa.dy = dy; wa.ws = ws;
            const dim3 grid((unsigned)((wa.waves + 3) / 4));
            constexpr int PF = GCONV_DWW_WALK_PF;
            if (s.sh == 1) {
                if (wa.rb == GCONV_DWW_WALK_RB1)
                    hipLaunchKernelGGL((sg_dw_wgrad_walk_kernel<1, PF, GCONV_DWW_WALK_RB1>), grid, dim3(256), 0, st, wa);
                else
                    hipLaunchKernelGGL((sg_dw_wgrad_walk_kernel<1, PF, GCONV_DWW_WALK_RB1S>), grid, dim3(256), 0, st, wa);
            } else {
                if (wa.rb == GCONV_DWW_WALK_RB2)
                    hipLaunchKernelGGL((sg_dw_wgrad_walk_kernel<2, PF, GCONV_DWW_WALK_RB2>), grid, dim3(256), 0, st, wa);
                else
                    hipLaunchKernelGGL((sg_dw_wgrad_walk_kernel<2, PF, GCONV_DWW_WALK_RB2S>), grid, dim3(256), 0, st, wa);
            }
            const int E = s.G * 9;
            hipLaunchKernelGGL(sg_dw_wgrad_reduce, dim3((E + 15) / 16), dim3(256), 0, st, ws, dw, s.N * wa.nbands,
                               s.G, 1, 1);
            return true;
        }
    }
    {
        SgWStreamArgs dsa;
        size_t dlds;
        if (sg_dw_stream_plan(s, &dsa, &mq, &dlds)) {
            dsa.x = x; dsa.dy = dy; dsa.ws = ws;
            constexpr int PF = kSgDwStreamPF;
            const dim3 grid(dsa.nchunks * s.G);
            if (s.sh == 1) {
                if (mq == 1) hipLaunchKernelGGL((sg_dw_wgrad_stream_kernel<1, 1, PF>), grid, dim3(256), dlds, st, dsa);
                else hipLaunchKernelGGL((sg_dw_wgrad_stream_kernel<1, 2, PF>), grid, dim3(256), dlds, st, dsa);
            } else {
                if (mq == 1) hipLaunchKernelGGL((sg_dw_wgrad_stream_kernel<2, 1, PF>), grid, dim3(256), dlds, st, dsa);
                else hipLaunchKernelGGL((sg_dw_wgrad_stream_kernel<2, 2, PF>), grid, dim3(256), dlds, st, dsa);
            }
            const int E = s.G * s.Kg * 9;
            hipLaunchKernelGGL(sg_dw_wgrad_reduce, dim3((E + 15) / 16), dim3(256), 0, st, ws, dw, dsa.nchunks, s.G,
                               s.Kg, mq);
            return true;
        }
    }
    if (sg_dw_wgrad_plan(s, &da, &mq)) {
        da.x = x; da.dy = dy; da.ws = ws;
        const int ngb = (s.G + kDwwGroups - 1) / kDwwGroups;
        const int blocks = ngb * da.nruns;
        const size_t lds = std::max((size_t)kDwwGroups * da.plane + (size_t)kDwwGroups * mq * da.dplane,
                                    (size_t)4 * kDwwGroups * mq * 9) * 4;
        if (da.S == 1) {
            if (mq == 1) hipLaunchKernelGGL((sg_dw_wgrad_kernel<1, 1>), dim3(blocks), dim3(256), lds, st, da);
            else hipLaunchKernelGGL((sg_dw_wgrad_kernel<2, 1>), dim3(blocks), dim3(256), lds, st, da);
        } else {
            if (mq == 1) hipLaunchKernelGGL((sg_dw_wgrad_kernel<1, 2>), dim3(blocks), dim3(256), lds, st, da);
            else hipLaunchKernelGGL((sg_dw_wgrad_kernel<2, 2>), dim3(blocks), dim3(256), lds, st, da);
        }
        const int E = s.G * s.Kg * 9;
        hipLaunchKernelGGL(sg_dw_wgrad_reduce, dim3((E + 15) / 16), dim3(256), 0, st, ws, dw, da.nruns, s.G,
                           s.Kg, mq);
        return true;
    }
    SgWStreamArgs sa;
    SgwStreamShape sh;
    if (sgw_stream_plan(s, &sa, &sh)) {
        sa.x = x; sa.dy = dy; sa.ws = ws;
        sgw_stream_dispatch(sa, sh, sa.nchunks * s.G, st);
        const int total = s.G * 16 * sh.CQ * sh.KQ * 9;
        hipLaunchKernelGGL(sg_wgrad_reduce, dim3((total + 15) / 16), dim3(256), 0, st, ws, dw,
                           sa.nchunks, s.G, s.Kg, s.Cg, 9, 4 * sh.KQ, 4 * sh.CQ);
        return true;
    }
    SgWArgs a;
    bool row64 = false;
    if (!sgw_plan(s, &a, &row64)) return false;
    a.x = x;
    a.dy = dy;
    a.ws = ws;
    const int T = s.kh * s.kw;
    const int blocks = s.N * a.nbands * s.G;
    if (row64) {
        const size_t lds = std::max((size_t)4 * a.plane + (size_t)4 * a.dplane, (size_t)4 * T * 16) * 4;
        const int nstep = (s.Wo + 15) / 16;
        const int rblocks = a.nruns * s.G;
        if (nstep == 1) hipLaunchKernelGGL(sg_wgrad_row64_kernel<1>, dim3(rblocks), dim3(256), lds, st, a);
        else if (nstep == 2) hipLaunchKernelGGL(sg_wgrad_row64_kernel<2>, dim3(rblocks), dim3(256), lds, st, a);
        else if (nstep == 3) hipLaunchKernelGGL(sg_wgrad_row64_kernel<3>, dim3(rblocks), dim3(256), lds, st, a);
        else hipLaunchKernelGGL(sg_wgrad_row64_kernel<4>, dim3(rblocks), dim3(256), lds, st, a);
        const int total = s.G * 16 * T;
        hipLaunchKernelGGL(sg_wgrad_reduce, dim3((total + 15) / 16), dim3(256), 0, st, ws, dw,
                           a.nruns, s.G, s.Kg, s.Cg, T, 4, 4);
        return true;
    } else {
        const size_t lds =
            std::max((size_t)ceil64(4 * a.plane) + (size_t)4 * a.dplane, (size_t)4 * T * 16) * 4;
        hipLaunchKernelGGL((sg_wgrad_kernel<3, 3>), dim3(blocks), dim3(256), lds, st, a);
    }
    const int total = s.G * 16 * T;
    hipLaunchKernelGGL(sg_wgrad_reduce, dim3((total + 15) / 16), dim3(256), 0, st, ws, dw,
                       s.N * a.nbands, s.G, s.Kg, s.Cg, T, 4, 4);
    return true;
}

}  // namespace gconv
