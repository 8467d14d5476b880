// conv_mfma.hip -- fp32-MFMA implicit-GEMM kernel for the forward pass and,
// at stride 1, for gradInput. Grouped 2-D convolution, NCHW.
//
// Per group g the forward pass is a GEMM
//     out[o, p] = sum_{r < Cin_g, t < kh*kw} W[o, r, t] * in[r, p shifted by tap t]
// over output pixels p (the im2col matrix is never built). gradInput at
// stride 1 is the same computation on dy with the filter transposed
// (W[k, c, t] read as W'[c, k, T-1-t]) and padding (k-1)*d - p: the
// adjoint of a stride-1 correlation is the correlation with the reversed
// kernel. One launch covers every group: the group is a grid coordinate
// and each group's planes are reached through offsets
// ("[Feature request] Groups support for SpatialConvolutionMM": offsets per
// group instead of narrowed copies, one kernel over all groups).
//
// Tiling (gfx950, wave64, v_mfma_f32_16x16x4f32):
//   block  = 256 threads = 4 waves; one image, BP = 64*MP consecutive output
//            pixels of that image, BO = 16*MO output channels of one group.
//   wave   = 16*MP pixels x BO channels: MP x MO accumulators of 16x16.
//   MFMA   = A: 16 pixels x 4 reduction channels (one tap), read from the
//            LDS input tile at a per-lane pixel base plus a per-tap offset;
//            B: 4 reduction channels x 16 output channels from the LDS
//            weight tile; D: lane l holds pixels 4*(l/16)+v of channel l%16.
//   LDS    = input rows covering the tile's pixels plus the kernel halo, all
//            padded columns, CC channels; weights [tap][CC][BO] of the chunk.
//            Zero padding is materialised in LDS, so the MFMA loop has no
//            masks. Reduction channels advance CC at a time; the next chunk
//            is fetched into registers while the current one is multiplied.
#include <algorithm>

#include "device_util.h"
#include "fastdiv.h"
#include "gconv.h"
#include "gconv_internal.h"

namespace gconv {
namespace {

struct ConvMfmaArgs {
    const float* in;
    const float* wgt;
    const float* bias;
    float* out;
    int N, G;
    int Cin_tot, Cin_g, Hin, Win;
    int Cout_tot, Cout_g, Hout, Wout;
    int sh, sw, dh, dw, ph, pw;
    int w_so, w_sr, w_gstride;  // weight strides: output channel, reduction channel, group
    int tiles_per_image, n_otiles;
    int LW, LR, plane;          // LDS input tile: row width, rows, channel plane stride
    int relu;                   // forward epilogue: max(v, 0)
    FastDiv div_RW, div_LW, div_Wout;
};

template <int KH, int KW, int MP, int MO, int CC, int XPF, bool FLIP>
__global__ void __launch_bounds__(256, 2) conv_mfma_kernel(ConvMfmaArgs a)
{
    constexpr int T = KH * KW;
    constexpr int BO = 16 * MO;
    constexpr int BOP = (BO % 64 == 16) ? BO : ((BO + 47) / 64) * 64 + 16;  // == 16 mod 64
    constexpr int WP = 16 * MP;
    constexpr int BP = 4 * WP;
    constexpr int PARTS = 256 / BO;                   // weight loader: threads per channel
    constexpr int WLEN = (CC * T + PARTS - 1) / PARTS;

    extern __shared__ float lds[];
    float* xs = lds;                     // [CC][plane]
    float* ws = lds + CC * a.plane;      // [T][CC][BOP]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q = lane >> 4;

    int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int ot = bid % a.n_otiles;
    bid /= a.n_otiles;
    const int g = bid % a.G;
    bid /= a.G;
    const int pt = bid % a.tiles_per_image;
    const int n = bid / a.tiles_per_image;

    const int P = a.Hout * a.Wout;
    const int p0 = pt * BP;
    const int p1 = min(P, p0 + BP);
    const int ho_first = (int)fastdiv((uint32_t)p0, a.div_Wout);
    const int hbase = ho_first * a.sh - a.ph;
    const int o0 = ot * BO;

    // Per-lane LDS offset of each of its MP pixels (tap (0,0), channel 0).
    // Pixels past the tile end are clamped to the last one (never stored).
    int base[MP];
#pragma unroll
    for (int f = 0; f < MP; ++f) {
        const int p = min(p0 + wave * WP + f * 16 + l16, p1 - 1);
        const int ho = (int)fastdiv((uint32_t)p, a.div_Wout);
        const int wo = p - ho * a.Wout;
        base[f] = (ho - ho_first) * a.sh * a.LW + wo * a.sw;
    }

    const float* in_g = a.in + ((size_t)n * a.Cin_tot + (size_t)g * a.Cin_g) * a.Hin * a.Win;
    const float* w_g = a.wgt + (size_t)g * a.w_gstride;
    const int RW = a.LR * a.LW;
    const int xtotal = CC * RW;

    float xr[XPF];
    float wr[WLEN];
    // This block's input planes (group g of image n) and group weights.
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(in_g, (uint32_t)a.Cin_g * a.Hin * a.Win * 4u);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_g, (uint32_t)a.w_gstride * 4u);
    const int dummy = CC * a.plane + T * CC * BOP;  // LDS slot that absorbs unused stores
    const int wo_ = tid % BO, wpart = tid / BO;

    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int k = 0; k < XPF; ++k) {
            const int e = tid + 256 * k;
            const int c = (int)fastdiv((uint32_t)e, a.div_RW);
            const int rem = e - c * RW;
            const int r = (int)fastdiv((uint32_t)rem, a.div_LW);
            const int col = rem - r * a.LW;
            const int h = hbase + r, w = col - a.pw;
            // Channels past the group end fall outside the resource and read 0.
            const bool ok = e < xtotal && (unsigned)h < (unsigned)a.Hin &&
                            (unsigned)w < (unsigned)a.Win;
            const uint32_t off = ok ? (uint32_t)(((c0 + c) * a.Hin + h) * a.Win + w) * 4u : kOOB;
            xr[k] = load_f32(rx, off);
        }
#pragma unroll
        for (int k = 0; k < WLEN; ++k) {
            const int rt = wpart * WLEN + k;
            const int r = rt / T, t = rt % T;
            const int oo = o0 + wo_, rr = c0 + r;
            const bool ok = wpart < PARTS && rt < CC * T && oo < a.Cout_g && rr < a.Cin_g;
            const uint32_t off =
                ok ? (uint32_t)(oo * a.w_so + rr * a.w_sr + (FLIP ? T - 1 - t : t)) * 4u : kOOB;
            wr[k] = load_f32(rw, off);
        }
    };
    auto store_chunk = [&]() {
#pragma unroll
        for (int k = 0; k < XPF; ++k) {
            const int e = tid + 256 * k;
            const int c = (int)fastdiv((uint32_t)e, a.div_RW);
            xs[e < xtotal ? c * a.plane + (e - c * RW) : dummy] = xr[k];
        }
#pragma unroll
        for (int k = 0; k < WLEN; ++k) {
            const int rt = wpart * WLEN + k;
            const int r = rt / T, t = rt % T;
            // ws starts CC*plane floats into LDS; the dummy slot follows the weight tile.
            ws[(wpart < PARTS && rt < CC * T) ? (t * CC + r) * BOP + wo_ : T * CC * BOP] = wr[k];
        }
    };

    f4 acc[MP][MO];
#pragma unroll
    for (int f = 0; f < MP; ++f)
#pragma unroll
        for (int m = 0; m < MO; ++m) acc[f][m] = f4{0.f, 0.f, 0.f, 0.f};

    const int nchunks = (a.Cin_g + CC - 1) / CC;
    load_chunk(0);
    store_chunk();
    __syncthreads();
    const float* xq = xs + q * a.plane;
    const float* wq = ws + q * BOP + l16;
    for (int chunk = 0; chunk < nchunks; ++chunk) {
        const bool more = chunk + 1 < nchunks;
        if (more) load_chunk((chunk + 1) * CC);
#pragma unroll 1
        for (int cq = 0; cq < CC / 4; ++cq) {
            // Operands of tap t+1 are read from LDS while the MFMAs of tap t
            // run; the scheduling barrier keeps the compiler from hoisting
            // every tap's loads (which would exhaust the register file).
            const float* xc = xq + cq * 4 * a.plane;
            const float* wc = wq + cq * 4 * BOP;
            float av[2][MP], bv[2][MO];
#pragma unroll
            for (int f = 0; f < MP; ++f) av[0][f] = xc[base[f]];
#pragma unroll
            for (int m = 0; m < MO; ++m) bv[0][m] = wc[m * 16];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int cur = t & 1, nxt = cur ^ 1;
                if (t + 1 < T) {
                    const int i = (t + 1) / KW, j = (t + 1) % KW;
                    const int toff = i * a.dh * a.LW + j * a.dw;
#pragma unroll
                    for (int f = 0; f < MP; ++f) av[nxt][f] = xc[base[f] + toff];
#pragma unroll
                    for (int m = 0; m < MO; ++m) bv[nxt][m] = wc[(t + 1) * CC * BOP + m * 16];
                }
#pragma unroll
                for (int f = 0; f < MP; ++f)
#pragma unroll
                    for (int m = 0; m < MO; ++m)
                        acc[f][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[cur][f], bv[cur][m],
                                                                         acc[f][m], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (more) {
            __syncthreads();  // every wave is done reading this chunk
            store_chunk();
            __syncthreads();  // the next chunk is in LDS
        }
    }

    // Epilogue: bias, then stores. Lane l holds pixels 4*(l/16)+v of channel l%16.
    float* out_g = a.out + ((size_t)n * a.Cout_tot + (size_t)g * a.Cout_g) * P;
    const bool vec4 = (P & 3) == 0;
#pragma unroll
    for (int m = 0; m < MO; ++m) {
        const int o = o0 + m * 16 + l16;
        if (o >= a.Cout_g) continue;
        const float bv = a.bias ? a.bias[g * a.Cout_g + o] : 0.f;
        float* orow = out_g + (size_t)o * P;
#pragma unroll
        for (int f = 0; f < MP; ++f) {
            const int pb = p0 + wave * WP + f * 16 + 4 * q;
            f4 v = acc[f][m];
            v.x += bv;
            v.y += bv;
            v.z += bv;
            v.w += bv;
            if (a.relu) {
                v.x = relu_if(v.x, 1);
                v.y = relu_if(v.y, 1);
                v.z = relu_if(v.z, 1);
                v.w = relu_if(v.w, 1);
            }
            if (vec4) {
                if (pb < p1) *(f4*)(orow + pb) = v;
            } else {
                if (pb + 0 < p1) orow[pb + 0] = v.x;
                if (pb + 1 < p1) orow[pb + 1] = v.y;
                if (pb + 2 < p1) orow[pb + 2] = v.z;
                if (pb + 3 < p1) orow[pb + 3] = v.w;
            }
        }
    }
}

// ---- flattened-pixel variant ------------------------------------------------
//
// Same GEMM, tiled differently: a block owns BPX = 16*MP*WPX consecutive
// output pixels of the flattened (image, row, column) index, so the tile count
// no longer rounds up per image and the last tile of an image is not mostly
// empty. Such a run of pixels touches at most two images (BPX <= Hout*Wout);
// the LDS input tile holds the needed input rows of the first image followed
// by those of the second ("virtual rows"). The block's WO*WPX waves split it
// as WPX pixel groups x WO output-channel groups; a wave owns MP pixel
// fragments of 16 and MO output fragments of 16 (three waves of one fragment
// cover 48 channels exactly).
//   - input planes go global -> LDS with buffer_load ... lds (no register
//     staging), double-buffered over chunks of 4 reduction channels;
//   - each wave keeps its own filter column (4 channels x T taps x MO) in
//     registers, prefetched one chunk ahead, so LDS holds only the input tile;
//   - per tap the LDS reads of the next tap are issued ahead of this tap's
//     MFMAs.
struct ConvFlatArgs {
    const float* in;
    const float* wgt;
    const float* bias;
    float* out;
    int N, G;
    int Cin_tot, Cin_g, Hin, Win;
    int Cout_tot, Cout_g, Hout, Wout;
    int sh, sw, dh, dw, ph, pw;
    int w_so, w_sr, w_gstride;
    int P, NP;                  // Hout*Wout, N*P
    int n_otiles;
    int LW, plane, nseg, bufsz; // LDS row width, channel plane, DMA segments per wave, floats per buffer
    int halo;                   // (kh-1)*dh + 1 input rows under one output row
    // Input upsampling (strided gradInput): Hin x Win is the virtual input, in
    // which only rows and columns divisible by uh, uw hold values, row h/uh and
    // column w/uw of the stored Hr x Wr planes; 1, 1 otherwise.
    int uh, uw, Hr, Wr;
    int relu;                   // forward epilogue: max(v, 0)
    int out_nhwc;               // store the output channels-last, [N][Hout*Wout][Cout_tot]
    FastDiv div_P, div_Wout, div_plane, div_LW;
    // Packed groups (pk_o > 0): a "group" of the launch is several real
    // groups side by side, pk_o output and pk_r reduction channels each, with
    // a block-diagonal filter (w_gs floats per real group; zero across groups).
    int pk_o, pk_r, w_gs;
    // Sub-pixel form of a strided gradInput (SP instances): the launch's
    // output channel o = (c*o_sh + du)*o_sw + dv at pixel (a, b) is dx channel
    // c of the group (sp_cg per group) at (a*o_sh + du, b*o_sw + dv) of the
    // o_H x o_W planes. With the padding written p = sp_bh*o_sh + sp_rh, that
    // row's stored taps are i = u + o_sh*i' with u = (du + p) mod o_sh, and
    // tap i reads dy row a + (du + p) div o_sh - i'; super-tap ti reads dy
    // row a + sp_mh + ti (sp_mh the least such offset). Columns alike. The
    // stored filter has sp_kh x sp_kw taps.
    int o_sh, o_sw, o_H, o_W;
    int sp_cg, sp_bh, sp_rh, sp_bw, sp_rw, sp_mh, sp_mw, sp_kh, sp_kw;
    int sp_vec;                 // 2x2 sub-pixels, Hout*Wout and Wout multiples of 4, o_W == 2*Wout, NCHW
};

// Lane l and lane l ^ 1 exchange a value (DPP quad permutation 1, 0, 3, 2).
__device__ __forceinline__ float swap_pair(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}

// INH: the input is channels-last ([N][Hr][Wr][Cin_tot]); the LDS tile then
// holds each pixel's 4 chunk channels together ([row][col][4]), filled by
// 16-byte DMA (one pixel per lane), and a fragment's 16 pixels x 4 channels
// read 64 consecutive floats.
// PK: packed groups (pk_o > 0; instances with one fragment and one wave
// across the output channels only), so the filter addressing of unpacked
// launches carries none of it.
template <int KH, int KW, int MP, int MO, int WO, int WPX, int NSX, bool FLIP, int MINW, bool INH = false,
          bool SP = false, bool PK = false>
__global__ void __launch_bounds__(64 * WO * WPX, MINW) conv_flat_kernel(ConvFlatArgs a)
{
    constexpr int T = KH * KW;
    constexpr int CC = 4;
    constexpr int NW = WO * WPX;
    constexpr int BPX = WPX * MP * 16;
    constexpr int BO = WO * MO * 16;

    extern __shared__ float lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q = lane >> 4;
    const int wo_i = wave % WO, wp_i = wave / WO;

    int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int ot = bid % a.n_otiles;
    bid /= a.n_otiles;
    const int g = bid % a.G;
    const int pt = bid / a.G;

    const int q0 = pt * BPX;
    const int q1 = min(a.NP, q0 + BPX);
    const int n0 = (int)fastdiv((uint32_t)q0, a.div_P);
    const int ho0 = (int)fastdiv((uint32_t)(q0 - n0 * a.P), a.div_Wout);
    const int nl = (int)fastdiv((uint32_t)(q1 - 1), a.div_P);
    const int hol = (int)fastdiv((uint32_t)(q1 - 1 - nl * a.P), a.div_Wout);
    int rows0, rows1;
    if (nl == n0) {
        rows0 = (hol - ho0) * a.sh + a.halo;
        rows1 = 0;
    } else {
        rows0 = (a.Hout - 1 - ho0) * a.sh + a.halo;
        rows1 = hol * a.sh + a.halo;
    }
    const int hA = ho0 * a.sh - a.ph;  // input row of virtual row 0
    const int HWin = a.Hr * a.Wr;

    // Per-lane global byte offset of each DMA segment element (chunk-relative:
    // the buffer resource moves with the chunk). Out-of-image taps, rows past
    // the tile and the plane padding read 0.
    uint32_t xoff[NSX];
#pragma unroll
    for (int k = 0; k < NSX; ++k) {
        const int e = (wave + NW * k) * 64 + lane;  // INH: the pixel slot of the tile
        const int c = INH ? 0 : (int)fastdiv((uint32_t)e, a.div_plane);
        const int rem = INH ? e : e - c * a.plane;
        const int v = (int)fastdiv((uint32_t)rem, a.div_LW);
        const int col = rem - v * a.LW;
        const bool second = v >= rows0;
        const int h = second ? v - rows0 - a.ph : hA + v;
        const int w = col - a.pw;
        bool ok = k < a.nseg && c < CC && v < rows0 + rows1 && (unsigned)h < (unsigned)a.Hin &&
                  (unsigned)w < (unsigned)a.Win;
        int hr = h, wr = w;
        if (a.uh != 1 || a.uw != 1) {   // upsampled input: the other positions are 0
            hr = h / a.uh;
            wr = w / a.uw;
            ok = ok && hr * a.uh == h && wr * a.uw == w;
        }
        if constexpr (INH)
            xoff[k] = ok ? (uint32_t)(((second ? HWin : 0) + hr * a.Wr + wr) * a.Cin_tot) * 4u : kOOB;
        else
            xoff[k] = ok ? (uint32_t)(((second ? a.Cin_tot : 0) + c) * HWin + hr * a.Wr + wr) * 4u : kOOB;
    }

    // LDS address (floats, buffer-relative) of each pixel fragment at tap 0,
    // reduction channel q of the chunk. Pixels past the tile end are clamped
    // to the last one (computed, never stored).
    int la[MP];
#pragma unroll
    for (int f = 0; f < MP; ++f) {
        const int qq = min(q0 + (wp_i * MP + f) * 16 + l16, q1 - 1);
        const int n = (int)fastdiv((uint32_t)qq, a.div_P);
        const int p = qq - n * a.P;
        const int ho = (int)fastdiv((uint32_t)p, a.div_Wout);
        const int wo = p - ho * a.Wout;
        const int v = (n == n0) ? (ho - ho0) * a.sh : rows0 + ho * a.sh;
        la[f] = INH ? (v * a.LW + wo * a.sw) * 4 + q : q * a.plane + v * a.LW + wo * a.sw;
    }

    // Filter operands: lane (l16, q) holds W[o = l16 of fragment m][r = c0 + q][tap].
    const int o0 = ot * BO;
    const float* w_g = a.wgt + (size_t)g * a.w_gstride;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_g, (uint32_t)a.w_gstride * 4u);
    int wbase[MO];  // -1: output channel past the group end
    int osub[PK ? MO : 1];  // packed groups: the real group of the output channel
    int soff[SP ? MO : 1][SP ? T : 1];  // sub-pixel form: stored tap of each super-tap, -1 none
#pragma unroll
    for (int m = 0; m < MO; ++m) {
        const int o = o0 + (wo_i * MO + m) * 16 + l16;
        if constexpr (PK) {
            osub[m] = o / a.pk_o;
            wbase[m] = o >= a.Cout_g ? -1 : osub[m] * a.w_gs + (o - osub[m] * a.pk_o) * a.w_so;
        } else {
            wbase[m] = o >= a.Cout_g ? -1 : o * a.w_so;
        }
        if constexpr (SP) {
            const int c = o / (a.o_sh * a.o_sw), rem = o - c * (a.o_sh * a.o_sw);
            const int du = rem / a.o_sw, dv = rem - du * a.o_sw;
            wbase[m] = o >= a.Cout_g ? -1 : c * a.w_so;
            const bool ch = du + a.sp_rh >= a.o_sh, cw = dv + a.sp_rw >= a.o_sw;
            const int Ah = a.sp_bh + ch - a.sp_mh, uh = du + a.sp_rh - (ch ? a.o_sh : 0);
            const int Aw = a.sp_bw + cw - a.sp_mw, uw = dv + a.sp_rw - (cw ? a.o_sw : 0);
#pragma unroll
            for (int ti = 0; ti < KH; ++ti)
#pragma unroll
                for (int tj = 0; tj < KW; ++tj) {
                    const int i = uh + a.o_sh * (Ah - ti), j = uw + a.o_sw * (Aw - tj);
                    soff[m][ti * KW + tj] =
                        (Ah - ti >= 0 && i < a.sp_kh && Aw - tj >= 0 && j < a.sp_kw) ? i * a.sp_kw + j : -1;
                }
        }
    }
    auto load_b = [&](int c0, float (&b)[MO][T]) {
        const int r = c0 + q;
        if constexpr (SP) {
#pragma unroll
            for (int m = 0; m < MO; ++m) {
                const uint32_t base =
                    (r < a.Cin_g && wbase[m] >= 0) ? (uint32_t)(wbase[m] + r * a.w_sr) * 4u : kOOB;
#pragma unroll
                for (int t = 0; t < T; ++t)
                    b[m][t] = load_f32(rw, soff[m][t] >= 0 ? base + (uint32_t)soff[m][t] * 4u : kOOB);
            }
            return;
        }
#pragma unroll
        for (int m = 0; m < MO; ++m) {
            // One select per fragment; the tap offsets then ride on the
            // instruction's immediate offset (out-of-range stays out of range).
            uint32_t base;
            if constexpr (PK) {
                // packed groups: filter values across real groups are 0
                const int rsub = r / a.pk_r, rr = r - rsub * a.pk_r;
                base = (r < a.Cin_g && wbase[m] >= 0 && rsub == osub[m]) ? (uint32_t)(wbase[m] + rr * a.w_sr) * 4u
                                                                          : kOOB;
            } else {
                base = (r < a.Cin_g && wbase[m] >= 0) ? (uint32_t)(wbase[m] + r * a.w_sr) * 4u : kOOB;
            }
#pragma unroll
            for (int t = 0; t < T; ++t) b[m][t] = load_f32(rw, base + (uint32_t)t * 4u);
        }
    };
    // Taps in memory order (so the loads merge into 16-byte ones); the flipped
    // filter of gradInput picks them in reverse at the MFMA.
    constexpr auto tap = [](int t) { return FLIP ? T - 1 - t : t; };

    const float* in_n0 = INH ? a.in + (size_t)n0 * HWin * a.Cin_tot + (size_t)g * a.Cin_g
                             : a.in + ((size_t)n0 * a.Cin_tot + (size_t)g * a.Cin_g) * HWin;
    const uint32_t second_recs = rows1 > 0 ? (uint32_t)a.Cin_tot * HWin : 0u;
    auto issue_x_nhwc = [&](int c0, int buf) {
        // Chunks are whole (Cin_g % 4 == 0): 16 bytes per pixel, all inside the group.
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(
            in_n0 + c0, (second_recs + (uint32_t)a.Cin_tot * HWin - (uint32_t)(g * a.Cin_g + c0)) * 4u);
        float* dst = lds + buf * a.bufsz + wave * 256;
#pragma unroll
        for (int k = 0; k < NSX; ++k)
            if (k < a.nseg) load_lds256(rx, dst + k * (NW * 256), xoff[k]);
    };
    auto issue_x = [&](int c0, int buf) {
        if constexpr (INH) {
            issue_x_nhwc(c0, buf);
            return;
        }
        const __amdgpu_buffer_rsrc_t rx =
            make_rsrc(in_n0 + (size_t)c0 * HWin, (second_recs + (uint32_t)(a.Cin_g - c0) * HWin) * 4u);
        // Channels past the group end: the second image's fall outside the
        // resource; the first image's would alias the next group, so mask them.
        // (A uniform branch: whole chunks issue their DMA with no per-lane select.)
        const int lim = min(CC, a.Cin_g - c0) * a.plane;
        float* dst = lds + buf * a.bufsz + wave * 64;
        if (lim >= CC * a.plane) {
#pragma unroll
            for (int k = 0; k < NSX; ++k)
                if (k < a.nseg) load_lds64(rx, dst + k * (NW * 64), xoff[k]);
        } else {
#pragma unroll
            for (int k = 0; k < NSX; ++k)
                if (k < a.nseg)
                    load_lds64(rx, dst + k * (NW * 64),
                               ((wave + NW * k) * 64 + lane < lim) ? xoff[k] : kOOB);
        }
    };

    f4 acc[MP][MO];
#pragma unroll
    for (int f = 0; f < MP; ++f)
#pragma unroll
        for (int m = 0; m < MO; ++m) acc[f][m] = f4{0.f, 0.f, 0.f, 0.f};

    const int nchunks = (a.Cin_g + CC - 1) / CC;
    float bn[MO][T];
    load_b(0, bn);
    issue_x(0, 0);
    for (int ch = 0; ch < nchunks; ++ch) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA of chunk ch landed
        __syncthreads();  // every wave's DMA landed; every wave is done with chunk ch-1
        float bc[MO][T];
#pragma unroll
        for (int m = 0; m < MO; ++m)
#pragma unroll
            for (int t = 0; t < T; ++t) bc[m][t] = bn[m][t];
        if (ch + 1 < nchunks) {
            issue_x((ch + 1) * CC, (ch + 1) & 1);
            load_b((ch + 1) * CC, bn);
        }
        if (MO == 1 && a.dw == 1) {
            // Unit column dilation: a row's taps sit at compile-time offsets
            // from one address per fragment, so the LDS reads take immediate
            // offsets and only each filter row's start is added. (Instances
            // with two output fragments per wave keep the general form: the
            // extra registers cost them more than the adds.)
            constexpr int CS = INH ? 4 : 1;
            const int rstep = a.dh * a.LW * CS;
            const int boff = (ch & 1) * a.bufsz;
            int ra[MP];
#pragma unroll
            for (int f = 0; f < MP; ++f) ra[f] = la[f] + boff;
            float av[2][MP];
#pragma unroll
            for (int f = 0; f < MP; ++f) av[0][f] = lds[ra[f]];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int cur = t & 1, nxt = cur ^ 1;
                if (t + 1 < T) {
                    const int j = (t + 1) % KW;
                    if (j == 0) {
#pragma unroll
                        for (int f = 0; f < MP; ++f) ra[f] += rstep;
                    }
#pragma unroll
                    for (int f = 0; f < MP; ++f) av[nxt][f] = lds[ra[f] + j * CS];
                }
#pragma unroll
                for (int f = 0; f < MP; ++f)
#pragma unroll
                    for (int m = 0; m < MO; ++m)
                        acc[f][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[cur][f], bc[m][tap(t)],
                                                                         acc[f][m], 0, 0, 0);
                if (t + 1 < T) __builtin_amdgcn_sched_group_barrier(0x100, MP, 0);  // LDS reads first
                __builtin_amdgcn_sched_group_barrier(0x008, MP * MO, 0);          // then the MFMAs
                __builtin_amdgcn_sched_barrier(0);
            }
            continue;
        }
        const float* xb = lds + (ch & 1) * a.bufsz;
        float av[2][MP];
#pragma unroll
        for (int f = 0; f < MP; ++f) av[0][f] = xb[la[f]];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int cur = t & 1, nxt = cur ^ 1;
            if (t + 1 < T) {
                const int i = (t + 1) / KW, j = (t + 1) % KW;
                const int toff = (i * a.dh * a.LW + j * a.dw) * (INH ? 4 : 1);
#pragma unroll
                for (int f = 0; f < MP; ++f) av[nxt][f] = xb[la[f] + toff];
            }
#pragma unroll
            for (int f = 0; f < MP; ++f)
#pragma unroll
                for (int m = 0; m < MO; ++m)
                    acc[f][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[cur][f], bc[m][tap(t)],
                                                                     acc[f][m], 0, 0, 0);
            if (t + 1 < T) __builtin_amdgcn_sched_group_barrier(0x100, MP, 0);  // LDS reads first
            __builtin_amdgcn_sched_group_barrier(0x008, MP * MO, 0);          // then the MFMAs
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Epilogue: lane (l16, q) holds output channel l16 of each fragment,
    // pixels 4q..4q+3 of each pixel fragment.
    const bool vec4 = (a.P & 3) == 0;
#pragma unroll
    for (int m = 0; m < MO; ++m) {
        const int o = o0 + (wo_i * MO + m) * 16 + l16;
        if (o >= a.Cout_g) continue;
        const float bv = a.bias ? a.bias[g * a.Cout_g + o] : 0.f;
        const size_t ch_off = (size_t)g * a.Cout_g + o;
#pragma unroll
        for (int f = 0; f < MP; ++f) {
            const int qb = q0 + (wp_i * MP + f) * 16 + 4 * q;
            f4 v = acc[f][m];
            v.x += bv;
            v.y += bv;
            v.z += bv;
            v.w += bv;
            if (a.relu) {
                v.x = relu_if(v.x, 1);
                v.y = relu_if(v.y, 1);
                v.z = relu_if(v.z, 1);
                v.w = relu_if(v.w, 1);
            }
            if constexpr (SP) {
                // Sub-pixel form: channel o is sub-pixel (du, dv) of dx channel c.
                const int ss = a.o_sh * a.o_sw;
                const int c = o / ss, rem = o - c * ss;
                const int du = rem / a.o_sw, dv = rem - du * a.o_sw;
                const size_t chd = (size_t)g * a.sp_cg + c;
                if (a.sp_vec) {
                    // dv = l16 & 1: the pair of lanes holds dx columns 2b..2b+7
                    // of one row; after the exchange the even lane has 2b..2b+3
                    // and the odd one 2b+4..2b+7, one 16-byte store each.
                    const float s0 = dv ? v.x : v.z, s1 = dv ? v.y : v.w;
                    const float r0 = swap_pair(s0), r1 = swap_pair(s1);
                    const f4 vs = dv ? f4{r0, v.z, r1, v.w} : f4{v.x, r0, v.y, r1};
                    if (qb < q1) {
                        const int n = (int)fastdiv((uint32_t)qb, a.div_P);
                        const int p = qb - n * a.P;
                        const int ho = (int)fastdiv((uint32_t)p, a.div_Wout);
                        const int wo = p - ho * a.Wout;
                        const int h = 2 * ho + du;
                        if (h < a.o_H)
                            *(f4*)(a.out + (((size_t)n * a.Cout_tot + chd) * a.o_H + h) * a.o_W + 2 * wo +
                                   4 * dv) = vs;
                    }
                } else {
                    const float vv[4] = {v.x, v.y, v.z, v.w};
                    const size_t Preal = (size_t)a.o_H * a.o_W;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int qq = qb + u;
                        if (qq < q1) {
                            const int n = (int)fastdiv((uint32_t)qq, a.div_P);
                            const int p = qq - n * a.P;
                            const int ho = (int)fastdiv((uint32_t)p, a.div_Wout);
                            const int wo = p - ho * a.Wout;
                            const int h = ho * a.o_sh + du, w = wo * a.o_sw + dv;
                            if (h < a.o_H && w < a.o_W) {
                                const size_t pr = (size_t)h * a.o_W + w;
                                if (a.out_nhwc) a.out[((size_t)n * Preal + pr) * a.Cout_tot + chd] = vv[u];
                                else a.out[((size_t)n * a.Cout_tot + chd) * Preal + pr] = vv[u];
                            }
                        }
                    }
                }
            } else if (a.out_nhwc) {
                // Channels-last output: for each pixel the 16 lanes of a lane
                // group write 16 consecutive channels (64 bytes).
                const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int qq = qb + u;
                    if (qq < q1) a.out[(size_t)qq * a.Cout_tot + ch_off] = vv[u];
                }
            } else if (vec4) {
                // P % 4 == 0 and q0 % 16 == 0: the four pixels share an image.
                if (qb < q1) {
                    const int n = (int)fastdiv((uint32_t)qb, a.div_P);
                    const int p = qb - n * a.P;
                    *(f4*)(a.out + ((size_t)n * a.Cout_tot + ch_off) * a.P + p) = v;
                }
            } else {
                const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int qq = qb + u;
                    if (qq < q1) {
                        const int n = (int)fastdiv((uint32_t)qq, a.div_P);
                        const int p = qq - n * a.P;
                        a.out[((size_t)n * a.Cout_tot + ch_off) * a.P + p] = vv[u];
                    }
                }
            }
        }
    }
}

// ---- host side ------------------------------------------------------------

constexpr int kMP = 4;
constexpr int kBP = 64 * kMP;

int bop_of(int BO) { return (BO % 64 == 16) ? BO : ((BO + 47) / 64) * 64 + 16; }

struct Geometry {
    int LW, LR, plane, xpf_needed;
};

Geometry tile_geometry(int Hout, int Wout, int sh, int sw, int dh, int dw, int kh, int kw, int CC)
{
    Geometry g;
    g.LW = (Wout - 1) * sw + (kw - 1) * dw + 1;
    const int rows_out = std::min(Hout, (kBP - 1) / Wout + 2);
    g.LR = (rows_out - 1) * sh + (kh - 1) * dh + 1;
    int plane = g.LR * g.LW;
    plane = ((plane + 47) / 64) * 64 + 16;  // == 16 (mod 64): the 4 lane groups hit distinct banks
    g.plane = plane;
    g.xpf_needed = (CC * g.LR * g.LW + 255) / 256;
    return g;
}

template <int KH, int KW, int MO, int CC, int XPF, bool FLIP>
void launch(const ConvMfmaArgs& a, int blocks, size_t lds, hipStream_t st)
{
    hipLaunchKernelGGL((conv_mfma_kernel<KH, KW, kMP, MO, CC, XPF, FLIP>), dim3(blocks), dim3(256),
                       lds, st, a);
}

template <int KH, int KW, int CC, bool FLIP>
bool dispatch_mo_xpf(int MO, int xpf, const ConvMfmaArgs& a, int blocks, size_t lds,
                     hipStream_t st)
{
#define GCONV_CASE(mo, x)                                             \
    if (MO == mo && xpf <= x) {                                       \
        launch<KH, KW, mo, CC, x, FLIP>(a, blocks, lds, st);          \
        return true;                                                  \
    }
    if constexpr (KH * KW <= 9) {
        GCONV_CASE(4, 16) GCONV_CASE(3, 16) GCONV_CASE(3, 24)
        GCONV_CASE(2, 16) GCONV_CASE(2, 24) GCONV_CASE(1, 16) GCONV_CASE(1, 24)
    } else {
        GCONV_CASE(2, 16) GCONV_CASE(1, 16) GCONV_CASE(1, 24)
    }
#undef GCONV_CASE
    return false;
}

// Problem in "forward" terms: input planes `in`, output planes `out`.
struct Problem {
    const float *in, *wgt, *bias;
    float* out;
    int N, G, Cin_tot, Cin_g, Hin, Win, Cout_tot, Cout_g, Hout, Wout;
    int kh, kw, sh, sw, dh, dw, ph, pw;
    int w_so, w_sr, w_gstride;
    bool flip;
    int uh = 1, uw = 1, Hr = 0, Wr = 0;  // input upsampling (flat kernel only), stored plane size
    int relu = 0;                        // forward epilogue
    int out_nhwc = 0;                    // channels-last output (flat kernel only)
    int in_nhwc = 0;                     // channels-last input (flat kernel only; Cin_g % 4 == 0)
    int pk_o = 0, pk_r = 0, w_gs = 0;    // packed groups (flat kernel only)
    // Sub-pixel form of a strided gradInput (flat kernel only): dx's stride,
    // extent and the mapping of super-taps to stored taps (the kernel
    // arguments of the same names).
    bool sp = false;
    int o_sh = 1, o_sw = 1, o_H = 0, o_W = 0;
    int sp_cg = 0, sp_bh = 0, sp_rh = 0, sp_bw = 0, sp_rw = 0, sp_mh = 0, sp_mw = 0, sp_kh = 0, sp_kw = 0;
};

// Groups with fewer than 16 output channels leave most of each 16-wide MFMA
// fragment idle, and a workgroup then reuses its input tile (whose per-lane
// DMA offsets cost it a fixed prologue) for only Cin_g / 4 chunks. Packing P
// consecutive groups into one launch group with a block-diagonal filter fills
// the fragment (the products across groups are with zero weights: the same
// MFMA count per output as the idle lanes had) and gives each workgroup P
// times the chunks. Channels of consecutive groups are contiguous, so the
// packed group is a plain group of P*Cin_g inputs and P*Cout_g outputs.
Problem pack_groups(Problem p)
{
    if (p.sp) return p;  // its output channels are already sub-pixels of a group's channels
    int P = 1;
    while (p.Cout_g * P * 2 <= 16 && p.G % (P * 2) == 0) P *= 2;
    if (P == 1) return p;
    p.pk_o = p.Cout_g;
    p.pk_r = p.Cin_g;
    p.w_gs = p.w_gstride;
    p.G /= P;
    p.Cout_g *= P;
    p.Cin_g *= P;
    p.w_gstride *= P;
    return p;
}

int choose_cc(const Problem& p) { return (p.kh * p.kw >= 16) ? 4 : 8; }

// Output-channel fragments per wave: as many as the group has (up to 4), but
// at most 2 for 25-tap filters, whose weight staging needs more registers.
int choose_mo(const Problem& p)
{
    const int cap = p.kh * p.kw <= 9 ? 4 : 2;
    return std::min(cap, (p.Cout_g + 15) / 16);
}

// The (MO, prefetch depth) instances compiled below.
bool instance_exists(int T, int MO, int xpf)
{
    if (T <= 9) return (MO == 4 && xpf <= 16) || (MO <= 3 && xpf <= 24);
    return (MO == 2 && xpf <= 16) || (MO == 1 && xpf <= 24);
}

bool problem_supported(const Problem& p)
{
    const bool k3 = p.kh == 3 && p.kw == 3, k5 = p.kh == 5 && p.kw == 5;
    if (!k3 && !k5) return false;
    if (p.Cout_g < 1 || p.Cin_g < 1) return false;
    const int CC = choose_cc(p);
    const Geometry geo = tile_geometry(p.Hout, p.Wout, p.sh, p.sw, p.dh, p.dw, p.kh, p.kw, CC);
    if (geo.xpf_needed > 24) return false;
    const int MO = choose_mo(p);
    if (!instance_exists(p.kh * p.kw, MO, geo.xpf_needed)) return false;
    const size_t lds =
        ((size_t)CC * geo.plane + (size_t)p.kh * p.kw * CC * bop_of(16 * MO) + 1) * 4;
    if (lds > 64 * 1024) return false;
    // Buffer resources address each group's input planes and weights in bytes below 2^31.
    // (the CC channels a chunk may read past the group end included)
    if ((int64_t)(p.Cin_g + CC) * p.Hin * p.Win * 4 >= (int64_t(1) << 31)) return false;
    if ((int64_t)p.w_gstride * 4 >= (int64_t(1) << 31)) return false;
    // Per-image extents stay far below 2^31 (FastDiv and 32-bit pixel indices).
    if ((int64_t)p.Hout * p.Wout >= (1 << 30) || (int64_t)CC * geo.LR * geo.LW >= (1 << 30))
        return false;
    return true;
}

bool run_problem(const Problem& p, hipStream_t st)
{
    const int CC = choose_cc(p);
    const Geometry geo = tile_geometry(p.Hout, p.Wout, p.sh, p.sw, p.dh, p.dw, p.kh, p.kw, CC);
    const int MO = choose_mo(p);
    const int BO = 16 * MO;
    ConvMfmaArgs a;
    a.in = p.in; a.wgt = p.wgt; a.bias = p.bias; a.out = p.out;
    a.relu = p.relu;
    a.N = p.N; a.G = p.G;
    a.Cin_tot = p.Cin_tot; a.Cin_g = p.Cin_g; a.Hin = p.Hin; a.Win = p.Win;
    a.Cout_tot = p.Cout_tot; a.Cout_g = p.Cout_g; a.Hout = p.Hout; a.Wout = p.Wout;
    a.sh = p.sh; a.sw = p.sw; a.dh = p.dh; a.dw = p.dw; a.ph = p.ph; a.pw = p.pw;
    a.w_so = p.w_so; a.w_sr = p.w_sr; a.w_gstride = p.w_gstride;
    a.tiles_per_image = (p.Hout * p.Wout + kBP - 1) / kBP;
    a.n_otiles = (p.Cout_g + BO - 1) / BO;
    a.LW = geo.LW; a.LR = geo.LR; a.plane = geo.plane;
    a.div_RW = make_fastdiv((uint32_t)(geo.LR * geo.LW));
    a.div_LW = make_fastdiv((uint32_t)geo.LW);
    a.div_Wout = make_fastdiv((uint32_t)p.Wout);
    const int64_t blocks64 = (int64_t)p.N * p.G * a.tiles_per_image * a.n_otiles;
    const int blocks = (int)blocks64;
    const size_t lds = ((size_t)CC * geo.plane + (size_t)p.kh * p.kw * CC * bop_of(BO) + 1) * 4;
    bool ok = false;
    if (p.kh == 3 && CC == 8 && !p.flip) ok = dispatch_mo_xpf<3, 3, 8, false>(MO, geo.xpf_needed, a, blocks, lds, st);
    else if (p.kh == 3 && CC == 8 && p.flip) ok = dispatch_mo_xpf<3, 3, 8, true>(MO, geo.xpf_needed, a, blocks, lds, st);
    else if (p.kh == 5 && CC == 4 && !p.flip) ok = dispatch_mo_xpf<5, 5, 4, false>(MO, geo.xpf_needed, a, blocks, lds, st);
    else if (p.kh == 5 && CC == 4 && p.flip) ok = dispatch_mo_xpf<5, 5, 4, true>(MO, geo.xpf_needed, a, blocks, lds, st);
    return ok;
}

Problem fwd_problem(const Shape& s, const float* x, const float* w, const float* bias, float* y)
{
    Problem p;
    p.in = x; p.wgt = w; p.bias = bias; p.out = y;
    p.N = s.N; p.G = s.G;
    p.Cin_tot = s.C; p.Cin_g = s.Cg; p.Hin = s.H; p.Win = s.W;
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

// gradInput: a forward correlation of dy with the transposed, tap-reversed
// filter and padding (k-1)*d - p, whose output extent is H x W. At stride s,
// dy is read as if upsampled by s (its values at multiples of s, zeros
// between): the adjoint of a strided correlation is the unit-stride
// correlation of the upsampled dy with the reversed filter.
Problem bwd_data_problem(const Shape& s, const float* dy, const float* w, float* dx)
{
    Problem p;
    p.in = dy; p.wgt = w; p.bias = nullptr; p.out = dx;
    p.N = s.N; p.G = s.G;
    p.Cin_tot = s.K; p.Cin_g = s.Kg;
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

// ---- flattened-pixel variant: host side --------------------------------------

struct FlatInst {
    int T, MO, WO, WPX, MP, NSX;
    int KH, KW;
    bool SP;  // the sub-pixel form of a strided gradInput (super-taps, depth-to-space output)
};
#ifndef GCONV_FLAT_MP3
#define GCONV_FLAT_MP3 5
#endif
// Compiled instances: output fragments per wave (MO), waves across output
// channels (WO) and across pixels (WPX), pixel fragments per wave (MP). With
// 64 channels per group, 5 fragments give 1255 tiles of 80 pixels for 32
// images of 56 x 56, which spread evenly over the 256 CUs.
// NSX: DMA segments (of 64 floats) per wave and buffer, at most (one
// register each). The plan takes the first instance of its shape whose tile
// fits: the larger-NSX copies serve strided layers, whose tiles span twice
// the input rows, and wide images; the 12-segment three-wave 5x5 copy takes
// AlexNet conv2's gradInput (48 channels per group, 27 x 27 planes: nine
// segments), which otherwise fell back to the per-image kernel (711 -> 667 us).
#define GCONV_FLAT_INSTS(X)                                                                \
    X(9, 3, 1, 4, 1, GCONV_FLAT_MP3, 8) X(9, 3, 2, 4, 1, 4, 12) X(9, 3, 1, 3, 1, 5, 8)     \
    X(9, 3, 1, 2, 2, 4, 8) X(9, 3, 1, 1, 4, 4, 12)                                         \
    X(25, 5, 1, 4, 1, 4, 8) X(25, 5, 2, 4, 1, 4, 8) X(25, 5, 1, 3, 1, 4, 8)                \
    X(25, 5, 1, 2, 2, 4, 8) X(25, 5, 1, 1, 4, 4, 12)                                       \
    X(9, 3, 2, 4, 1, 4, 16) X(9, 3, 1, 1, 4, 4, 24) X(25, 5, 1, 3, 1, 4, 12)
// Sub-pixel instances (never flipped): super-filters of 1x1 (2x2 filters at
// stride 2), 2x2 (3x3 at stride 2 or 3) and 3x3 (4x4 and 5x5 at stride 2),
// over the same wave layouts.
#define GCONV_SP_SHAPES(X, mo, wo, wpx, mp, nsx) \
    X(1, mo, wo, wpx, mp, nsx) X(2, mo, wo, wpx, mp, nsx) X(3, mo, wo, wpx, mp, nsx)
#define GCONV_SP_INSTS(X)                                                     \
    GCONV_SP_SHAPES(X, 1, 1, 4, 4, 12) GCONV_SP_SHAPES(X, 1, 2, 2, 4, 8)       \
    GCONV_SP_SHAPES(X, 1, 4, 1, 5, 8) GCONV_SP_SHAPES(X, 2, 4, 1, 4, 12) GCONV_SP_SHAPES(X, 2, 1, 4, 4, 12)
#define GCONV_FLAT_ENTRY(t, k, mo, wo, wpx, mp, nsx) {t, mo, wo, wpx, mp, nsx, k, k, false},
#define GCONV_SP_ENTRY(k, mo, wo, wpx, mp, nsx) {k * k, mo, wo, wpx, mp, nsx, k, k, true},
constexpr FlatInst kFlatInsts[] = {GCONV_FLAT_INSTS(GCONV_FLAT_ENTRY) GCONV_SP_INSTS(GCONV_SP_ENTRY)};
#undef GCONV_FLAT_ENTRY
#undef GCONV_SP_ENTRY

struct FlatPlan {
    FlatInst inst;
    int LW, plane, nseg, bufsz;
    size_t lds_bytes;
    int blocks;
};

bool flat_plan(const Problem& p_in, FlatPlan& fp)
{
    const Problem p = pack_groups(p_in);
    if (p.sp) {
        if (!(p.kh == p.kw && p.kh >= 1 && p.kh <= 3 && !p.flip)) return false;
    } else if (!((p.kh == 3 && p.kw == 3) || (p.kh == 5 && p.kw == 5))) {
        return false;
    }
    const int nfrag = (p.Cout_g + 15) / 16;
    const int mo0 = nfrag > 4 ? 2 : 1;
    // waves across output channels (sub-pixel instances: 1, 2 or 4)
    const int wo0 = nfrag > 4 ? 4 : (p.sp && nfrag == 3) ? 4 : nfrag;
    // Sub-pixel form with two fragments (8 channels per group at stride 2):
    // one wave takes both over 256 pixels where the images hold that many,
    // so each workgroup's set-up (DMA offsets, tap map, store addresses)
    // serves twice the MFMAs; else the two-wave layout.
    const bool wide = p.sp && nfrag == 2;
    const FlatInst* inst = nullptr;
    int64_t plane = 0, nseg = 0, LW = 0, P = (int64_t)p.Hout * p.Wout;
    for (int pass = wide ? 0 : 1; pass < 2 && !inst; ++pass)
    for (const FlatInst& fi : kFlatInsts) {
        const int mo = pass == 0 ? 2 : mo0, wo = pass == 0 ? 1 : wo0;
        if (!(fi.KH == p.kh && fi.KW == p.kw && fi.SP == p.sp && fi.MO == mo && fi.WO == wo))
            continue;
        const int NWi = fi.WO * fi.WPX;
        const int BPXi = fi.WPX * fi.MP * 16;
        if (P < BPXi) continue;  // a tile must span at most two images
        const int halo = (p.kh - 1) * p.dh + 1;
        // Output rows a tile's BPXi consecutive pixels touch: at most `span`
        // in all, at most Hout of them in one image. A tile that crosses into
        // the next image stages both images' rows, each part with its own
        // halo, and its parts together may hold more rows than one image has.
        const int64_t span = (BPXi - 1) / p.Wout + 2;
        const int R1 = (int)std::min<int64_t>(p.Hout, span);      // within one image
        const int R2 = (int)std::min<int64_t>(2 * (int64_t)p.Hout, span);  // across two
        const int LR = std::max((R1 - 1) * p.sh + halo, (R2 - 2) * p.sh + 2 * halo);
        LW = (int64_t)(p.Wout - 1) * p.sw + (p.kw - 1) * p.dw + 1;
        plane = LR * LW;
        // == 16 (mod 64): the 4 lane groups hit distinct banks. At column
        // stride 2 a fragment's 16 pixels read every other float (16 even
        // banks), so an odd plane puts the other channel lane of each
        // half-wave on the odd banks.
        plane = p.sw == 2 && !p.in_nhwc ? ((plane + 63) / 64) * 64 + 1 : ((plane + 47) / 64) * 64 + 16;
        // channels-last input: one 16-byte DMA lane per pixel of the LR x LW tile
        nseg = p.in_nhwc ? (LR * LW + 64 * NWi - 1) / (64 * NWi) : (4 * plane + 64 * NWi - 1) / (64 * NWi);
        // (16 bytes a lane in the channels-last form, so its double buffer must
        // also fit the CU's 160 KiB of LDS)
        if (nseg <= fi.NSX && (!p.in_nhwc || 2 * nseg * 64 * NWi * 16 <= 160 * 1024)) {
            inst = &fi;
            break;
        }
    }
    if (!inst) return false;
    fp.inst = *inst;
    const int NW = inst->WO * inst->WPX;
    const int BPX = inst->WPX * inst->MP * 16;
    const int64_t NP = (int64_t)p.N * P;
    if (NP + BPX >= (int64_t(1) << 31)) return false;
    fp.LW = (int)LW;
    fp.plane = (int)plane;
    fp.nseg = (int)nseg;
    fp.bufsz = (int)(nseg * 64 * NW * (p.in_nhwc ? 4 : 1));
    fp.lds_bytes = (size_t)2 * fp.bufsz * 4;
    // Buffer resources: two images' worth of one group's planes, and one
    // group's weights, addressed in bytes below 2^31.
    if ((int64_t)(p.Cin_tot + p.Cin_g) * p.Hr * p.Wr * 4 >= (int64_t(1) << 31)) return false;
    if (p.in_nhwc && ((p.Cin_g & 3) != 0 || (p.Cin_tot & 3) != 0 ||
                      (int64_t)2 * p.Hr * p.Wr * p.Cin_tot * 4 >= (int64_t(1) << 31)))
        return false;
    if ((int64_t)p.w_gstride * 4 >= (int64_t(1) << 31)) return false;
    const int BO = inst->WO * inst->MO * 16;
    const int64_t blocks = ((NP + BPX - 1) / BPX) * p.G * ((p.Cout_g + BO - 1) / BO);
    if (blocks >= (int64_t(1) << 31)) return false;
    fp.blocks = (int)blocks;
    return true;
}

template <int KH, int KW, int MP, int MO, int WO, int WPX, int NSX, bool FLIP, bool INH, bool SP = false,
          bool PK = false>
void launch_flat(const ConvFlatArgs& a, const FlatPlan& fp, hipStream_t st)
{
    constexpr int MINW = (KH * KW <= 9) ? 4 : 2;
    auto kern = conv_flat_kernel<KH, KW, MP, MO, WO, WPX, NSX, FLIP, MINW, INH, SP, PK>;
    hipLaunchKernelGGL(kern, dim3(fp.blocks), dim3(64 * WO * WPX), fp.lds_bytes, st, a);
}

template <bool INH>
bool dispatch_sp(const ConvFlatArgs& a, const FlatPlan& fp, hipStream_t st)
{
    const FlatInst& i = fp.inst;
#define GCONV_SP_CASE(k, mo, wo, wpx, mp, nsx)                                                     \
    if (i.SP && i.KH == k && i.MO == mo && i.WO == wo && i.WPX == wpx && i.MP == mp && i.NSX == nsx) { \
        launch_flat<k, k, mp, mo, wo, wpx, nsx, false, INH, true>(a, fp, st);              \
        return true;                                                                             \
    }
    GCONV_SP_INSTS(GCONV_SP_CASE)
#undef GCONV_SP_CASE
    return false;
}

template <bool FLIP, bool INH>
bool dispatch_flat(const ConvFlatArgs& a, const FlatPlan& fp, hipStream_t st)
{
    const FlatInst& i = fp.inst;
#define GCONV_FLAT_CASE(t, k, mo, wo, wpx, mp, nsx)                                     \
    if (!i.SP && i.T == t && i.MO == mo && i.WO == wo && i.WPX == wpx && i.MP == mp && i.NSX == nsx) { \
        if (!a.pk_o) {                                                                 \
            launch_flat<k, k, mp, mo, wo, wpx, nsx, FLIP, INH>(a, fp, st);              \
            return true;                                                               \
        }                                                                              \
        if constexpr (mo == 1 && wo == 1) {                                            \
            launch_flat<k, k, mp, mo, wo, wpx, nsx, FLIP, INH, false, true>(a, fp, st); \
            return true;                                                               \
        }                                                                              \
        return false;                                                                  \
    }
    GCONV_FLAT_INSTS(GCONV_FLAT_CASE)
#undef GCONV_FLAT_CASE
    return false;
}

bool run_flat(const Problem& p_in, hipStream_t st)
{
    FlatPlan fp;
    if (!flat_plan(p_in, fp)) return false;
    const Problem p = pack_groups(p_in);
    ConvFlatArgs a;
    a.in = p.in; a.wgt = p.wgt; a.bias = p.bias; a.out = p.out;
    a.N = p.N; a.G = p.G;
    a.Cin_tot = p.Cin_tot; a.Cin_g = p.Cin_g; a.Hin = p.Hin; a.Win = p.Win;
    a.Cout_tot = p.Cout_tot; a.Cout_g = p.Cout_g; a.Hout = p.Hout; a.Wout = p.Wout;
    a.sh = p.sh; a.sw = p.sw; a.dh = p.dh; a.dw = p.dw; a.ph = p.ph; a.pw = p.pw;
    a.w_so = p.w_so; a.w_sr = p.w_sr; a.w_gstride = p.w_gstride;
    a.P = p.Hout * p.Wout;
    a.NP = p.N * a.P;
    const int BO = fp.inst.WO * fp.inst.MO * 16;
    a.n_otiles = (p.Cout_g + BO - 1) / BO;
    a.LW = fp.LW; a.plane = fp.plane; a.nseg = fp.nseg; a.bufsz = fp.bufsz;
    a.halo = (p.kh - 1) * p.dh + 1;
    a.uh = p.uh; a.uw = p.uw; a.Hr = p.Hr; a.Wr = p.Wr;
    a.relu = p.relu;
    a.out_nhwc = p.out_nhwc;
    a.div_P = make_fastdiv((uint32_t)a.P);
    a.div_Wout = make_fastdiv((uint32_t)p.Wout);
    a.div_plane = make_fastdiv((uint32_t)fp.plane);
    a.div_LW = make_fastdiv((uint32_t)fp.LW);
    a.pk_o = p.pk_o; a.pk_r = p.pk_r; a.w_gs = p.w_gs;
    a.o_sh = p.o_sh; a.o_sw = p.o_sw; a.o_H = p.o_H; a.o_W = p.o_W;
    a.sp_cg = p.sp_cg; a.sp_bh = p.sp_bh; a.sp_rh = p.sp_rh; a.sp_bw = p.sp_bw; a.sp_rw = p.sp_rw;
    a.sp_mh = p.sp_mh; a.sp_mw = p.sp_mw; a.sp_kh = p.sp_kh; a.sp_kw = p.sp_kw;
    a.sp_vec = p.sp && p.o_sh == 2 && p.o_sw == 2 && !p.out_nhwc && a.P % 4 == 0 && p.Wout % 4 == 0 &&
               p.o_W == 2 * p.Wout && ((uintptr_t)p.out & 15) == 0;
    if (p.sp) return p.in_nhwc ? dispatch_sp<true>(a, fp, st) : dispatch_sp<false>(a, fp, st);
    if (p.in_nhwc) return p.flip ? dispatch_flat<true, true>(a, fp, st) : dispatch_flat<false, true>(a, fp, st);
    return p.flip ? dispatch_flat<true, false>(a, fp, st) : dispatch_flat<false, false>(a, fp, st);
}

bool use_flat(const Problem& p)
{
#ifdef GCONV_NO_FLAT
    (void)p;
    return false;
#else
    FlatPlan fp;
    return flat_plan(p, fp);
#endif
}

// ---- strided gradInput in sub-pixel form -----------------------------------------
//
// dx[h][w] sums w[k][c][i][j] * dy[k][(h + ph - i)/sh][(w + pw - j)/sw] over
// the taps whose quotients are exact. With h + ph = sh*A + u (0 <= u < sh, the
// row's phase) only the taps i = u + sh*i' qualify, and tap i reads dy row
// A - i'; columns alike. Group the dx pixels into blocks of sh x sw, block
// (a, b) holding pixels (a*sh + du, b*sw + dv): the pixel at du has
// A = a + (du + ph) div sh, so every pixel of the block reads dy rows a + d
// for offsets d within a small spread E. The block is thus a unit-stride
// correlation of the stored dy with an E x E super-filter and Cg*sh*sw output
// channels, one per (channel, sub-pixel), whose super-taps that match no
// stored tap are zero. One launch covers every phase over a shared dy tile and
// stores whole dx rows. The zero taps cost MFMA work (16 super-taps for the 9
// real ones of a 3x3 filter at stride 2); against one launch per phase (exact
// taps, but every other dx column written per launch, which doubles the HBM
// writes, and four launches with a quarter of the pixels each) it was faster
// on every layer measured: 254 -> 102 us for 256 channels in groups of 8 at
// 56 x 56, 204 -> 152 us for 128 dense channels, 347 -> 185 us for 512 -> 256
// channels at 28 x 28.

// Least dy offset and spread of a dimension's super-taps: the sub-pixel at
// du has phase u = (du + p) mod s, whose taps i = u + s*i' (i < k) read dy at
// offset (du + p) div s - i'.
void sp_extent(int k, int st, int pad, int* dmin, int* ext)
{
    const int b = pad / st, r = pad % st;
    int lo = 1 << 30, hi = -(1 << 30);
    for (int du = 0; du < st; ++du) {
        const bool c = du + r >= st;
        const int A = b + c, u = du + r - (c ? st : 0);
        if (u >= k) continue;  // no tap: the sub-pixel's dx values are 0
        const int Ti = (k - u + st - 1) / st;
        lo = std::min(lo, A - (Ti - 1));
        hi = std::max(hi, A);
    }
    *dmin = lo;
    *ext = hi - lo + 1;
}

bool sp_problem(const Shape& s, const float* dy, const float* w, float* dx, Problem* out)
{
    if (!(s.sh > 1 || s.sw > 1) || s.dh != 1 || s.dw != 1 || s.ph < 0 || s.pw < 0) return false;
    int mh, eh, mw, ew;
    sp_extent(s.kh, s.sh, s.ph, &mh, &eh);
    sp_extent(s.kw, s.sw, s.pw, &mw, &ew);
    const int E = std::max(eh, ew);  // the shorter dimension's extra taps match no stored tap
    if (E > 3 || s.sh * s.sw > 16) return false;
    const int T = s.kh * s.kw;
    Problem p;
    p.in = dy; p.wgt = w; p.bias = nullptr; p.out = dx;
    p.N = s.N; p.G = s.G;
    p.Cin_tot = s.K; p.Cin_g = s.Kg; p.Hin = s.Ho; p.Win = s.Wo; p.Hr = s.Ho; p.Wr = s.Wo;
    p.Cout_tot = s.C; p.Cout_g = s.Cg * s.sh * s.sw;
    p.Hout = (s.H + s.sh - 1) / s.sh; p.Wout = (s.W + s.sw - 1) / s.sw;
    p.kh = E; p.kw = E; p.sh = 1; p.sw = 1; p.dh = 1; p.dw = 1;
    p.ph = -mh; p.pw = -mw;
    p.w_so = T; p.w_sr = s.Cg * T; p.w_gstride = s.Kg * s.Cg * T;
    p.flip = false;
    p.sp = true;
    p.sp_cg = s.Cg;
    p.sp_bh = s.ph / s.sh; p.sp_rh = s.ph % s.sh; p.sp_bw = s.pw / s.sw; p.sp_rw = s.pw % s.sw;
    p.sp_mh = mh; p.sp_mw = mw; p.sp_kh = s.kh; p.sp_kw = s.kw;
    p.o_sh = s.sh; p.o_sw = s.sw; p.o_H = s.H; p.o_W = s.W;
    if (!use_flat(p)) return false;
    *out = p;
    return true;
}

bool sp_ok(const Shape& s, bool in_nhwc)
{
#ifdef GCONV_NO_SUBPIXEL
    (void)s; (void)in_nhwc;
    return false;
#else
    Problem p;
    if (!sp_problem(s, nullptr, nullptr, nullptr, &p)) return false;
    p.in_nhwc = in_nhwc;
    return use_flat(p);
#endif
}

bool run_sp(const Shape& s, const float* dy, const float* w, float* dx, bool in_nhwc, bool out_nhwc,
            hipStream_t st)
{
    Problem p;
    if (!sp_problem(s, dy, w, dx, &p)) return false;
    p.in_nhwc = in_nhwc;
    p.out_nhwc = out_nhwc;
    return run_flat(p, st);
}

}  // namespace

bool igemm_fwd_supported(const Shape& s)
{
    const Problem p = fwd_problem(s, nullptr, nullptr, nullptr, nullptr);
    return use_flat(p) || problem_supported(p);
}

bool igemm_bwd_data_subpixel_ok(const Shape& s) { return sp_ok(s, false); }

bool igemm_bwd_data_supported(const Shape& s)
{
    if (sp_ok(s, false)) return true;
    const Problem p = bwd_data_problem(s, nullptr, nullptr, nullptr);
    if (p.uh != 1 || p.uw != 1) return use_flat(p);  // only the flat kernel upsamples
    return use_flat(p) || problem_supported(p);
}

bool igemm_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y,
               hipStream_t st)
{
    const Problem p = fwd_problem(s, x, w, bias, y);
    return use_flat(p) ? run_flat(p, st) : run_problem(p, st);
}

bool igemm_bwd_data(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st)
{
    if (sp_ok(s, false)) return run_sp(s, dy, w, dx, false, false, st);
    const Problem p = bwd_data_problem(s, dy, w, dx);
    if (use_flat(p)) return run_flat(p, st);
    if (p.uh != 1 || p.uw != 1) return false;
    return run_problem(p, st);
}

// The flat kernel stores its output channels-last: the NCHW-input ops of the
// NHWC layout write y or dx in place, with no reordering after them. False
// (nothing launched) where the flat kernel does not take the shape.
bool igemm_nhwc_out_supported(const Shape& s, int op)
{
    if (op == GCONV_OP_FWD) return use_flat(fwd_problem(s, nullptr, nullptr, nullptr, nullptr));
    if (op == GCONV_OP_BWD_DATA)
        return sp_ok(s, false) || use_flat(bwd_data_problem(s, nullptr, nullptr, nullptr));
    return false;
}

bool igemm_fwd_nhwc_out(const Shape& s, const float* x, const float* w, const float* bias, float* y,
                        hipStream_t st)
{
    Problem p = fwd_problem(s, x, w, bias, y);
    if (!use_flat(p)) return false;
    p.out_nhwc = 1;
    return run_flat(p, st);
}

bool igemm_bwd_data_nhwc_out(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st)
{
    if (sp_ok(s, false)) return run_sp(s, dy, w, dx, false, true, st);
    Problem p = bwd_data_problem(s, dy, w, dx);
    if (!use_flat(p)) return false;
    p.out_nhwc = 1;
    return run_flat(p, st);
}

// Channels-last in and out: the flat kernel's loader reads NHWC pixels with
// 16-byte DMA (4 channels per pixel) where the group's channels come in whole
// quads; no reordering at all.
static Problem nhwc_io(Problem p)
{
    p.in_nhwc = 1;
    p.out_nhwc = 1;
    return p;
}

bool igemm_nhwc_io_supported(const Shape& s, int op)
{
    if (op == GCONV_OP_FWD) return use_flat(nhwc_io(fwd_problem(s, nullptr, nullptr, nullptr, nullptr)));
    if (op == GCONV_OP_BWD_DATA)
        return sp_ok(s, true) || use_flat(nhwc_io(bwd_data_problem(s, nullptr, nullptr, nullptr)));
    return false;
}

bool igemm_fwd_nhwc_io(const Shape& s, const float* x, const float* w, const float* bias, float* y, hipStream_t st)
{
    const Problem p = nhwc_io(fwd_problem(s, x, w, bias, y));
    return use_flat(p) && run_flat(p, st);
}

bool igemm_bwd_data_nhwc_io(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st)
{
    if (sp_ok(s, true)) return run_sp(s, dy, w, dx, true, true, st);
    const Problem p = nhwc_io(bwd_data_problem(s, dy, w, dx));
    return use_flat(p) && run_flat(p, st);
}

}  // namespace gconv
