// wgrad_mfma.hip -- fp32-MFMA gradWeight for grouped 2-D convolution, NCHW.
//
//   dw[g*Kg + k, c, i, j] = sum_{n, ho, wo} dy[n, g*Kg + k, ho, wo]
//                               * x[n, g*Cg + c, ho*sh - ph + i*dh, wo*sw - pw + j*dw]
//
// For every tap (i, j) this is a GEMM over output pixels: rows = the Cg input
// channels, columns = the Kg output channels, reduction = N*Ho*Wo pixels.
// Each wave keeps one 16x16 accumulator per tap and per output-channel
// fragment, so an input value read once from LDS feeds all taps' MFMAs.
//
//   v_mfma_f32_16x16x4f32: A = 16 input channels x 4 pixels (x at the tap's
//   shifted position), B = 4 pixels x 16 output channels (dy), D: lane l holds
//   dw[c = 4*(l/16)+v][k = l%16].
//
// The pixel reduction is split: the N*Ho output rows are cut into chunks of R
// rows of one image, and each block reduces a contiguous run of chunks for one
// (group, input-channel tile, output-channel tile). Blocks write partial tiles
// to the workspace in the accumulator's own order; a second kernel sums the
// splits in a fixed order and scatters into dw, so results are deterministic
// (no atomics). Tiles are staged global -> LDS directly (buffer loads with an
// LDS destination; out-of-range offsets write 0, which is the zero padding),
// double-buffered so the next chunk streams in while this one is multiplied.
#include <algorithm>

#include "fastdiv.h"
#include "gconv_internal.h"

namespace gconv {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// 64 lanes load one dword each into 64 consecutive LDS floats at `dst`.
__device__ __forceinline__ void load_lds64(__amdgpu_buffer_rsrc_t r, float* dst, uint32_t byte_off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, byte_off, 0, 0, 0);
}

__device__ __forceinline__ int xcd_remap(int b, int nb)
{
    const int per = nb >> 3, rem = nb & 7, x = b & 7, i = b >> 3;
    return x * per + min(x, rem) + i;
}

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

template <int KH, int KW, int WC, int WK, int R>
__global__ void __launch_bounds__(256, 2) wgrad_mfma_kernel(WgradArgs a)
{
    constexpr int T = KH * KW;
    constexpr int CT = 16 * WC;
    constexpr int KT = 16 * WK * (4 / WC);

    extern __shared__ float lds[];
    const int buf_floats = CT * a.XS + KT * a.DS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int l16 = lane & 15, q = lane >> 4;
    const int wc = wave % WC, wk = wave / WC;

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

    // Issue the loads of chunk `ch` into LDS buffer `b` (all four waves share the work).
    auto issue = [&](int ch, int b) {
        float* xs = lds + b * buf_floats;
        float* ds = xs + CT * a.XS;
        const int n = (int)fastdiv((uint32_t)ch, a.div_cpi);
        const int ho0 = (ch - n * a.chunks_per_image) * R;
        const float* xg = a.x + ((size_t)n * a.C + (size_t)g * a.Cg + c0) * a.H * a.W;
        const float* dyg = a.dy + ((size_t)n * a.K + (size_t)g * a.Kg + k0) * a.Ho * a.Wo;
        // Channels past the group end fall outside these resources and read 0.
        const __amdgpu_buffer_rsrc_t rx =
            make_rsrc(xg, (uint32_t)max(0, min(CT, a.Cg - c0)) * a.H * a.W * 4u);
        const __amdgpu_buffer_rsrc_t rd =
            make_rsrc(dyg, (uint32_t)max(0, min(KT, a.Kg - k0)) * a.Ho * a.Wo * 4u);
        const int hb = ho0 * a.sh - a.ph;
        const int xlen = a.LR * a.LW;
        for (int i = wave; i < CT * a.nsx; i += 4) {
            const int c = i / a.nsx, sg = i - c * a.nsx;
            const int e = sg * 64 + lane;
            const int r = (int)fastdiv((uint32_t)e, a.div_LW);
            const int col = e - r * a.LW;
            const int h = hb + r, w = col - a.pw;
            const bool ok = e < xlen && (unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W;
            load_lds64(rx, xs + c * a.XS + sg * 64,
                       ok ? (uint32_t)((c * a.H + h) * a.W + w) * 4u : kOOB);
        }
        const int dlen = R * a.WoP;
        for (int i = wave; i < KT * a.nsd; i += 4) {
            const int k = i / a.nsd, sg = i - k * a.nsd;
            const int e = sg * 64 + lane;
            const int r = (int)fastdiv((uint32_t)e, a.div_WoP);
            const int col = e - r * a.WoP;
            const int ho = ho0 + r;
            const bool ok = e < dlen && ho < a.Ho && col < a.Wo;
            load_lds64(rd, ds + k * a.DS + sg * 64,
                       ok ? (uint32_t)((k * a.Ho + ho) * a.Wo + col) * 4u : kOOB);
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
        const int rows = min(R, a.Ho - ho0);
        const float* xl = xs + (wc * 16 + l16) * a.XS + q * a.sw;
        const float* dl = ds + (wk * 16 * WK + l16) * a.DS + q;
        for (int r = 0; r < rows; ++r) {
            const float* xr = xl + r * a.sh * a.LW;
            const float* dr = dl + r * a.WoP;
            for (int st = 0; st < nsteps; ++st) {
                const int xo = st * 4 * a.sw;
                float av[T], bv[WK];
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int i = t / KW, j = t % KW;
                    av[t] = xr[xo + i * a.dh * a.LW + j * a.dw];
                }
#pragma unroll
                for (int m = 0; m < WK; ++m) bv[m] = dr[m * 16 * a.DS + st * 4];
#pragma unroll
                for (int t = 0; t < T; ++t)
#pragma unroll
                    for (int m = 0; m < WK; ++m)
                        acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t], bv[m], acc[t][m],
                                                                         0, 0, 0);
            }
        }
        __syncthreads();  // every wave is done with buffer b before it is refilled
    }

    // Partial tile in accumulator order: [split][tile][wave][t][m][v][lane].
    const int tile = (g * a.n_ctiles + ct) * a.n_ktiles + kt;
    const int n_tiles = a.G * a.n_ctiles * a.n_ktiles;
    float* out = a.ws + (((size_t)s * n_tiles + tile) * 4 + wave) * (size_t)(T * WK * 256);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < WK; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) out[(t * WK + m) * 256 + v * 64 + lane] = acc[t][m][v];
}

// dw from the partial tiles: sum over splits in index order, then scatter.
template <int T, int WC, int WK>
__global__ void __launch_bounds__(256) wgrad_reduce_kernel(const float* __restrict__ ws,
                                                           float* __restrict__ dw, int splits,
                                                           int n_ctiles, int n_ktiles, int Cg,
                                                           int Kg, int per_split)
{
    constexpr int CT = 16 * WC;
    constexpr int KT = 16 * WK * (4 / WC);
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= per_split) return;
    float sum = 0.f;
    for (int s = 0; s < splits; ++s) sum += ws[(size_t)s * per_split + j];
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
    int WC, WK, R;
};

Config choose_config(const Shape& s)
{
    // One 16-channel input tile per wave column; four waves along output
    // channels. Rows per chunk keep a step loop of >= ~10 quads.
    Config c;
    c.WC = 1;
    c.WK = 1;
    c.R = std::max(1, std::min(4, 64 / std::max(1, s.Wo)));
    if (c.R > s.Ho) c.R = s.Ho;
    return c;
}

struct Plan {
    bool ok;
    Config cfg;
    WgradArgs a;
    int blocks;
    size_t lds_bytes, ws_floats;
    int per_split;
};

int ceil64(int v) { return (v + 63) / 64 * 64; }

Plan make_plan(const Shape& s, int max_splits_override = 0)
{
    Plan p{};
    p.ok = false;
    const bool k3 = s.kh == 3 && s.kw == 3, k5 = s.kh == 5 && s.kw == 5;
    if (!k3 && !k5) return p;
    if (s.N < 1) return p;
    const Config cfg = choose_config(s);
    const int CT = 16 * cfg.WC, KT = 16 * cfg.WK * (4 / cfg.WC), R = cfg.R;
    const int T = s.kh * s.kw;
    WgradArgs& a = p.a;
    a.N = s.N; a.C = s.C; a.H = s.H; a.W = s.W; a.K = s.K; a.Ho = s.Ho; a.Wo = s.Wo;
    a.G = s.G; a.Cg = s.Cg; a.Kg = s.Kg;
    a.sh = s.sh; a.sw = s.sw; a.dh = s.dh; a.dw = s.dw; a.ph = s.ph; a.pw = s.pw;
    a.n_ctiles = (s.Cg + CT - 1) / CT;
    a.n_ktiles = (s.Kg + KT - 1) / KT;
    a.chunks_per_image = (s.Ho + R - 1) / R;
    const int64_t chunks_total = (int64_t)s.N * a.chunks_per_image;
    if (chunks_total >= (1 << 30)) return p;
    a.chunks_total = (int)chunks_total;
    a.WoP = (s.Wo + 3) / 4 * 4;
    a.LW = (s.Wo - 1) * s.sw + (s.kw - 1) * s.dw + 1;
    a.LR = (R - 1) * s.sh + (s.kh - 1) * s.dh + 1;
    // The last quad of a row may reach up to 3 columns (times the stride)
    // past the row end: keep those reads inside the loaded (zero-filled) span.
    const int xspan = a.LR * a.LW + 4 * s.sw;
    a.nsx = (xspan + 63) / 64;
    a.XS = a.nsx * 64 + 4;  // == 4 (mod 64): the 4 pixel lanes of a channel hit distinct banks
    a.nsd = (R * a.WoP + 63) / 64;
    a.DS = a.nsd * 64 + 4;
    const size_t buf = (size_t)CT * a.XS + (size_t)KT * a.DS;
    p.lds_bytes = 2 * buf * 4;
    if (p.lds_bytes > 64 * 1024) return p;
    // Tiles are addressed with 32-bit byte offsets, including the channels a
    // tile may reach past the end of its group.
    if ((int64_t)(s.Cg + CT) * s.H * s.W * 4 >= (int64_t(1) << 31)) return p;
    if ((int64_t)(s.Kg + KT) * s.Ho * s.Wo * 4 >= (int64_t(1) << 31)) return p;
    const int n_tiles = s.G * a.n_ctiles * a.n_ktiles;
    // Splits: about two blocks per CU in total, at most one chunk run each.
    int splits = std::max(1, 512 / n_tiles);
    if (max_splits_override > 0) splits = max_splits_override;
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

template <int KH, int KW, int WC, int WK, int R>
void launch_main(const Plan& p, hipStream_t st)
{
    hipLaunchKernelGGL((wgrad_mfma_kernel<KH, KW, WC, WK, R>), dim3(p.blocks), dim3(256),
                       p.lds_bytes, st, p.a);
}

template <int KH, int KW>
bool launch_r(const Plan& p, hipStream_t st)
{
    switch (p.cfg.R) {
        case 1: launch_main<KH, KW, 1, 1, 1>(p, st); return true;
        case 2: launch_main<KH, KW, 1, 1, 2>(p, st); return true;
        case 3: launch_main<KH, KW, 1, 1, 3>(p, st); return true;
        case 4: launch_main<KH, KW, 1, 1, 4>(p, st); return true;
        default: return false;
    }
}

}  // namespace

bool igemm_bwd_filter_supported(const Shape& s) { return make_plan(s).ok; }

size_t igemm_bwd_filter_workspace(const Shape& s)
{
    const Plan p = make_plan(s);
    return p.ok ? p.ws_floats * sizeof(float) : 0;
}

bool igemm_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws,
                      hipStream_t st)
{
    Plan p = make_plan(s);
    if (!p.ok || p.cfg.WC != 1 || p.cfg.WK != 1) return false;
    p.a.x = x;
    p.a.dy = dy;
    p.a.ws = ws;
    bool ok = false;
    if (s.kh == 3) ok = launch_r<3, 3>(p, st);
    else if (s.kh == 5) ok = launch_r<5, 5>(p, st);
    if (!ok) return false;
    const int T = s.kh * s.kw;
    const int blocks = (p.per_split + 255) / 256;
    if (T == 9)
        hipLaunchKernelGGL((wgrad_reduce_kernel<9, 1, 1>), dim3(blocks), dim3(256), 0, st, ws, dw,
                           p.a.splits, p.a.n_ctiles, p.a.n_ktiles, s.Cg, s.Kg, p.per_split);
    else
        hipLaunchKernelGGL((wgrad_reduce_kernel<25, 1, 1>), dim3(blocks), dim3(256), 0, st, ws, dw,
                           p.a.splits, p.a.n_ctiles, p.a.n_ktiles, s.Cg, s.Kg, p.per_split);
    return true;
}

}  // namespace gconv
