// gemm_fc.hip -- fully-connected mode: a convolution whose kernel covers the
// whole unpadded input (kh == H, kw == W, no padding, so Ho = Wo = 1) is one
// dense layer on the flattened image ("SpatialConvolution running in
// fully-connected mode is very slow, even with R4": MatConvNet switches to a
// fully-connected layer there, and the View + Linear replacement gives the same
// result). With X = x.view(N, C*H*W) and Wm = w.view(K, C*kh*kw), per group:
//     forward     Y  = X  * Wm^T + b     (M = N, cols = K,   reduction = D)
//     gradInput   dX = dY * Wm           (M = N, cols = D,   reduction = K)
//     gradWeight  dW = dY^T * X          (M = K, cols = D,   reduction = N)
// All three run on one fp32-MFMA GEMM kernel, C[M x Nc] = A[M x R] * B[R x Nc],
// templated on which index of A and of B is contiguous in memory.
//
// Block tile 128 x 128, reduction stages of 32, four waves of 64 x 64 each
// (4 x 4 accumulators of v_mfma_f32_16x16x4f32). Stages are copied global ->
// LDS directly (buffer loads with an LDS destination; out-of-range offsets
// write 0), double-buffered. An operand whose reduction index is contiguous is
// kept as [row][32] with its 16-byte chunks XOR-swizzled by row, and each lane
// reads 4 consecutive reduction values with one 128-bit LDS read; the MFMA
// steps consume them in a permuted order (any bijection of the reduction index
// applied to both operands leaves the sum unchanged). An operand whose row
// index is contiguous is kept as [32][row + 4], or as [8][row][4] with four
// consecutive reduction values of a row side by side. The MFMA's A/B roles are
// swapped so that each lane ends up holding 4 consecutive output columns,
// stored as one 16-byte write.
#include <algorithm>

#include "device_util.h"
#include "fastdiv.h"
#include "gconv.h"
#include "gconv_internal.h"

namespace gconv {
namespace {

constexpr int BM = 128, BN = 128, BR = 32;
// Operand layouts of a stage in LDS:
//   LR: reduction index contiguous in memory; [row][32], the 16-byte chunks
//       of a row XOR-swizzled by the row;
//   LN: row index contiguous; [32][row + 4];
//   LI: row index contiguous; [32/4][row][4], four consecutive reduction
//       values of a row side by side (one 128-bit LDS read a fragment, where
//       LN takes four 32-bit reads, but each load instruction then gathers
//       four 64-byte runs of global memory instead of one 256-byte run).
constexpr int LR = 0, LN = 1, LI = 2;
constexpr int SROW = BM + 4;          // row stride of an LN tile (== 4 mod 8)
template <int L>
constexpr int tile_floats()
{
    return L == LR ? BM * BR : L == LN ? BR * SROW : BR * BM;
}

// C[M x N] = A[M x R] * B[R x N] for Z batch entries. Entry z uses block
// z % a_mod of A (a_gs floats apart), z % b_mod of B, z % c_mod of C and
// z % bias_mod of the bias: the groups of a layer, or (image, group) pairs
// that share one weight block.
struct GemmArgs {
    const float* A;
    const float* B;
    const float* bias;
    float* C;
    int M, N, R, Z;
    int a_ld, b_ld, c_ld;          // leading dimension of A, B, C (their non-unit stride)
    int a_mod, b_mod, c_mod, bias_mod;
    int64_t a_gs, b_gs, c_gs, bias_gs;  // batch-entry offsets (floats)
    int bias_rows;                 // bias indexed by the row (1) or by the column (0)
    int relu;                      // epilogue: max(v, 0) after the bias
    uint32_t a_bytes, b_bytes;     // extent each entry's A / B resource may address
    // Reduction over several images (RIMG kernels): reduction index r is
    // position r % r_img of image r / r_img, images a_is / b_is floats apart.
    int r_img;
    FastDiv div_rimg;
    int64_t a_is, b_is;
    // Split reduction: workgroup slice ks covers [ks*r_split, (ks+1)*r_split)
    // and writes its partial C c_split floats after slice ks - 1.
    int nsplit, r_split;
    int64_t c_split;
    int m_tiles, n_tiles;
    // Balanced form (SK kernels): sk_nb blocks share the sk_total = tiles *
    // sk_spt (tile, stage) iterations; split tiles' parts go to sk_ws.
    // A launch that first ran whole tiles in full rounds gives the balanced
    // form only the tiles from sk_t0 on (tile t of the form is tile sk_t0 + t).
    int sk_nb, sk_spt, sk_t0;
    int64_t sk_total;
    float* sk_ws;
};

// Load one 32-deep stage of an operand into LDS.
//   LR: element (row, r) at P[row*ld + r]; LDS [row][32], chunk c of row
//       `row` stored at chunk position c ^ (row & 7).
//   LN: element (row, r) at P[r*ld + row]; LDS [r][SROW].
//   LI: element (row, r) at P[r*ld + row]; LDS [r/4][row][r%4]: each
//       instruction fills 16 rows x 4 reduction values.
template <int LAY, bool RIMG = false>
__device__ __forceinline__ void load_stage(__amdgpu_buffer_rsrc_t rs, float* dst, int row0, int rows,
                                           int r0, int R, int ld, int wave, int lane,
                                           const GemmArgs* ga = nullptr, int64_t img_stride = 0)
{
    if constexpr (LAY == LR) {
        // 64 instructions of 64 floats = 2 rows of 32 each.
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int i = wave + 4 * k;
            const int row = 2 * i + (lane >> 5);
            const int chunk = ((lane & 31) >> 2) ^ (row & 7);
            const int r = 4 * chunk + (lane & 3);
            const bool ok = row0 + row < rows && r0 + r < R;
            uint32_t off;
            if constexpr (RIMG) {
                const uint32_t ra = (uint32_t)(r0 + r);
                const uint32_t img = fastdiv(ra, ga->div_rimg);
                off = (uint32_t)((int64_t)(row0 + row) * ld + (int64_t)img * img_stride +
                                 (ra - img * (uint32_t)ga->r_img)) * 4u;
            } else {
                off = (uint32_t)((row0 + row) * ld + r0 + r) * 4u;
            }
            load_lds64(rs, dst + i * 64, ok ? off : kOOB);
        }
    } else if constexpr (LAY == LN) {
        // 32 rows of 128 floats = 2 instructions per row.
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int i = wave + 4 * k;
            const int r = i >> 1, h = i & 1;
            const int row = h * 64 + lane;
            const bool ok = r0 + r < R && row0 + row < rows;
            load_lds64(rs, dst + r * SROW + h * 64,
                       ok ? (uint32_t)((r0 + r) * ld + row0 + row) * 4u : kOOB);
        }
    } else {
        // 8 groups of 4 reduction values x 128 rows = 8 instructions a group.
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int i = wave + 4 * k;
            const int r = 4 * (i >> 3) + (lane & 3);
            const int row = (i & 7) * 16 + (lane >> 2);
            const bool ok = r0 + r < R && row0 + row < rows;
            load_lds64(rs, dst + i * 64, ok ? (uint32_t)((r0 + r) * ld + row0 + row) * 4u : kOOB);
        }
    }
}

// Per-lane byte offsets of the 16 load instructions of a stage at reduction
// index r0 (the same lanes and LDS slots as load_stage); rows past `rows` get
// kOOB. A later stage at r0 + t*BR adds the uniform t*BR*4 (LR) or
// t*BR*ld*4 bytes as the instruction's scalar offset, so a stage that lies
// wholly inside the reduction needs no per-lane arithmetic.
template <int LAY>
__device__ __forceinline__ void stage_offsets(uint32_t (&off)[16], int row0, int rows, int r0, int ld, int wave,
                                              int lane)
{
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int i = wave + 4 * k;
        if constexpr (LAY == LR) {
            const int row = 2 * i + (lane >> 5);
            const int chunk = ((lane & 31) >> 2) ^ (row & 7);
            const int r = 4 * chunk + (lane & 3);
            off[k] = row0 + row < rows ? (uint32_t)((row0 + row) * ld + r0 + r) * 4u : kOOB;
        } else if constexpr (LAY == LN) {
            const int r = i >> 1, h = i & 1;
            const int row = h * 64 + lane;
            off[k] = row0 + row < rows ? (uint32_t)((r0 + r) * ld + row0 + row) * 4u : kOOB;
        } else {
            const int r = 4 * (i >> 3) + (lane & 3);
            const int row = (i & 7) * 16 + (lane >> 2);
            off[k] = row0 + row < rows ? (uint32_t)((r0 + r) * ld + row0 + row) * 4u : kOOB;
        }
    }
}

template <int LAY>
__device__ __forceinline__ void load_stage_fast(__amdgpu_buffer_rsrc_t rs, float* dst, const uint32_t (&off)[16],
                                                uint32_t soff, int wave)
{
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int i = wave + 4 * k;
        if constexpr (LAY == LN) load_lds64s(rs, dst + (i >> 1) * SROW + (i & 1) * 64, off[k], soff);
        else load_lds64s(rs, dst + i * 64, off[k], soff);
    }
}

// Operand values of one 16-deep reduction group (4 MFMA steps) for fragment
// rows row0..row0+15 of an LDS stage: v[s] feeds MFMA step s.
template <int LAY>
__device__ __forceinline__ f4 frag(const float* t, int row, int kg, int q)
{
    if constexpr (LAY == LR) {
        const int chunk = (kg * 4 + q) ^ (row & 7);
        return *(const f4*)(t + row * BR + chunk * 4);
    } else if constexpr (LAY == LN) {
        const int r = kg * 16 + q * 4;
        return f4{t[(r + 0) * SROW + row], t[(r + 1) * SROW + row], t[(r + 2) * SROW + row],
                  t[(r + 3) * SROW + row]};
    } else {
        return *(const f4*)(t + ((kg * 4 + q) * BM + row) * 4);
    }
}

// Tile (mt, nt) of linear index L of the m_tiles x n_tiles grid. Tiles go in
// groups of 8 row panels: consecutive blocks (which an XCD runs together)
// walk an 8-tall strip of the tile grid, so the stage slices of a few A and B
// panels serve many tiles from L2 (fully-connected mode: gradWeight's reads
// 1.9 -> 0.7 GB, forward 2.5% faster; the results are those of the row-major
// order, tile for tile).
#ifndef GCONV_GEMM_GROUP_M
#define GCONV_GEMM_GROUP_M 8
#endif
__device__ __forceinline__ void tile_of(const GemmArgs& a, int L, int& mt, int& nt)
{
    constexpr int GM = GCONV_GEMM_GROUP_M;
    const int grp = L / (GM * a.n_tiles);
    const int first_m = grp * GM;
    const int gm = min(a.m_tiles - first_m, GM);
    const int in_grp = L - grp * GM * a.n_tiles;
    mt = first_m + in_grp % gm;
    nt = in_grp / gm;
}

// Stores a finished 128 x 128 tile: lane (l16, q) of wave (wm, wn) holds
// C[m0 + wm*64 + i*16 + l16][n0 + wn*64 + j*16 + 4q .. +3] in acc[i][j], plus
// the bias (per column, or per row) and the activation. NI < 4: only the
// fragment rows i0 .. i0 + NI - 1, held in acc[i - i0][j].
template <int NI = 4>
__device__ __forceinline__ void store_tile(const GemmArgs& a, int mt, int nt, int z, int ks, const f4 (&acc)[NI][4],
                                           int wm, int wn, int l16, int q, int i0 = 0)
{
    const int m0 = mt * BM, n0 = nt * BN;
    float* Cg = a.C + (z % a.c_mod) * a.c_gs + ks * a.c_split;
    const float* bias = a.bias ? a.bias + (z % a.bias_mod) * a.bias_gs : nullptr;
    const bool vec = (a.N & 3) == 0 && (a.c_ld & 3) == 0 && ((uintptr_t)Cg & 15) == 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + j * 16 + 4 * q;
        f4 bv = f4{0.f, 0.f, 0.f, 0.f};
        if (bias && !a.bias_rows) {
            bv.x = n + 0 < a.N ? bias[n + 0] : 0.f;
            bv.y = n + 1 < a.N ? bias[n + 1] : 0.f;
            bv.z = n + 2 < a.N ? bias[n + 2] : 0.f;
            bv.w = n + 3 < a.N ? bias[n + 3] : 0.f;
        }
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) {
            const int m = m0 + wm * 64 + (i0 + ii) * 16 + l16;
            if (m >= a.M) continue;
            f4 v = acc[ii][j] + bv;
            if (bias && a.bias_rows) v += bias[m];
            if (a.relu) {
                v.x = relu_if(v.x, 1);
                v.y = relu_if(v.y, 1);
                v.z = relu_if(v.z, 1);
                v.w = relu_if(v.w, 1);
            }
            float* row = Cg + (size_t)m * a.c_ld;
            if (vec && n + 3 < a.N) {
                *(f4*)(row + n) = v;
            } else {
                if (n + 0 < a.N) row[n + 0] = v.x;
                if (n + 1 < a.N) row[n + 1] = v.y;
                if (n + 2 < a.N) row[n + 2] = v.z;
                if (n + 3 < a.N) row[n + 3] = v.w;
            }
        }
    }
}

// Balanced form: the grid is sk_nb = min(512, T) blocks and block b takes
// iterations [b*T/nb, (b+1)*T/nb) of the sequence of (tile, stage) pairs,
// T = tiles * spt, tile-major (tile t = L + z * mn in the tile order above),
// so no block's range is empty. With at most as many tiles as blocks a
// block's range is at most spt long, so it covers parts of at most two
// tiles (or one whole tile); their sums go to the
// block's two workspace slots (16 float4 a thread, [slot][k][thread], so each
// store is one coalesced row), and gemm_sk_fixup adds each tile's parts in
// block order. Every block thus does the same number of MFMAs whatever the
// tile count.
__device__ __forceinline__ int64_t sk_it0(const GemmArgs& a, int b)
{
    return (int64_t)b * a.sk_total / a.sk_nb;
}

// Block holding iteration x: the largest b with sk_it0(b) <= x.
__device__ __forceinline__ int sk_block_of(const GemmArgs& a, int64_t x)
{
    return (int)(((x + 1) * a.sk_nb - 1) / a.sk_total);
}

template <int A_L, int B_L, bool RIMG, bool SK>
__global__ void __launch_bounds__(256, 2) gemm_fc_kernel(GemmArgs a)
{
    static_assert(!RIMG || (A_L == LR && B_L == LR), "the image-split reduction needs contiguous reductions");
    static_assert(!(RIMG && SK), "the balanced form takes plain reductions");
    constexpr int TA = tile_floats<A_L>();
    constexpr int TB = tile_floats<B_L>();
    extern __shared__ float lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;  // wave's 64x64 quadrant
    const int mn = a.m_tiles * a.n_tiles;

    // Stages [s_begin, s_end) of tile (mt, nt) of batch entry z, reduction
    // slice ks, into acc (zeroed first).
    auto run_tile = [&](int mt, int nt, int z, int ks, int s_begin, int s_end, f4 (&acc)[4][4]) {
        const int m0 = mt * BM, n0 = nt * BN;
        const int r_begin = ks * a.r_split;
        const int r_end = min(a.R, r_begin + a.r_split);
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A + (z % a.a_mod) * a.a_gs, a.a_bytes);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.B + (z % a.b_mod) * a.b_gs, a.b_bytes);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

        // Stages wholly inside the reduction (all but a ragged last one) load
        // through precomputed lane offsets; the image-split reduction, whose
        // offsets jump at image boundaries, and a ragged stage take the masked
        // per-element path.
        const int full = RIMG ? 0 : (r_end - r_begin) / BR;
        uint32_t offa[16], offb[16];
        if constexpr (!RIMG) {
            stage_offsets<A_L>(offa, m0, a.M, r_begin, a.a_ld, wave, lane);
            stage_offsets<B_L>(offb, n0, a.N, r_begin, a.b_ld, wave, lane);
        } else {
            // The image-split reduction: lane parts at reduction index 0; a
            // stage inside one image adds the image's and the position's
            // offset as the scalar offset.
            stage_offsets<A_L>(offa, m0, a.M, 0, a.a_ld, wave, lane);
            stage_offsets<B_L>(offb, n0, a.N, 0, a.b_ld, wave, lane);
        }
        const uint32_t step_a = A_L == LR ? BR * 4u : (uint32_t)(BR * a.a_ld) * 4u;
        const uint32_t step_b = B_L == LR ? BR * 4u : (uint32_t)(BR * a.b_ld) * 4u;
        auto issue = [&](int stage, int b) {
            float* ta = lds + b * (TA + TB);
            float* tb = ta + TA;
            if (!RIMG && stage < full) {
                load_stage_fast<A_L>(ra, ta, offa, (uint32_t)stage * step_a, wave);
                load_stage_fast<B_L>(rb, tb, offb, (uint32_t)stage * step_b, wave);
                return;
            }
            if constexpr (RIMG) {
                const int r0 = __builtin_amdgcn_readfirstlane(r_begin + stage * BR);
                const int img = (int)fastdiv((uint32_t)r0, a.div_rimg);
                const int p0 = r0 - img * a.r_img;
                if (r0 + BR <= r_end && p0 + BR <= a.r_img) {
                    load_stage_fast<A_L>(ra, ta, offa, (uint32_t)(img * a.a_is + p0) * 4u, wave);
                    load_stage_fast<B_L>(rb, tb, offb, (uint32_t)(img * a.b_is + p0) * 4u, wave);
                    return;
                }
            }
            load_stage<A_L, RIMG>(ra, ta, m0, a.M, r_begin + stage * BR, r_end, a.a_ld, wave, lane, &a, a.a_is);
            load_stage<B_L, RIMG>(rb, tb, n0, a.N, r_begin + stage * BR, r_end, a.b_ld, wave, lane, &a, a.b_is);
        };

        const int nst = (r_end - r_begin + BR - 1) / BR;
        const int s1 = s_end < 0 ? nst : s_end;
        issue(s_begin, 0);
        for (int st = s_begin; st < s1; ++st) {
            const int b = (st - s_begin) & 1;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (st + 1 < s1) issue(st + 1, b ^ 1);
            const float* ta = lds + b * (TA + TB);
            const float* tb = ta + TA;
#pragma unroll
            for (int kg = 0; kg < BR / 16; ++kg) {
                f4 av[4], bv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) av[i] = frag<A_L>(ta, wm * 64 + i * 16 + l16, kg, q);
#pragma unroll
                for (int j = 0; j < 4; ++j) bv[j] = frag<B_L>(tb, wn * 64 + j * 16 + l16, kg, q);
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            // A role <- B operand, B role <- A operand: lane l
                            // then holds C[m = l%16][n = 4*(l/16) + v].
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[j][s], av[i][s],
                                                                             acc[i][j], 0, 0, 0);
            }
            __syncthreads();
        }
    };

    f4 acc[4][4];
    if constexpr (!SK) {
        int bid = xcd_remap(blockIdx.x, gridDim.x);
        const int L = bid % mn;
        bid /= mn;
        const int z = bid % a.Z;
        const int ks = bid / a.Z;
        int mt, nt;
        tile_of(a, L, mt, nt);
        run_tile(mt, nt, z, ks, 0, -1, acc);
        store_tile(a, mt, nt, z, ks, acc, wm, wn, l16, q);
    } else {
        // The block's range: the end of tile t0 (all of it, or all of its
        // range) and perhaps the start of t0 + 1, to slots 0 and 1.
        const int b = xcd_remap(blockIdx.x, gridDim.x);
        const int spt = a.sk_spt;
        const int64_t it0 = sk_it0(a, b), it1 = sk_it0(a, b + 1);
        const int t0 = (int)(it0 / spt);
        const int s0 = (int)(it0 - (int64_t)t0 * spt);
        const int64_t end0 = min((int64_t)(t0 + 1) * spt, it1);
        auto part = [&](int t, int sb, int se, int slot_i) {
            const int L = (t + a.sk_t0) % mn, z = (t + a.sk_t0) / mn;
            int mt, nt;
            tile_of(a, L, mt, nt);
            run_tile(mt, nt, z, 0, sb, se, acc);
            f4* slot = reinterpret_cast<f4*>(a.sk_ws) + (size_t)(2 * b + slot_i) * (16 * 256);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) slot[(i * 4 + j) * 256 + tid] = acc[i][j];
        };
        if (it0 < it1) part(t0, s0, (int)(end0 - (int64_t)t0 * spt), 0);
        if (end0 < it1) part(t0 + 1, 0, (int)(it1 - (int64_t)(t0 + 1) * spt), 1);
    }
}

// Every tile of the balanced form: tile t's parts, held by blocks b_lo ..
// b_hi (one block for a tile held whole), are added in block order (each
// block's slot 0 holds its first tile, slot 1 its second) and stored with the
// bias and activation. Four blocks a tile, one a row of fragments
// (blockIdx.y), so that enough waves keep the part reads in flight.
__global__ void __launch_bounds__(256) gemm_sk_fixup(GemmArgs a)
{
    const int t = blockIdx.x;
    const int spt = a.sk_spt;
    const int b_lo = sk_block_of(a, (int64_t)t * spt), b_hi = sk_block_of(a, (int64_t)(t + 1) * spt - 1);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;
    const int i = blockIdx.y;
    f4 acc[1][4];
    const f4* ws = reinterpret_cast<const f4*>(a.sk_ws);
    for (int b = b_lo; b <= b_hi; ++b) {
        const int first = (int)(sk_it0(a, b) / spt);
        const f4* slot = ws + (size_t)(2 * b + (t == first ? 0 : 1)) * (16 * 256);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f4 v = slot[(i * 4 + j) * 256 + tid];
            acc[0][j] = b == b_lo ? v : acc[0][j] + v;
        }
    }
    const int mn = a.m_tiles * a.n_tiles;
    int mt, nt;
    tile_of(a, (t + a.sk_t0) % mn, mt, nt);
    store_tile<1>(a, mt, nt, (t + a.sk_t0) / mn, 0, acc, wm, wn, l16, q, i);
}

// Sum of the split partials: out[e] = sum_s ws[s*E + e]. A workgroup owns 16
// consecutive elements (16 float4 when E % 4 == 0); its 16 thread rows take
// every 16th slice, and their 16 partial sums are added in a fixed order.
template <typename V>
__global__ void __launch_bounds__(256) gemm_split_reduce(const V* __restrict__ ws, V* __restrict__ out,
                                                         int64_t E, int nsplit)
{
    __shared__ V part[16][17];
    const int q = threadIdx.x & 15, sg = threadIdx.x >> 4;
    const int64_t e = (int64_t)blockIdx.x * 16 + q;
    V sum{};
    if (e < E) {
#pragma unroll 4
        for (int sl = sg; sl < nsplit; sl += 16) sum += ws[(int64_t)sl * E + e];
    }
    part[sg][q] = sum;
    __syncthreads();
    if (sg == 0 && e < E) {
        V t = part[0][q];
#pragma unroll
        for (int i = 1; i < 16; ++i) t += part[i][q];
        out[e] = t;
    }
}

// Sum of a few split partials with the forward pass's epilogue:
// out[e] = act(bias[e % bias_n] + sum_s ws[s*E + e]), slices added in order
// (bias may be NULL; V = f4 needs E and bias_n multiples of 4). One thread
// per element (or float4): each partial is read once, coalesced.
template <typename V>
__global__ void __launch_bounds__(256) gemm_split_epilogue(const V* __restrict__ ws, V* __restrict__ out,
                                                           int64_t E, int nsplit, const float* __restrict__ bias,
                                                           int bias_n, int relu)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= E) return;
    V sum = ws[e];
    for (int sl = 1; sl < nsplit; ++sl) sum += ws[(int64_t)sl * E + e];
    if constexpr (sizeof(V) == sizeof(f4)) {
        if (bias) {
            const int c = (int)((e * 4) % bias_n);
            sum += *(const f4*)(bias + c);
        }
        if (relu) {
            sum.x = relu_if(sum.x, 1);
            sum.y = relu_if(sum.y, 1);
            sum.z = relu_if(sum.z, 1);
            sum.w = relu_if(sum.w, 1);
        }
    } else {
        if (bias) sum += bias[e % bias_n];
        sum = relu_if(sum, relu);
    }
    out[e] = sum;
}

// Defaults that make the batch entries plain groups with one reduction slice.
void plain(GemmArgs& a)
{
    a.a_mod = a.b_mod = a.c_mod = a.bias_mod = a.Z;
    a.bias_rows = 0;
    a.relu = 0;
    a.r_img = 0;
    a.div_rimg = make_fastdiv(1);
    a.a_is = a.b_is = 0;
    a.nsplit = 1;
    a.r_split = a.R;
    a.c_split = 0;
}

// Blocks of the balanced form: two a CU.
constexpr int kSkBlocks = 512;

#ifndef GCONV_GEMM_NO_SK
constexpr bool kSkOn = true;
#else
constexpr bool kSkOn = false;
#endif

// Whether a one-slice GEMM over `tiles` output tiles takes the balanced form:
// from a tile per CU (fewer tiles split their reduction instead) to fewer
// than one tile per block slot, where one round of whole tiles leaves CUs
// with a single block, which does not keep a CU's matrix cores busy
// (fully-connected mode's forward, 416 tiles: 1.036 -> 0.953 ms). With more
// tiles the dispatcher's handing of tiles to free slots balances better than
// a fixed split of the sequence (its gradInput, 936 tiles: 0.959 ms whole,
// 1.089 balanced; gradWeight, 2304 tiles: 0.962 against 1.045).
// (The form itself needs fewer tiles than blocks: a block then covers parts
// of at most two tiles.)
bool use_sk(int64_t tiles) { return kSkOn && tiles >= 256 && tiles < kSkBlocks; }

// Whether a larger one-slice GEMM over an R-long reduction runs its whole
// rounds of kSkBlocks tiles as plain blocks and hands a last round of at
// most half that many tiles, which would leave CUs with a single block, to
// the balanced form. Only long reductions gain: fully-connected mode's
// gradWeight (2304 tiles of 50 stages, a last round of 256) 995 -> 962 us
// in four alternating runs, 949 -> 891 in two more; the channels-last 1x1
// layer's forward (1568 tiles of 8 stages) went
// 150 -> 161 us and its gradInput (3136 of 4) 167 -> 182, where the two more
// launches cost more than the short last round.
#ifndef GCONV_GEMM_SK_TAIL
#define GCONV_GEMM_SK_TAIL 1
#endif
constexpr int kSkTailMinStages = 32;
#ifndef GCONV_GEMM_SK_TAIL_MAX
#define GCONV_GEMM_SK_TAIL_MAX (kSkBlocks / 2)
#endif
bool use_sk_tail(int64_t tiles, int R)
{
    const int64_t r = tiles % kSkBlocks;
    return kSkOn && GCONV_GEMM_SK_TAIL && tiles > kSkBlocks && r > 0 && r <= GCONV_GEMM_SK_TAIL_MAX &&
           (R + BR - 1) / BR >= kSkTailMinStages;
}
bool use_sk_any(int64_t tiles, int R) { return use_sk(tiles) || use_sk_tail(tiles, R); }

// Workspace of the balanced form: two 128 x 128 slots a block.
size_t sk_workspace() { return (size_t)2 * kSkBlocks * BM * BN * sizeof(float); }

// One launch of the GEMM: one block per (tile, batch entry, reduction slice),
// or, with sk_ws, the balanced form (up to kSkBlocks blocks over the tile-stage
// sequence, one slice) and its fix-up pass over the split tiles.
template <int A_L, int B_L, bool RIMG = false>
void launch(GemmArgs& a, hipStream_t st, float* sk_ws = nullptr)
{
    constexpr int TA = tile_floats<A_L>();
    constexpr int TB = tile_floats<B_L>();
    const size_t lds = 2 * (size_t)(TA + TB) * 4;
    a.m_tiles = (a.M + BM - 1) / BM;
    a.n_tiles = (a.N + BN - 1) / BN;
    const int tiles = a.m_tiles * a.n_tiles * a.Z;
    if constexpr (!RIMG) {
        if (sk_ws && (tiles < kSkBlocks || use_sk_tail(tiles, a.R))) {
            // whole rounds first (none below kSkBlocks tiles)
            const int dp = tiles / kSkBlocks * kSkBlocks;
            if (dp > 0) {
                auto kdp = gemm_fc_kernel<A_L, B_L, false, false>;
                static const bool attr_dp = hipFuncSetAttribute((const void*)kdp,
                                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                                160 * 1024) == hipSuccess;
                (void)attr_dp;
                hipLaunchKernelGGL(kdp, dim3(dp), dim3(256), lds, st, a);
            }
            a.sk_spt = (a.R + BR - 1) / BR;
            a.sk_t0 = dp;
            a.sk_total = (int64_t)(tiles - dp) * a.sk_spt;
            // no block without iterations: every block in a tile's range then
            // holds a part of it (a few tiles of few stages have fewer
            // (tile, stage) pairs than kSkBlocks)
            a.sk_nb = (int)std::min<int64_t>(kSkBlocks, a.sk_total);
            a.sk_ws = sk_ws;
            auto kern = gemm_fc_kernel<A_L, B_L, false, true>;
            static const bool attr = hipFuncSetAttribute((const void*)kern,
                                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                                         160 * 1024) == hipSuccess;
            (void)attr;
            hipLaunchKernelGGL(kern, dim3(a.sk_nb), dim3(256), lds, st, a);
            hipLaunchKernelGGL(gemm_sk_fixup, dim3(tiles - dp, 4), dim3(256), 0, st, a);
            return;
        }
    }
    const int blocks = tiles * a.nsplit;
    auto kern = gemm_fc_kernel<A_L, B_L, RIMG, false>;
    static const bool attr = hipFuncSetAttribute((const void*)kern,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 160 * 1024) == hipSuccess;
    (void)attr;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), lds, st, a);
}

// Byte extent of one group's operand: rows x leading dimension (the last row
// only as far as it is used), which must stay below 2^30.
bool extent_ok(int64_t rows, int64_t ld, int64_t used_last)
{
    const int64_t e = ((rows - 1) * ld + used_last) * 4;
    return e > 0 && e < (int64_t(1) << 30);
}

}  // namespace

// LDS layout of the row-contiguous FC operands (gradInput's filter, gradWeight's
// dy; gradWeight's x stays LN): LI where a block's reduction runs at least
// kLiMinStages stages, LN below. LI saves LDS reads but makes each stage's
// fetch gather four 64-byte runs, which a short reduction cannot hide.
// Measured: fully-connected mode (gradInput 128 stages, gradWeight 50),
// four alternating runs each, gradInput 1032 -> 1017 us and gradWeight 980
// -> 963 against LN (LI on both gradWeight operands: 975); the channels-last
// 1x1 layer's gradInput (4 stages) 165 -> 175 us with LI, its gradWeight
// (256 slices of 25 stages) 132 -> 122.
constexpr int kLiMinStages = 16;
bool use_li(int r_split) { return (r_split + BR - 1) / BR >= kLiMinStages; }

bool fc_supported(const Shape& s)
{
    if (!is_fc_mode(s)) return false;
    const int64_t D = (int64_t)s.Cg * s.kh * s.kw;     // per-group flattened extent
    const int64_t Dt = (int64_t)s.C * s.H * s.W;        // full row of x
    if (s.N < 1) return false;
    // A and B resources of every op (see the launchers below).
    return extent_ok(s.N, Dt, D) && extent_ok(s.N, s.K, s.Kg) && extent_ok(s.Kg, D, D) &&
           D < (1 << 30) && s.w_elems < (int64_t(1) << 28);
}

// Reduction slices for a GEMM whose output tiles alone leave CUs idle. With
// T tiles and n slices each CU works through about ceil(T*n / CUs) units of
// 1/n of a tile, so a split pays when it fills CUs that would otherwise wait
// out the last round. It costs a pass that reads the n partials of the E
// outputs and writes the result (the partials themselves are written while
// the matrix cores are busy). Each slice keeps at least 8 stages. The
// constants are MI355X's: 256 CUs, about 0.48 TFLOP/s per CU on one 128 x 128
// tile stream, about 4.5 TB/s for the partials pass.
// Grids of at least one tile per CU are not split: two blocks share a CU and
// the blocks do not run in lockstep rounds, so the uneven last round costs
// less than this count says, and the partials pass more. Fully-connected
// mode measured so: gradInput's 936 tiles ran 955 us whole against 1001-1034
// in two to four slices, the forward's 416 tiles 1081-1111 against 1095-1120.
static int balance_splits(int64_t tiles, int64_t R, int64_t E, int max_split)
{
    constexpr int64_t kCUs = 256;
    constexpr double kTileRate = 0.48e12, kPassBw = 4.5e12, kLaunch = 4e-6;
    if (tiles >= kCUs) return 1;
    const double t_tile = 2.0 * BM * BN * (double)R / kTileRate;
    int best = 1;
    double best_t = 0.0;
    for (int n = 1; n <= max_split; ++n) {
        if (n > 1 && R / n < 8 * BR) break;
        const double rounds = (double)((tiles * n + kCUs - 1) / kCUs);
        double t = rounds / n * t_tile;
        if (n > 1) t += (double)(n + 1) * (double)E * 4.0 / kPassBw + kLaunch;  // the partials pass
        if (n == 1 || t < 0.98 * best_t) {
            best = n;
            best_t = t;
        }
    }
    return best;
}

static void fc_data_split(const Shape& s, int op, int* nsplit, int* r_split)
{
    const int64_t D = (int64_t)s.Cg * s.kh * s.kw;
    int64_t M = s.N, N, R, E;
    if (op == GCONV_OP_FWD) { N = s.Kg; R = D; E = (int64_t)s.N * s.K; }
    else { N = D; R = s.Kg; E = (int64_t)s.N * s.C * s.H * s.W; }
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN) * s.G;
    const int n = balance_splits(tiles, R, E, 6);
    int64_t rs = (R + n - 1) / n;
    rs = (rs + BR - 1) / BR * BR;
    *r_split = (int)rs;
    *nsplit = (int)((R + rs - 1) / rs);
}

// Output tiles of the FC forward (gradInput) GEMM over all groups.
// Reduction length of the forward (C*kh*kw a group) and gradInput (K a group) GEMMs.
static int fc_data_reduction(const Shape& s, int op)
{
    return op == GCONV_OP_FWD ? s.Cg * s.kh * s.kw : s.Kg;
}
static int64_t fc_data_tiles(const Shape& s, int op)
{
    const int64_t D = (int64_t)s.Cg * s.kh * s.kw;
    const int64_t N = op == GCONV_OP_FWD ? s.Kg : D;
    return ((s.N + BM - 1) / BM) * ((N + BN - 1) / BN) * s.G;
}

size_t fc_data_workspace(const Shape& s, int op)
{
    int nsplit, r_split;
    fc_data_split(s, op, &nsplit, &r_split);
    if (nsplit <= 1) return use_sk_any(fc_data_tiles(s, op), fc_data_reduction(s, op)) ? sk_workspace() : 0;
    const int64_t E = op == GCONV_OP_FWD ? (int64_t)s.N * s.K : (int64_t)s.N * s.C * s.H * s.W;
    return (size_t)nsplit * (size_t)E * 4;
}

static void split_epilogue(const float* ws, float* out, int64_t E, int nsplit, const float* bias,
                           int bias_n, int relu, hipStream_t st)
{
    const bool v4 = (E & 3) == 0 && ((uintptr_t)out & 15) == 0 &&
                    (!bias || ((bias_n & 3) == 0 && ((uintptr_t)bias & 15) == 0));
    if (v4) {
        const int64_t E4 = E / 4;
        hipLaunchKernelGGL(gemm_split_epilogue<f4>, dim3((unsigned)((E4 + 255) / 256)), dim3(256), 0, st,
                           (const f4*)ws, (f4*)out, E4, nsplit, bias, bias_n, relu);
    } else {
        hipLaunchKernelGGL(gemm_split_epilogue<float>, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, st,
                           ws, out, E, nsplit, bias, bias_n, relu);
    }
}

// y[n, g*Kg + k] = sum_d x[n, g*D + d] * w[g*Kg + k, d] + b. When the tiles
// spread unevenly the reduction is split into slices whose partials go to the
// workspace, and one pass adds them in slice order with the bias and the
// activation.
bool fc_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y, float* ws,
            hipStream_t st)
{
    const int D = s.Cg * s.kh * s.kw, Dt = s.C * s.H * s.W;
    int nsplit, r_split;
    fc_data_split(s, GCONV_OP_FWD, &nsplit, &r_split);
    if (nsplit > 1 && !ws) return false;
    GemmArgs a{};
    a.A = x; a.B = w; a.bias = nsplit > 1 ? nullptr : bias; a.C = nsplit > 1 ? ws : y;
    a.M = s.N; a.N = s.Kg; a.R = D; a.Z = s.G;
    plain(a);
    a.a_ld = Dt; a.b_ld = D; a.c_ld = s.K;
    a.a_gs = D; a.b_gs = (int64_t)s.Kg * D; a.c_gs = s.Kg; a.bias_gs = s.Kg;
    a.relu = nsplit > 1 ? 0 : s.relu;
    a.a_bytes = (uint32_t)(((int64_t)(s.N - 1) * Dt + D) * 4);
    a.b_bytes = (uint32_t)((int64_t)s.Kg * D * 4);
    a.nsplit = nsplit;
    a.r_split = r_split;
    a.c_split = (int64_t)s.N * s.K;
    const bool sk = nsplit == 1 && use_sk_any(fc_data_tiles(s, GCONV_OP_FWD), fc_data_reduction(s, GCONV_OP_FWD));
    if (sk && !ws) return false;
    launch<LR, LR>(a, st, sk ? ws : nullptr);
    if (nsplit > 1) split_epilogue(ws, y, (int64_t)s.N * s.K, nsplit, bias, s.K, s.relu, st);
    return true;
}

// dx[n, g*D + d] = sum_k dy[n, g*Kg + k] * w[g*Kg + k, d] (split like the forward pass)
bool fc_bwd_data(const Shape& s, const float* dy, const float* w, float* dx, float* ws, hipStream_t st)
{
    const int D = s.Cg * s.kh * s.kw, Dt = s.C * s.H * s.W;
    int nsplit, r_split;
    fc_data_split(s, GCONV_OP_BWD_DATA, &nsplit, &r_split);
    if (nsplit > 1 && !ws) return false;
    GemmArgs a{};
    a.A = dy; a.B = w; a.bias = nullptr; a.C = nsplit > 1 ? ws : dx;
    a.M = s.N; a.N = D; a.R = s.Kg; a.Z = s.G;
    plain(a);
    a.a_ld = s.K; a.b_ld = D; a.c_ld = Dt;
    a.a_gs = s.Kg; a.b_gs = (int64_t)s.Kg * D; a.c_gs = D; a.bias_gs = 0;
    a.a_bytes = (uint32_t)(((int64_t)(s.N - 1) * s.K + s.Kg) * 4);
    a.b_bytes = (uint32_t)((int64_t)s.Kg * D * 4);
    a.nsplit = nsplit;
    a.r_split = r_split;
    a.c_split = (int64_t)s.N * Dt;
    const bool sk = nsplit == 1 && use_sk_any(fc_data_tiles(s, GCONV_OP_BWD_DATA), fc_data_reduction(s, GCONV_OP_BWD_DATA));
    if (sk && !ws) return false;
    if (use_li(r_split)) launch<LR, LI>(a, st, sk ? ws : nullptr);
    else launch<LR, LN>(a, st, sk ? ws : nullptr);
    if (nsplit > 1) split_epilogue(ws, dx, (int64_t)s.N * Dt, nsplit, nullptr, 1, 0, st);
    return true;
}

// Reduction slices of a gradWeight GEMM over R rows with `tiles` output tiles:
// enough slices for about 512 workgroups, each slice at least 8 stages deep
// and a multiple of the stage depth (one slice when the tiles alone fill the
// chip, as in the fully-connected layer of the cudnn.torch issue).
static void split_rows(int64_t R, int64_t tiles, int* nsplit, int* r_split)
{
    int64_t want = std::max<int64_t>(1, (512 + tiles - 1) / tiles);
    want = std::min<int64_t>(want, std::max<int64_t>(1, R / (8 * BR)));
    int64_t rs = (R + want - 1) / want;
    rs = (rs + BR - 1) / BR * BR;
    *r_split = (int)rs;
    *nsplit = (int)((R + rs - 1) / rs);
}

static void fc_split(const Shape& s, int* nsplit, int* r_split)
{
    const int64_t D = (int64_t)s.Cg * s.kh * s.kw;
    split_rows(s.N, (int64_t)((s.Kg + BM - 1) / BM) * ((D + BN - 1) / BN) * s.G, nsplit, r_split);
}

// Output tiles of the FC gradWeight GEMM over all groups.
static int64_t fc_filter_tiles(const Shape& s)
{
    const int64_t D = (int64_t)s.Cg * s.kh * s.kw;
    return (int64_t)((s.Kg + BM - 1) / BM) * ((D + BN - 1) / BN) * s.G;
}

size_t fc_bwd_filter_workspace(const Shape& s)
{
    int nsplit, r_split;
    fc_split(s, &nsplit, &r_split);
    if (nsplit <= 1) return use_sk_any(fc_filter_tiles(s), s.N) ? sk_workspace() : 0;
    return (size_t)nsplit * (size_t)s.w_elems * 4;
}

static void split_reduce(const float* ws, float* dw, int64_t E, int nsplit, hipStream_t st)
{
    if ((E & 3) == 0 && ((uintptr_t)dw & 15) == 0) {
        hipLaunchKernelGGL(gemm_split_reduce<f4>, dim3((unsigned)((E / 4 + 15) / 16)), dim3(256), 0, st,
                           (const f4*)ws, (f4*)dw, E / 4, nsplit);
    } else {
        hipLaunchKernelGGL(gemm_split_reduce<float>, dim3((unsigned)((E + 15) / 16)), dim3(256), 0, st, ws, dw,
                           E, nsplit);
    }
}

// dw[g*Kg + k, d] = sum_n dy[n, g*Kg + k] * x[n, g*D + d]; with few output
// tiles (many rows: a 1x1 layer over N*H*W channels-last pixels) the rows are
// split over workgroup slices whose partials are added in slice order.
bool fc_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws, hipStream_t st)
{
    const int D = s.Cg * s.kh * s.kw, Dt = s.C * s.H * s.W;
    int nsplit, r_split;
    fc_split(s, &nsplit, &r_split);
    if (nsplit > 1 && !ws) return false;
    GemmArgs a{};
    a.A = dy; a.B = x; a.bias = nullptr; a.C = nsplit > 1 ? ws : dw;
    a.M = s.Kg; a.N = D; a.R = s.N; a.Z = s.G;
    plain(a);
    a.a_ld = s.K; a.b_ld = Dt; a.c_ld = D;
    a.a_gs = s.Kg; a.b_gs = D; a.c_gs = (int64_t)s.Kg * D; a.bias_gs = 0;
    a.a_bytes = (uint32_t)(((int64_t)(s.N - 1) * s.K + s.Kg) * 4);
    a.b_bytes = (uint32_t)(((int64_t)(s.N - 1) * Dt + D) * 4);
    a.nsplit = nsplit;
    a.r_split = r_split;
    a.c_split = s.w_elems;
    const bool sk = nsplit == 1 && use_sk_any(fc_filter_tiles(s), s.N);
    if (sk && !ws) return false;
    if (use_li(r_split)) launch<LI, LN>(a, st, sk ? ws : nullptr);
    else launch<LN, LN>(a, st, sk ? ws : nullptr);
    if (nsplit > 1) split_reduce(ws, dw, s.w_elems, nsplit, st);
    return true;
}

// ---- pointwise (1x1, stride 1, no padding) ------------------------------------
// Per image n and group g, with P = H*W and the planes as matrices:
//     forward     Y[n,g]  (Kg x P) = W[g] (Kg x Cg) * X[n,g] (Cg x P) + b
//     gradInput   dX[n,g] (Cg x P) = W[g]^T * dY[n,g] (Kg x P)
//     gradWeight  dW[g]   (Kg x Cg) = sum_n dY[n,g] * X[n,g]^T
// The first two are N*G GEMMs that share the weight block of their group; the
// third reduces over every image and pixel, split over workgroup slices whose
// partials are added in slice order.

bool pointwise_supported(const Shape& s)
{
    if (!(s.kh == 1 && s.kw == 1 && s.sh == 1 && s.sw == 1 && s.ph == 0 && s.pw == 0)) return false;
    if (s.Ho != s.H || s.Wo != s.W) return false;  // no end padding: y planes are H x W
    if (s.N < 1) return false;
    const int64_t P = (int64_t)s.H * s.W;
    if (P * s.N >= (int64_t(1) << 31) || s.x_elems >= (int64_t(1) << 31) || s.y_elems >= (int64_t(1) << 31))
        return false;
    // gradWeight addresses a group's planes across all images from one resource.
    return extent_ok(s.N, (int64_t)s.C * P, (int64_t)s.Cg * P) &&
           extent_ok(s.N, (int64_t)s.K * P, (int64_t)s.Kg * P) && extent_ok(s.Kg, s.Cg, s.Cg);
}

// Reduction slices of the pointwise gradWeight GEMM (over every image's pixels).
static void pointwise_split(const Shape& s, int* nsplit, int* r_split)
{
    split_rows((int64_t)s.N * s.H * s.W, (int64_t)((s.Kg + BM - 1) / BM) * ((s.Cg + BN - 1) / BN) * s.G,
               nsplit, r_split);
}

size_t pointwise_bwd_filter_workspace(const Shape& s)
{
    int nsplit, r_split;
    pointwise_split(s, &nsplit, &r_split);
    return nsplit > 1 ? (size_t)nsplit * (size_t)s.w_elems * 4 : 0;
}

// y[n, g*Kg + k, p] = sum_c w[g*Kg + k, c] * x[n, g*Cg + c, p] + b[g*Kg + k]
void pointwise_fwd(const Shape& s, const float* x, const float* w, const float* bias, float* y,
                   hipStream_t st)
{
    const int P = s.H * s.W;
    GemmArgs a{};
    a.A = w; a.B = x; a.bias = bias; a.C = y;
    a.M = s.Kg; a.N = P; a.R = s.Cg; a.Z = s.N * s.G;
    plain(a);
    a.a_mod = s.G; a.bias_mod = s.G;
    a.a_ld = s.Cg; a.b_ld = P; a.c_ld = P;
    a.a_gs = (int64_t)s.Kg * s.Cg; a.b_gs = (int64_t)s.Cg * P; a.c_gs = (int64_t)s.Kg * P;
    a.bias_gs = s.Kg; a.bias_rows = 1;
    a.relu = s.relu;
    a.a_bytes = (uint32_t)((int64_t)s.Kg * s.Cg * 4);
    a.b_bytes = (uint32_t)((int64_t)s.Cg * P * 4);
    launch<LR, LN>(a, st);
}

// dx[n, g*Cg + c, p] = sum_k w[g*Kg + k, c] * dy[n, g*Kg + k, p]
void pointwise_bwd_data(const Shape& s, const float* dy, const float* w, float* dx, hipStream_t st)
{
    const int P = s.H * s.W;
    GemmArgs a{};
    a.A = w; a.B = dy; a.bias = nullptr; a.C = dx;
    a.M = s.Cg; a.N = P; a.R = s.Kg; a.Z = s.N * s.G;
    plain(a);
    a.a_mod = s.G;
    a.a_ld = s.Cg; a.b_ld = P; a.c_ld = P;
    a.a_gs = (int64_t)s.Kg * s.Cg; a.b_gs = (int64_t)s.Kg * P; a.c_gs = (int64_t)s.Cg * P;
    a.a_bytes = (uint32_t)((int64_t)s.Kg * s.Cg * 4);
    a.b_bytes = (uint32_t)((int64_t)s.Kg * P * 4);
    launch<LN, LN>(a, st);
}

// dw[g*Kg + k, c] = sum_{n, p} dy[n, g*Kg + k, p] * x[n, g*Cg + c, p]
bool pointwise_bwd_filter(const Shape& s, const float* x, const float* dy, float* dw, float* ws,
                          hipStream_t st)
{
    const int P = s.H * s.W;
    int nsplit, r_split;
    pointwise_split(s, &nsplit, &r_split);
    if (nsplit > 1 && !ws) return false;
    GemmArgs a{};
    a.A = dy; a.B = x; a.bias = nullptr; a.C = nsplit > 1 ? ws : dw;
    a.M = s.Kg; a.N = s.Cg; a.R = s.N * P; a.Z = s.G;
    plain(a);
    a.a_ld = P; a.b_ld = P; a.c_ld = s.Cg;
    a.a_gs = (int64_t)s.Kg * P; a.b_gs = (int64_t)s.Cg * P; a.c_gs = (int64_t)s.Kg * s.Cg;
    a.a_bytes = (uint32_t)(((int64_t)(s.N - 1) * s.K * P + (int64_t)s.Kg * P) * 4);
    a.b_bytes = (uint32_t)(((int64_t)(s.N - 1) * s.C * P + (int64_t)s.Cg * P) * 4);
    a.r_img = P;
    a.div_rimg = make_fastdiv((uint32_t)P);
    a.a_is = (int64_t)s.K * P;
    a.b_is = (int64_t)s.C * P;
    a.nsplit = nsplit;
    a.r_split = r_split;
    a.c_split = s.w_elems;
    launch<LR, LR, true>(a, st);
    if (nsplit > 1) split_reduce(ws, dw, s.w_elems, nsplit, st);
    return true;
}

}  // namespace gconv
