// bias.hip -- gradBias for grouped 2-D convolution:
//   db[k] = sum over n, ho, wo of dy[n, k, ho, wo]
// (a plain reduction of dy over everything but the channel: the DLPrimitives
// Blog, "Pointwise Broadcast Reduce", the bias-gradient formula).
//
// Deterministic. A CU streaming from HBM is limited by the loads it can keep
// in flight (about 60 GB/s per CU measured), so a reduction group (a
// channel's planes, or a block of columns of a [rows, K] gradient) is split
// over S workgroups whenever the groups alone would occupy fewer than about
// 512 workgroups; each writes its partial to the workspace ([S][K]), and a
// second small kernel adds each channel's S partials in slice order. With
// S = 1 the workgroup writes db itself: one launch, no workspace.
// (A one-launch form, where the last workgroup of a group to arrive adds the
// partials, needs device-scope fences, which on MI355X write back and
// invalidate an XCD's L2 per workgroup: it measured two to thirty times
// slower.)
//   plane layout (Ho*Wo > 1): group k is channel k, its N planes taken as one
//     sequence of N*Ho*Wo values, cut into S contiguous slices;
//   column layout (Ho*Wo == 1, dy is [N, K]: fully-connected mode, NHWC):
//     group b is a block of columns, its rows cut into S slices; wide rows
//     give a thread 4 columns, narrow rows (K < 1024) give a block several
//     whole rows per wave instruction.
#include <algorithm>

#include "device_util.h"
#include "fastdiv.h"
#include "gconv_internal.h"

namespace gconv {
namespace {

constexpr int kB = 256;
constexpr int kTargetBlocks = 512;      // about two workgroups per CU
struct BiasArgs {
    const float* dy;
    float* db;
    float* part;                 // [S][K] partials (S > 1)
    int N, K, P, S;
    int len, total, chunk;       // plane layout: values per plane (floats or f4), N*len, per slice
    FastDiv div_len;
    int rows_chunk, KT;          // column layouts: rows per slice, column quads per block (narrow rows)
};

// Plane layout: workgroup (s, k) sums values [s*chunk, (s+1)*chunk) of
// channel k's N planes, then the four wave sums are added in order. A thread
// keeps U loads in flight: 8 of 16 bytes, or 32 of 4 bytes when the planes
// are not whole float4s (either way 32 KB per 256-thread workgroup, which is
// what keeps a CU's share of the HBM bandwidth busy); the one-pass form's
// 1024 threads keep 16 each (256 KB: one CU streams a whole channel).
template <bool VEC, int NT>
__global__ void __launch_bounds__(NT) bias_planes(BiasArgs a)
{
    constexpr int U = VEC ? (NT == 1024 ? 16 : 8) : 32;  // 16 a thread for the one-pass form
    constexpr int NW = NT / 64;
    __shared__ float red[NW];
    const int s = blockIdx.x, k = blockIdx.y;
    const int i_end = min(a.total, (s + 1) * a.chunk);
    float acc = 0.f;
    f4 a4 = f4{0.f, 0.f, 0.f, 0.f};
    for (int i0 = s * a.chunk + threadIdx.x; i0 < i_end; i0 += U * NT) {
        if constexpr (VEC) {
            f4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * NT;
                v[u] = f4{0.f, 0.f, 0.f, 0.f};
                if (i < i_end) {
                    const int n = (int)fastdiv((uint32_t)i, a.div_len);
                    v[u] = reinterpret_cast<const f4*>(a.dy + ((int64_t)n * a.K + k) * a.P)[i - n * a.len];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) a4 += v[u];
        } else {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * NT;
                v[u] = 0.f;
                if (i < i_end) {
                    const int n = (int)fastdiv((uint32_t)i, a.div_len);
                    v[u] = a.dy[((int64_t)n * a.K + k) * a.P + (i - n * a.len)];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) acc += v[u];
        }
    }
    if constexpr (VEC) acc = (a4.x + a4.y) + (a4.z + a4.w);
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x != 0) return;
    float t = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) t += red[w];
    if (a.S == 1) {
        a.db[k] = t;
        return;
    }
    a.part[(int64_t)s * a.K + k] = t;
}

// Column layout, wide rows: block (b, s) gives each thread 4 consecutive
// columns (4*(b*256 + t) ..) and sums rows [s*rows_chunk, ..) of them.
__global__ void __launch_bounds__(kB) bias_cols(BiasArgs a)
{
    const int b = blockIdx.x, s = blockIdx.y;
    const int k4 = b * kB + threadIdx.x;
    const bool on = k4 * 4 < a.K;
    const int n0 = s * a.rows_chunk, n1 = min(a.N, n0 + a.rows_chunk);
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
    if (on) {
        // eight rows in flight per thread, added in row order
        for (int nb = n0; nb < n1; nb += 8) {
            f4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = nb + u < n1 ? reinterpret_cast<const f4*>(a.dy + (int64_t)(nb + u) * a.K)[k4]
                                   : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += v[u];
        }
    }
    if (a.S == 1) {
        if (on) reinterpret_cast<f4*>(a.db)[k4] = acc;
        return;
    }
    if (on) reinterpret_cast<f4*>(a.part + (int64_t)s * a.K)[k4] = acc;
}

// Column layout, narrow rows (K a multiple of 4 below 1024: NHWC gradients):
// a block is KT column quads x 256/KT row phases, so each wave instruction
// reads whole consecutive rows; thread (c, r) adds rows n0 + r, n0 + r +
// 256/KT, ... of its quad, and the row phases are added in order through LDS.
__global__ void __launch_bounds__(kB) bias_rows(BiasArgs a)
{
    __shared__ f4 part[kB];
    const int b = blockIdx.x, s = blockIdx.y;
    const int n0 = s * a.rows_chunk, n1 = min(a.N, n0 + a.rows_chunk);
    const int K4 = a.K >> 2;
    const int ct = threadIdx.x % a.KT, rt = threadIdx.x / a.KT, RT = kB / a.KT;
    const int c4 = b * a.KT + ct;
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
    if (c4 < K4) {
#pragma unroll 8
        for (int n = n0 + rt; n < n1; n += RT) acc += reinterpret_cast<const f4*>(a.dy + (int64_t)n * a.K)[c4];
    }
    part[threadIdx.x] = acc;
    __syncthreads();
    const bool lead = rt == 0 && c4 < K4;
    f4 t = f4{0.f, 0.f, 0.f, 0.f};
    if (lead) {
        t = part[ct];
        for (int r = 1; r < RT; ++r) t += part[r * a.KT + ct];
    }
    if (a.S == 1) {
        if (lead) reinterpret_cast<f4*>(a.db)[c4] = t;
        return;
    }
    if (lead) reinterpret_cast<f4*>(a.part + (int64_t)s * a.K)[c4] = t;
}

// Column layout with K not a multiple of 4 (or misaligned pointers): one
// column per thread.
__global__ void __launch_bounds__(kB) bias_cols_scalar(BiasArgs a)
{
    const int b = blockIdx.x, s = blockIdx.y;
    const int k = b * kB + threadIdx.x;
    const bool on = k < a.K;
    const int n0 = s * a.rows_chunk, n1 = min(a.N, n0 + a.rows_chunk);
    float acc = 0.f;
    if (on) {
        for (int nb = n0; nb < n1; nb += 16) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = nb + u < n1 ? a.dy[(int64_t)(nb + u) * a.K + k] : 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u) acc += v[u];
        }
    }
    if (a.S == 1) {
        if (on) a.db[k] = acc;
        return;
    }
    if (on) a.part[(int64_t)s * a.K + k] = acc;
}

// db[k] = sum over s of part[s*K + k], slices in order. Block = 16 channels x
// 16 slice groups: thread (kk, sg) adds slices sg, sg + 16, ... in order, then
// the 16 group sums are added in order.
__global__ void __launch_bounds__(kB) bias_finalize(const float* __restrict__ part, float* __restrict__ db, int K,
                                                    int S)
{
    __shared__ float red[16][17];
    const int kk = threadIdx.x & 15, sg = threadIdx.x >> 4;
    const int k = blockIdx.x * 16 + kk;
    float acc = 0.f;
    if (k < K) {
#pragma unroll 4
        for (int j = sg; j < S; j += 16) acc += part[(int64_t)j * K + k];
    }
    red[sg][kk] = acc;
    __syncthreads();
    if (sg != 0 || k >= K) return;
    float sum = red[0][kk];
#pragma unroll
    for (int i = 1; i < 16; ++i) sum += red[i][kk];
    db[k] = sum;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Column quads per block of the narrow-row kernel (a power of two up to 64).
int rows_kt(int K)
{
    int kt = 1;
    while (kt < 64 && kt < K / 4) kt *= 2;
    return kt;
}

enum Form { kPlanes, kCols, kRows, kColsScalar };

// How the reduction is laid out and split. Column forms depend only on K (the
// vector width never changes the workspace); `vec` (16-byte loads) also
// needs aligned pointers, checked at launch.
struct Plan {
    Form form;
    int groups, S;
    int len, total, chunk, rows_chunk, KT;
    bool vec;
};

Plan make_plan(const Shape& s, bool ptr_aligned)
{
    Plan p{};
    const int P = s.Ho * s.Wo;
    if (P > 1) {
        p.form = kPlanes;
        p.vec = (P & 3) == 0 && ptr_aligned;
        p.len = p.vec ? P / 4 : P;
        p.total = s.N * p.len;
        p.groups = s.K;
        // Enough slices for about 512 workgroups, each with at least 8192
        // floats (8 loads per thread); the cap S0 does not depend on the
        // load width, and the slices actually used never exceed it. Where
        // two slices would do, one 1024-thread workgroup per channel in one
        // launch is faster than the second launch (AlexNet conv2's 256
        // channels: 22.6 against 24.2 us).
        const int64_t floats = (int64_t)s.N * P;
        int64_t S0 = std::max<int64_t>(1, std::min<int64_t>((kTargetBlocks + s.K - 1) / s.K, floats / 8192));
        // One 1024-thread workgroup per channel (no second launch) where
        // that is faster by a model fitted on the box: a lone CU streams about
        // 36 GB/s, a split reduction about 5.5 TB/s plus a finalize launch of
        // about 4 us. 144 channels of 56 x 56 (or 28 x 28) take the single
        // pass (26.7 -> 24.5 us, 11.4 -> 9.7 us); 64 and 128 channels keep the
        // split (10.7 against 12.8 us, 22.4 against 23.7 us).
        if (S0 > 2) {
            const double bytes = (double)floats * 4.0;
            const double single = bytes / 36e9 * (double)((s.K + 255) / 256) + 1.5e-6;
            const double split = bytes * s.K / 5.5e12 + 4.7e-6;
            if (single < split) S0 = 1;
        } else {
            S0 = 1;
        }
        p.chunk = (int)((p.total + S0 - 1) / S0);
        p.S = (p.total + p.chunk - 1) / p.chunk;
        return p;
    }
    // [N, K] rows
    int cols_per_block;
    if ((s.K & 3) == 0 && ptr_aligned && s.K < 1024) {
        p.form = kRows;
        p.KT = rows_kt(s.K);
        cols_per_block = 4 * p.KT;
    } else if ((s.K & 3) == 0 && ptr_aligned) {
        p.form = kCols;
        cols_per_block = 4 * kB;
    } else {
        p.form = kColsScalar;
        cols_per_block = kB;
    }
    p.vec = p.form != kColsScalar;
    p.groups = (s.K + cols_per_block - 1) / cols_per_block;
    int S = (kTargetBlocks + p.groups - 1) / p.groups;
    S = std::max(1, std::min(S, std::max(1, s.N / 8)));  // at least 8 rows per slice
    p.rows_chunk = (s.N + S - 1) / S;
    p.S = (s.N + p.rows_chunk - 1) / p.rows_chunk;
    return p;
}

size_t plan_workspace(const Shape& s, const Plan& p)
{
    return p.S <= 1 ? 0 : (size_t)p.S * s.K * sizeof(float);
}

}  // namespace

size_t bias_workspace_bytes(const Shape& s)
{
    if (s.N == 0) return 0;
    // The plan depends on whether the pointers allow 16-byte loads; the
    // workspace covers both.
    const Plan a = make_plan(s, true), u = make_plan(s, false);
    return std::max(plan_workspace(s, a), plan_workspace(s, u));
}

void bias_reduce(const Shape& s, const float* dy, float* db, float* ws, hipStream_t st)
{
    const bool al = aligned16(dy) && aligned16(db) && aligned16(ws);
    Plan p = make_plan(s, al);
    BiasArgs a{};
    a.dy = dy;
    a.db = db;
    a.N = s.N; a.K = s.K; a.P = s.Ho * s.Wo; a.S = p.S;
    a.len = p.len; a.total = p.total; a.chunk = p.chunk;
    a.div_len = make_fastdiv((uint32_t)std::max(1, p.len));
    a.rows_chunk = p.rows_chunk; a.KT = p.KT;
    a.part = ws;
    switch (p.form) {
        case kPlanes:
            if (p.S == 1) {
                if (p.vec) hipLaunchKernelGGL((bias_planes<true, 1024>), dim3(1, s.K), dim3(1024), 0, st, a);
                else hipLaunchKernelGGL((bias_planes<false, 1024>), dim3(1, s.K), dim3(1024), 0, st, a);
            } else {
                if (p.vec) hipLaunchKernelGGL((bias_planes<true, kB>), dim3(p.S, s.K), dim3(kB), 0, st, a);
                else hipLaunchKernelGGL((bias_planes<false, kB>), dim3(p.S, s.K), dim3(kB), 0, st, a);
            }
            break;
        case kCols: hipLaunchKernelGGL(bias_cols, dim3(p.groups, p.S), dim3(kB), 0, st, a); break;
        case kRows: hipLaunchKernelGGL(bias_rows, dim3(p.groups, p.S), dim3(kB), 0, st, a); break;
        case kColsScalar: hipLaunchKernelGGL(bias_cols_scalar, dim3(p.groups, p.S), dim3(kB), 0, st, a); break;
    }
    if (p.S > 1) hipLaunchKernelGGL(bias_finalize, dim3((s.K + 15) / 16), dim3(kB), 0, st, ws, db, s.K, p.S);
}

}  // namespace gconv
