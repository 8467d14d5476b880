// bias.hip -- gradBias for grouped 2-D convolution, NCHW fp32:
//   db[k] = sum over n, ho, wo of dy[n, k, ho, wo]
// (a plain reduction of dy over everything but the channel: "Pointwise
// Broadcast/Reduce" on the dlprimitives blog, the bias-gradient formula).
// Deterministic throughout. Where each channel is small (at most 1 MiB of
// planes), one 1024-thread workgroup per channel sums it in one pass; the
// launch and finalize of a second pass cost more than the extra parallelism
// gains there. Otherwise two passes: split blocks write partial sums laid out
// [split][channel], then a second kernel adds each channel's splits in a
// fixed order (consecutive channels read consecutive partials).
//   plane layout (Ho*Wo > 1): block (s, k) sums images [s*chunk, (s+1)*chunk)
//     of plane k, with 16-byte loads when the plane length is a multiple of 4;
//   column layout (Ho*Wo == 1, dy is [N, K], fully-connected mode): block
//     (kb, s) sums rows [s*chunk, (s+1)*chunk) of 1024 columns (4 per thread);
//     narrower rows (NHWC gradients) take several rows per wave instead.
#include "device_util.h"
#include "fastdiv.h"
#include "gconv_internal.h"

namespace gconv {
namespace {

constexpr int kB = 256;

// Sum of v over the 256 threads; the total is returned to thread 0.
__device__ __forceinline__ float block_sum(float v, float* lds4)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) lds4[wave] = v;
    __syncthreads();
    float t = 0.f;
    if (threadIdx.x == 0) t = ((lds4[0] + lds4[1]) + lds4[2]) + lds4[3];
    return t;
}

template <bool VEC>
__global__ void __launch_bounds__(kB)
bias_planes_partial(const float* __restrict__ dy, float* __restrict__ ws, int N, int K, int P,
                    int chunk)
{
    __shared__ float lds4[4];
    const int sidx = blockIdx.x, k = blockIdx.y;
    const int n0 = sidx * chunk, n1 = min(N, n0 + chunk);
    float acc = 0.f;
    if constexpr (VEC) {
        const int P4 = P >> 2;
        f4 a4 = f4{0.f, 0.f, 0.f, 0.f};
        for (int n = n0; n < n1; ++n) {
            const f4* plane = reinterpret_cast<const f4*>(dy + ((int64_t)n * K + k) * P);
#pragma unroll 4
            for (int p = threadIdx.x; p < P4; p += kB) a4 += plane[p];
        }
        acc = (a4.x + a4.y) + (a4.z + a4.w);
    } else {
        for (int n = n0; n < n1; ++n) {
            const float* plane = dy + ((int64_t)n * K + k) * P;
#pragma unroll 4
            for (int p = threadIdx.x; p < P; p += kB) acc += plane[p];
        }
    }
    const float tot = block_sum(acc, lds4);
    if (threadIdx.x == 0) ws[(int64_t)sidx * K + k] = tot;
}

template <bool VEC>
__global__ void __launch_bounds__(kB)
bias_cols_partial(const float* __restrict__ dy, float* __restrict__ ws, int N, int K, int chunk)
{
    const int sidx = blockIdx.y;
    const int n0 = sidx * chunk, n1 = min(N, n0 + chunk);
    if constexpr (VEC) {
        const int k4 = blockIdx.x * kB + threadIdx.x;  // 4 columns per thread
        if (k4 * 4 >= K) return;
        f4 a = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int n = n0; n < n1; ++n) a += reinterpret_cast<const f4*>(dy + (int64_t)n * K)[k4];
        reinterpret_cast<f4*>(ws + (int64_t)sidx * K)[k4] = a;
    } else {
        const int k = blockIdx.x * kB + threadIdx.x;
        if (k >= K) return;
        float a = 0.f;
#pragma unroll 4
        for (int n = n0; n < n1; ++n) a += dy[(int64_t)n * K + k];
        ws[(int64_t)sidx * K + k] = a;
    }
}

// Column layout with narrow rows (dy is [rows, K] with K a multiple of 4 and
// fewer than 1024 columns: NHWC gradients): a block of 256 threads is KT
// column quads x (256 / KT) row phases, so a wave reads whole consecutive rows
// (KT = 16 for K = 64: four 256-byte rows per wave instruction). Thread (c, r)
// adds rows r0 + r, r0 + r + 256/KT, ... of its column quad; the row phases
// are then added in order through LDS, one partial per column and split.
__global__ void __launch_bounds__(kB)
bias_rows_partial(const float* __restrict__ dy, float* __restrict__ ws, int N, int K, int chunk, int KT)
{
    __shared__ f4 part[kB];
    const int sidx = blockIdx.y;
    const int n0 = sidx * chunk, n1 = min(N, n0 + chunk);
    const int K4 = K >> 2;
    const int ct = threadIdx.x % KT, rt = threadIdx.x / KT, RT = kB / KT;
    const int c4 = blockIdx.x * KT + ct;
    f4 a = f4{0.f, 0.f, 0.f, 0.f};
    if (c4 < K4) {
#pragma unroll 8
        for (int n = n0 + rt; n < n1; n += RT) a += reinterpret_cast<const f4*>(dy + (int64_t)n * K)[c4];
    }
    part[threadIdx.x] = a;
    __syncthreads();
    if (rt != 0 || c4 >= K4) return;
    f4 t = part[ct];
    for (int r = 1; r < RT; ++r) t += part[r * KT + ct];
    reinterpret_cast<f4*>(ws + (int64_t)sidx * K)[c4] = t;
}

// db[k] = sum over s of ws[s*K + k]. Block = 16 channels x 16 split groups:
// thread (kk, sg) adds splits sg, sg+16, ... in order, then the 16 group sums
// are added in order (deterministic; many partials per channel spread over
// the whole block instead of one thread).
__global__ void __launch_bounds__(kB)
bias_finalize(const float* __restrict__ ws, float* __restrict__ db, int K, int S)
{
    __shared__ float part[16][17];
    const int kk = threadIdx.x & 15, sg = threadIdx.x >> 4;
    const int k = blockIdx.x * 16 + kk;
    float acc = 0.f;
    if (k < K) {
#pragma unroll 4
        for (int s = sg; s < S; s += 16) acc += ws[(int64_t)s * K + k];
    }
    part[sg][kk] = acc;
    __syncthreads();
    if (sg != 0 || k >= K) return;
    float sum = part[0][kk];
#pragma unroll
    for (int i = 1; i < 16; ++i) sum += part[i][kk];
    db[k] = sum;
}

// One pass, one 1024-thread workgroup per channel (shapes where every channel
// is small enough for one CU): thread t sums elements t, t + 1024, ... of the
// channel's N planes taken as one sequence (eight independent loads in flight
// per thread), then the 16 wave sums are added in order. No partials, no
// second launch.
constexpr int kB1 = 1024;
template <bool VEC>
__global__ void __launch_bounds__(kB1)
bias_planes_single(const float* __restrict__ dy, float* __restrict__ db, int N, int K, int P, FastDiv div_len)
{
    __shared__ float red[16];
    const int k = blockIdx.x;
    const int len = VEC ? (P >> 2) : P;    // elements (f4 or float) per plane
    const int total = N * len;
    float acc = 0.f;
    f4 a4 = f4{0.f, 0.f, 0.f, 0.f};
    for (int i0 = threadIdx.x; i0 < total; i0 += 8 * kB1) {
        if constexpr (VEC) {
            f4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * kB1;
                v[u] = f4{0.f, 0.f, 0.f, 0.f};
                if (i < total) {
                    const int n = (int)fastdiv((uint32_t)i, div_len);
                    v[u] = reinterpret_cast<const f4*>(dy + ((int64_t)n * K + k) * P)[i - n * len];
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) a4 += v[u];
        } else {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * kB1;
                v[u] = 0.f;
                if (i < total) {
                    const int n = (int)fastdiv((uint32_t)i, div_len);
                    v[u] = dy[((int64_t)n * K + k) * P + (i - n * len)];
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += v[u];
        }
    }
    if constexpr (VEC) acc = (a4.x + a4.y) + (a4.z + a4.w);
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = red[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) t += red[i];
        db[k] = t;
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// The one-pass form: planes (Ho*Wo > 1), at most 1 MiB per channel, and
// either enough channels to occupy a quarter of the CUs or little data in all.
bool bias_single(const Shape& s)
{
#ifdef GCONV_BIAS_TWO_PASS
    return false;
#else
    const int64_t P = (int64_t)s.Ho * s.Wo;
    const int64_t per = (int64_t)s.N * P;  // floats per channel
    return P > 1 && per * 4 <= (int64_t(1) << 20) && (s.K >= 64 || per * s.K * 4 <= (int64_t(8) << 20));
#endif
}
bool cols_vec(const Shape& s) { return (s.K & 3) == 0; }

// Column quads per block of the narrow-row column kernel (a power of two up to
// 64); 0 when the rows are wide enough for one thread per column quad.
int rows_kt(const Shape& s)
{
    if (!cols_vec(s) || s.K >= 1024) return 0;
    int kt = 1;
    while (kt < 64 && kt < s.K / 4) kt *= 2;
    return kt;
}

// Splits: about 2048 partial blocks for the plane layout (whole images per
// block); about 1024 blocks of 1024 columns for the column layout.
int bias_splits(const Shape& s)
{
    const int P = s.Ho * s.Wo;
    int S;
    if (P == 1 && rows_kt(s) > 0) {
        // (512 blocks: 2048 left the finalize adding 128 partials per thread)
        const int kb = (s.K / 4 + rows_kt(s) - 1) / rows_kt(s);
        S = (512 + kb - 1) / kb;
    } else if (P == 1) {
        const int cpb = cols_vec(s) ? 4 * kB : kB;  // columns per block
        const int kb = (s.K + cpb - 1) / cpb;
        S = (512 + kb - 1) / kb;
    } else {
        S = (2048 + s.K - 1) / s.K;
    }
    if (S > s.N) S = s.N;
    if (S < 1) S = 1;
    return S;
}

}  // namespace

size_t bias_workspace_bytes(const Shape& s)
{
    if (s.N == 0 || bias_single(s)) return 0;
    return (size_t)s.K * (size_t)bias_splits(s) * sizeof(float);
}

void bias_reduce(const Shape& s, const float* dy, float* db, float* ws, hipStream_t st)
{
    const int P = s.Ho * s.Wo;
    if (bias_single(s)) {
        if ((P & 3) == 0 && aligned16(dy))
            hipLaunchKernelGGL(bias_planes_single<true>, dim3(s.K), dim3(kB1), 0, st, dy, db, s.N, s.K, P,
                               make_fastdiv((uint32_t)(P >> 2)));
        else
            hipLaunchKernelGGL(bias_planes_single<false>, dim3(s.K), dim3(kB1), 0, st, dy, db, s.N, s.K, P,
                               make_fastdiv((uint32_t)P));
        return;
    }
    const int S = bias_splits(s);
    const int chunk = (s.N + S - 1) / S;
    if (P == 1 && rows_kt(s) > 0 && aligned16(dy) && aligned16(ws)) {
        const int kt = rows_kt(s);
        hipLaunchKernelGGL(bias_rows_partial, dim3((s.K / 4 + kt - 1) / kt, S), dim3(kB), 0, st, dy, ws, s.N,
                           s.K, chunk, kt);
    } else if (P == 1) {
        // (the split count, hence the workspace size, does not depend on the
        // pointers: only the load width does)
        if (cols_vec(s) && aligned16(dy) && aligned16(ws))
            hipLaunchKernelGGL(bias_cols_partial<true>, dim3((s.K / 4 + kB - 1) / kB, S), dim3(kB),
                               0, st, dy, ws, s.N, s.K, chunk);
        else
            hipLaunchKernelGGL(bias_cols_partial<false>, dim3((s.K + kB - 1) / kB, S), dim3(kB), 0,
                               st, dy, ws, s.N, s.K, chunk);
    } else if ((P & 3) == 0 && aligned16(dy)) {
        hipLaunchKernelGGL(bias_planes_partial<true>, dim3(S, s.K), dim3(kB), 0, st, dy, ws, s.N,
                           s.K, P, chunk);
    } else {
        hipLaunchKernelGGL(bias_planes_partial<false>, dim3(S, s.K), dim3(kB), 0, st, dy, ws, s.N,
                           s.K, P, chunk);
    }
    hipLaunchKernelGGL(bias_finalize, dim3((s.K + 15) / 16), dim3(kB), 0, st, ws, db, s.K, S);
}

}  // namespace gconv
