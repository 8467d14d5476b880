// layout.hip -- reordering between channels-last (NHWC) and channels-first
// (NCHW) activations: for each of N images, the [R][Cc] matrix of R pixels by
// Cc channels becomes [Cc][R], or back. The gconv_layout NHWC ops run the
// NCHW kernels between such reorderings (the DLPrimitives Blog measures the
// same 3x3 layer in both layouts; TensorFlow's channels-last tensors are the
// common NHWC source).
//
// A 256-thread workgroup moves one 64 x 64 tile through LDS: it reads 64
// source rows of 64 consecutive floats (each wave a whole 256-byte row per
// instruction) and writes 64 destination rows the same way, so both sides
// are coalesced. The LDS tile has a 65-float row pitch, so the column reads
// of the write phase fall in distinct banks. HBM-bound: each float is read
// once and written once.
#include "device_util.h"
#include "gconv_internal.h"

namespace gconv {
namespace {

constexpr int kT = 64;

// dst[n][c][r] = src[n][r][c] for r < R, c < Cc.
__global__ void __launch_bounds__(256) transpose_tiles(const float* __restrict__ src, float* __restrict__ dst,
                                                       int R, int Cc, int tiles_r, int tiles_c)
{
    __shared__ float tile[kT][kT + 1];
    int bid = blockIdx.x;
    const int tc = bid % tiles_c;
    bid /= tiles_c;
    const int tr = bid % tiles_r;
    const int n = bid / tiles_r;
    const size_t img = (size_t)n * R * Cc;
    const float* s = src + img;
    float* d = dst + img;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = tr * kT, c0 = tc * kT;
    // Read: wave w takes source rows w, w + 4, ...; lane = column.
    const int c = c0 + lane;
    for (int i = wave; i < kT; i += 4) {
        const int r = r0 + i;
        if (r < R && c < Cc) tile[i][lane] = s[(size_t)r * Cc + c];
    }
    __syncthreads();
    // Write: wave w takes destination rows (source columns) w, w + 4, ...;
    // lane = source row.
    const int r = r0 + lane;
    for (int i = wave; i < kT; i += 4) {
        const int cc = c0 + i;
        if (cc < Cc && r < R) d[(size_t)cc * R + r] = tile[lane][i];
    }
}

}  // namespace

bool transpose_batched(const float* src, float* dst, int64_t N, int64_t R, int64_t Cc, hipStream_t st)
{
    if (N == 0 || R == 0 || Cc == 0) return true;
    if (R >= (int64_t(1) << 30) || Cc >= (int64_t(1) << 30)) return false;
    const int64_t tiles_r = (R + kT - 1) / kT, tiles_c = (Cc + kT - 1) / kT;
    const int64_t blocks = N * tiles_r * tiles_c;
    if (blocks >= (int64_t(1) << 31)) return false;
    hipLaunchKernelGGL(transpose_tiles, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, (int)R, (int)Cc,
                       (int)tiles_r, (int)tiles_c);
    return true;
}

}  // namespace gconv
