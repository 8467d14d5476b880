/*
 * gconv_oracle.c -- plain, slow CPU reference for grouped 2-D convolution
 * in channels-first (NCHW) layout, accumulated in fp64.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The GPU library
 * shares no code, header or table with it, and must never call it.
 *
 * What it computes (the plain definition, written as gathers):
 *   - Groups: the C input planes and the K output planes are each cut into
 *     G contiguous blocks; output block g sees only input block g, so every
 *     filter has C/G planes and the weight holds K*(C/G) filter planes
 *     ("[Feature request] Groups support for SpatialConvolutionMM", the
 *     opening definition of groups and the per-group narrow() draft, whose
 *     plane offsets are groupPlane*(group-1)).
 *   - Cross-correlation (no kernel flip), zero padding, stride, dilation, the
 *     constructor order (nInputPlane, nOutputPlane, kW, kH, dW, dH, padW,
 *     padH, groups) of the same issue; flip-free because the kernel==input
 *     case must equal a Linear layer on the flattened input with the weight
 *     viewed as [K, C*kh*kw] ("SpatialConvolution running in fully-connected
 *     mode is very slow, even with R4", the View+Linear replacement).
 *   - Bias: added per output plane, bias[k] broadcast over (n, h, w); its
 *     gradient is the sum of dy over dims (0, 2, 3) (DLPrimitives Blog,
 *     "Pointwise Broadcast Reduce").
 *   - The four tensors of the module: output, gradInput, gradWeight,
 *     gradBias (the clnn issue's weight/bias/gradWeight/gradBias remark, and
 *     the four diffs of the cudnn.torch issue's MatConvNet comparison).
 *
 * Every result element also gets A_e, the sum of |product| over the terms
 * of its own reduction (plus |bias| in the forward pass). A_e scales the
 * rounding tolerance a float32 implementation is judged by.
 *
 * Parallelism: OpenMP over independent output elements only. Each element's
 * sum runs in the fixed loop order written below; nothing is blocked, fused
 * or reordered.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t N, C, H, W, K, kh, kw;
    int64_t stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, groups;
    /* Zero rows below the input and columns right of it. pad_h / pad_w are
     * the rows above and columns left of it, the only ones that shift the tap
     * coordinates below; the end padding only lengthens the output (the
     * DLPrimitives Blog, "TensorFlow": TensorFlow's "same" padding may differ
     * at the start and the end of an axis). */
    int64_t pad_h_end, pad_w_end;
} oracle_desc;

/* Output extent along one axis: floor((in + p0 + p1 - d(k-1) - 1) / s) + 1,
 * or 0 when the dilated kernel does not fit (a negative numerator). */
static int64_t out_extent(int64_t in, int64_t k, int64_t s, int64_t p0, int64_t p1, int64_t d)
{
    int64_t num = in + p0 + p1 - d * (k - 1) - 1;
    if (num < 0) return 0;
    return num / s + 1;
}

/* Returns 0 when the descriptor is valid, and fills Ho/Wo; nonzero otherwise.
 * An empty batch (N == 0) is valid: the outputs are empty, and the weight and
 * bias gradients are sums over no terms, i.e. 0. */
int oracle_output_dims(const oracle_desc* d, int64_t* Ho, int64_t* Wo)
{
    if (d->N < 0 || d->C < 1 || d->H < 1 || d->W < 1 || d->K < 1 || d->kh < 1 || d->kw < 1)
        return 1;
    if (d->stride_h < 1 || d->stride_w < 1 || d->dil_h < 1 || d->dil_w < 1) return 1;
    if (d->pad_h < 0 || d->pad_w < 0 || d->groups < 1) return 1;
    if (d->pad_h_end < 0 || d->pad_w_end < 0) return 1;
    if (d->C % d->groups != 0 || d->K % d->groups != 0) return 2;
    *Ho = out_extent(d->H, d->kh, d->stride_h, d->pad_h, d->pad_h_end, d->dil_h);
    *Wo = out_extent(d->W, d->kw, d->stride_w, d->pad_w, d->pad_w_end, d->dil_w);
    if (*Ho < 1 || *Wo < 1) return 1;
    return 0;
}

/* ---- forward: y[n,k,ho,wo] = b[k] + sum_{c,i,j} w[k,c,i,j] * x[n, g*Cg+c, h, w] ---- */
static void fwd_elem(const oracle_desc* d, int64_t Ho, int64_t Wo, const double* x,
                     const double* wt, const double* bias, int64_t e, double* val, double* mag)
{
    const int64_t Cg = d->C / d->groups, Kg = d->K / d->groups;
    const int64_t wo = e % Wo, ho = (e / Wo) % Ho, k = (e / (Wo * Ho)) % d->K,
                  n = e / (Wo * Ho * d->K);
    const int64_t g = k / Kg;
    double s = 0.0, a = 0.0;
    for (int64_t c = 0; c < Cg; ++c)
        for (int64_t i = 0; i < d->kh; ++i)
            for (int64_t j = 0; j < d->kw; ++j) {
                const int64_t h = ho * d->stride_h - d->pad_h + i * d->dil_h;
                const int64_t w = wo * d->stride_w - d->pad_w + j * d->dil_w;
                if (h < 0 || h >= d->H || w < 0 || w >= d->W) continue; /* zero padding */
                const double p = wt[((k * Cg + c) * d->kh + i) * d->kw + j] *
                                 x[((n * d->C + g * Cg + c) * d->H + h) * d->W + w];
                s += p;
                a += fabs(p);
            }
    if (bias) {
        s += bias[k];
        a += fabs(bias[k]);
    }
    *val = s;
    *mag = a;
}

/* ---- gradInput: dx[n, g*Cg+c, h, w] = sum over the taps that read (h, w) ----
 * A tap (k, i, j) of output (ho, wo) reads input row ho*sh - ph + i*dh; so the
 * output rows that read h are ho = (h + ph - i*dh) / sh where that division is
 * exact and 0 <= ho < Ho (likewise for columns). */
static void bwd_data_elem(const oracle_desc* d, int64_t Ho, int64_t Wo, const double* dy,
                          const double* wt, int64_t e, double* val, double* mag)
{
    const int64_t Cg = d->C / d->groups, Kg = d->K / d->groups;
    const int64_t w = e % d->W, h = (e / d->W) % d->H, ca = (e / (d->W * d->H)) % d->C,
                  n = e / (d->W * d->H * d->C);
    const int64_t g = ca / Cg, c = ca % Cg;
    double s = 0.0, a = 0.0;
    for (int64_t k = g * Kg; k < (g + 1) * Kg; ++k)
        for (int64_t i = 0; i < d->kh; ++i)
            for (int64_t j = 0; j < d->kw; ++j) {
                const int64_t th = h + d->pad_h - i * d->dil_h;
                const int64_t tw = w + d->pad_w - j * d->dil_w;
                if (th < 0 || tw < 0) continue;
                if (th % d->stride_h != 0 || tw % d->stride_w != 0) continue;
                const int64_t ho = th / d->stride_h, wo = tw / d->stride_w;
                if (ho >= Ho || wo >= Wo) continue;
                const double p = wt[((k * Cg + c) * d->kh + i) * d->kw + j] *
                                 dy[((n * d->K + k) * Ho + ho) * Wo + wo];
                s += p;
                a += fabs(p);
            }
    *val = s;
    *mag = a;
}

/* ---- gradWeight: dw[k,c,i,j] = sum_{n,ho,wo} dy[n,k,ho,wo] * x[n, g*Cg+c, h, w] ---- */
static void bwd_filter_elem(const oracle_desc* d, int64_t Ho, int64_t Wo, const double* x,
                            const double* dy, int64_t e, double* val, double* mag)
{
    const int64_t Cg = d->C / d->groups, Kg = d->K / d->groups;
    const int64_t j = e % d->kw, i = (e / d->kw) % d->kh, c = (e / (d->kw * d->kh)) % Cg,
                  k = e / (d->kw * d->kh * Cg);
    const int64_t g = k / Kg;
    double s = 0.0, a = 0.0;
    for (int64_t n = 0; n < d->N; ++n)
        for (int64_t ho = 0; ho < Ho; ++ho)
            for (int64_t wo = 0; wo < Wo; ++wo) {
                const int64_t h = ho * d->stride_h - d->pad_h + i * d->dil_h;
                const int64_t w = wo * d->stride_w - d->pad_w + j * d->dil_w;
                if (h < 0 || h >= d->H || w < 0 || w >= d->W) continue;
                const double p = dy[((n * d->K + k) * Ho + ho) * Wo + wo] *
                                 x[((n * d->C + g * Cg + c) * d->H + h) * d->W + w];
                s += p;
                a += fabs(p);
            }
    *val = s;
    *mag = a;
}

/* ---- gradBias: db[k] = sum_{n,ho,wo} dy[n,k,ho,wo] ---- */
static void bwd_bias_elem(const oracle_desc* d, int64_t Ho, int64_t Wo, const double* dy,
                          int64_t k, double* val, double* mag)
{
    double s = 0.0, a = 0.0;
    for (int64_t n = 0; n < d->N; ++n)
        for (int64_t ho = 0; ho < Ho; ++ho)
            for (int64_t wo = 0; wo < Wo; ++wo) {
                const double v = dy[((n * d->K + k) * Ho + ho) * Wo + wo];
                s += v;
                a += fabs(v);
            }
    *val = s;
    *mag = a;
}

/*
 * Entry points. `idx` lists the flat (row-major) indices of the result
 * elements to compute; when `idx` is NULL, all `count` elements 0..count-1
 * are computed. `val[t]` and `mag[t]` receive the value and A_e of element
 * idx[t]. Return 0 on success, 1 on an invalid descriptor, 3 when an index
 * lies outside the result tensor (those slots are left untouched).
 */
int oracle_fwd(const oracle_desc* d, const double* x, const double* wt, const double* bias,
               const int64_t* idx, int64_t count, double* val, double* mag)
{
    int64_t Ho, Wo;
    int bad = 0;
    if (oracle_output_dims(d, &Ho, &Wo) != 0) return 1;
    const int64_t total = d->N * d->K * Ho * Wo;
#pragma omp parallel for schedule(dynamic, 64) reduction(| : bad)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t e = idx ? idx[t] : t;
        if (e < 0 || e >= total) { bad |= 1; continue; }
        fwd_elem(d, Ho, Wo, x, wt, bias, e, &val[t], &mag[t]);
    }
    return bad ? 3 : 0;
}

int oracle_bwd_data(const oracle_desc* d, const double* dy, const double* wt,
                    const int64_t* idx, int64_t count, double* val, double* mag)
{
    int64_t Ho, Wo;
    int bad = 0;
    if (oracle_output_dims(d, &Ho, &Wo) != 0) return 1;
    const int64_t total = d->N * d->C * d->H * d->W;
#pragma omp parallel for schedule(dynamic, 64) reduction(| : bad)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t e = idx ? idx[t] : t;
        if (e < 0 || e >= total) { bad |= 1; continue; }
        bwd_data_elem(d, Ho, Wo, dy, wt, e, &val[t], &mag[t]);
    }
    return bad ? 3 : 0;
}

int oracle_bwd_filter(const oracle_desc* d, const double* x, const double* dy,
                      const int64_t* idx, int64_t count, double* val, double* mag)
{
    int64_t Ho, Wo;
    int bad = 0;
    if (oracle_output_dims(d, &Ho, &Wo) != 0) return 1;
    const int64_t total = d->K * (d->C / d->groups) * d->kh * d->kw;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t e = idx ? idx[t] : t;
        if (e < 0 || e >= total) { bad |= 1; continue; }
        bwd_filter_elem(d, Ho, Wo, x, dy, e, &val[t], &mag[t]);
    }
    return bad ? 3 : 0;
}

int oracle_bwd_bias(const oracle_desc* d, const double* dy, const int64_t* idx, int64_t count,
                    double* val, double* mag)
{
    int64_t Ho, Wo;
    int bad = 0;
    if (oracle_output_dims(d, &Ho, &Wo) != 0) return 1;
    const int64_t total = d->K;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t e = idx ? idx[t] : t;
        if (e < 0 || e >= total) { bad |= 1; continue; }
        bwd_bias_elem(d, Ho, Wo, dy, e, &val[t], &mag[t]);
    }
    return bad ? 3 : 0;
}

/* Number of OpenMP threads the entry points above will use. */
int oracle_num_threads(void)
{
    int n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}
