// fastdiv.h -- division of non-negative 32-bit integers (< 2^31) by a runtime
// divisor fixed for a whole launch, as a multiply-high, an add and a shift
// (the round-up method of Granlund & Montgomery, "Division by invariant
// integers using multiplication", 1994). The host computes the magic once.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#include <hip/hip_runtime.h>
#define GCONV_HD __host__ __device__
#else
#define GCONV_HD
#endif

namespace gconv {

struct FastDiv {
    uint32_t d;  // divisor (>= 1)
    uint32_t m;  // magic multiplier
    uint32_t s;  // shift
};

// Host: magic for divisor d >= 1. With s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1, q = (umulhi(n, m) + n) >> s equals n / d
// for every 0 <= n < 2^31 (the sum stays below 2^32 there).
inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t s = 0;
    while ((uint64_t(1) << s) < d) ++s;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, s};
}

GCONV_HD inline uint32_t fastdiv(uint32_t n, const FastDiv& f)
{
#ifdef __HIP_DEVICE_COMPILE__
    const uint32_t t = __umulhi(n, f.m);
#else
    const uint32_t t = (uint32_t)(((uint64_t)n * f.m) >> 32);
#endif
    return (t + n) >> f.s;
}

}  // namespace gconv
