// device_util.h -- small device helpers shared by the HIP kernels of the
// grouped-convolution library (gfx950): raw buffer resources, loads through
// them (to registers, or straight into LDS) and the XCD-aware block order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gconv {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// A byte offset at or past a resource's size reads 0 without touching memory;
// sizes stay below 2^31 and kOOB is past every one of them.
constexpr uint32_t kOOB = 0x80000000u;

// Raw buffer resource over [p, p + bytes). Every caller passes a wave-uniform
// base and size; readfirstlane states that, so the resource lives in scalar
// registers (a resource the compiler takes for divergent makes it wrap each
// load in a loop over the lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes)
{
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    void* up = (void*)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(up, (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// 32-bit raw buffer load of a float (the builtin returns the bits as an integer).
__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// 32-bit raw buffer store of a float; out-of-range offsets are dropped.
__device__ __forceinline__ void store_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_off, 0, 0);
}

// The 64 lanes load one dword each into 64 consecutive LDS floats at `dst`
// (wave-uniform); out-of-range offsets write 0.
__device__ __forceinline__ void load_lds64(__amdgpu_buffer_rsrc_t r, float* dst, uint32_t byte_off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, byte_off, 0, 0, 0);
}

// As load_lds64 with a wave-uniform byte offset `soff` added to every lane's
// `byte_off` (an SGPR operand: advancing a stream of loads by a uniform step
// costs no vector instruction). Lanes given kOOB still read 0.
__device__ __forceinline__ void load_lds64s(__amdgpu_buffer_rsrc_t r, float* dst, uint32_t byte_off, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, byte_off, (int)soff, 0, 0);
}

// The 64 lanes load 16 bytes each into 256 consecutive LDS floats at `dst`
// (lane i to dst + 4i; wave-uniform `dst`); out-of-range offsets write 0.
__device__ __forceinline__ void load_lds256(__amdgpu_buffer_rsrc_t r, float* dst, uint32_t byte_off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, byte_off, 0, 0, 0);
}

// Workgroups are dispatched round-robin over the 8 XCDs of the MI355X (block b
// runs on XCD b % 8). Renumber so that each XCD gets a contiguous range of
// logical tiles: neighbouring tiles then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int nb)
{
    const int per = nb >> 3, rem = nb & 7, x = b & 7, i = b >> 3;
    return x * per + min(x, rem) + i;
}

}  // namespace gconv
