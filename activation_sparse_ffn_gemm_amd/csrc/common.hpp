// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "twell.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

#define DEVI __device__ __forceinline__

// bfloat16 <-> float32. A bf16 is the high half of a float32, so widening is a
// shift; narrowing rounds to nearest, ties to even (quiet NaN kept quiet).
DEVI float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
DEVI float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
DEVI float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
DEVI uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Element type traits: how many elements a 16-byte chunk holds and how to widen.
template <int DT> struct elem;
template <> struct elem<TWELL_BF16> {
    typedef uint16_t storage;
    static constexpr int per16 = 8;
    DEVI static void widen(const uint4 &v, float *o)
    {
        o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
        o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
    }
    DEVI static float load1(const void *p, size_t i) { return bf16_to_f32(((const uint16_t *)p)[i]); }
    DEVI static void store1(void *p, size_t i, float v) { ((uint16_t *)p)[i] = f32_to_bf16(v); }
};
template <> struct elem<TWELL_F32> {
    typedef float storage;
    static constexpr int per16 = 4;
    DEVI static void widen(const uint4 &v, float *o)
    {
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    }
    DEVI static float load1(const void *p, size_t i) { return ((const float *)p)[i]; }
    DEVI static void store1(void *p, size_t i, float v) { ((float *)p)[i] = v; }
};

DEVI uint4 ldg16(const void *p) { return *(const uint4 *)p; }

// Sum over the 64 lanes of a wavefront; every lane gets the total.
DEVI float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

DEVI int wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int n = __shfl_up(v, o, 64);
        if (lane >= o)
            v += n;
    }
    return v;
}

DEVI uint32_t lanemask_lt32(int lane32) { return (1u << lane32) - 1u; }

DEVI void raise_status(int32_t *status, int bits)
{
    if (status)
        atomicOr(status, bits);
}

// Host-side launch helpers (defined in api.hip).
int twell_launch_check();
