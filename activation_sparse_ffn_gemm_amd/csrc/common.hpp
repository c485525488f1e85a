// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <climits>
#include <stddef.h>
#include <stdint.h>

#include "twell.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
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
// The same rounding (nearest, ties to even) by gfx950's conversion
// instruction, two values at once: low half a, high half b. NaN inputs are
// not supported by the layer and may come out with another quiet payload.
DEVI uint32_t f32x2_to_bf16x2(float a, float b)
{
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
// hi = bf16(v), lo = bf16(v - hi): the bf16 pair carrying v to about 16
// significant bits, as (hi, lo) in the low and high halves
DEVI uint32_t f32_to_bf16_hilo(float v)
{
    const __bf16 hi = (__bf16)v;
    const bf16x2_t p = {hi, (__bf16)(v - (float)hi)};
    return __builtin_bit_cast(uint32_t, p);
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
// Within each row of 16 lanes the sum is formed with DPP lane moves (no LDS
// traffic): swap neighbours (quad_perm 1,0,3,2), swap pairs (2,3,0,1), mirror
// each half-row, mirror the row. Every lane then holds its row's sum; the four
// row sums are read into scalar registers and added in a fixed order.
template <int CTRL> DEVI float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
DEVI float wave_sum(float v)
{
    v += dpp_mov<0xB1>(v);  // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);  // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v); // row_half_mirror
    v += dpp_mov<0x140>(v); // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
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

// This wave's index in its workgroup, as a scalar: values derived from it
// (a token or row per wave, its row pointers) then live in scalar registers.
DEVI int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Broadcast lane `src` (wave-uniform) of v to every lane, through a scalar register.
DEVI int bcast(int v, int src) { return __builtin_amdgcn_readlane(v, src); }
DEVI float bcast(float v, int src)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

DEVI void raise_status(int32_t *status, int bits)
{
    if (status)
        atomicOr(status, bits);
}

// MI355X has 8 XCDs, each with its own L2, and hands consecutive workgroup
// ids to the XCDs in turn: workgroup b runs on XCD b % 8.
constexpr int NXCD = 8;

// ---- optional kernel timing of one API call (see twell_timing_t)
struct Timer {
    twell_timing_t *t;
    hipStream_t s;
    Timer(twell_timing_t *t_, hipStream_t s_) : t(t_), s(s_)
    {
        if (t) {
            t->n_used = 0;
            if (t->n_events > 0 && hipEventRecord((hipEvent_t)t->events[0], s) == hipSuccess)
                t->n_used = 1;
        }
    }
    void mark(const char *name)
    {
        if (!t || t->n_used <= 0 || t->n_used >= t->n_events || t->n_used > TWELL_TIMING_MAX)
            return;
        t->names[t->n_used - 1] = name;
        if (hipEventRecord((hipEvent_t)t->events[t->n_used], s) == hipSuccess)
            ++t->n_used;
    }
};
