// Whole d_model rows held across a wave64, read with 4-byte lanes.
//
// A row of d_model elements is ndw 4-byte words (two bf16 or one f32 each).
// Lane l of a wave owns words base + c * 64 + l, c < NW, of a part of the row
// (part p starts at word p * NW * 64). A wave instruction then reads 256
// contiguous bytes of the row; gathering random rows this way runs about three
// times faster on MI355X than with 16-byte lanes (measured), because more
// independent requests are in flight per byte.
#pragma once

#include "common.hpp"

constexpr int ACC_NW = 8; // words per lane in kernels that hold a row of accumulators

// Fourth word of a raw buffer descriptor on gfx9-family parts: 32-bit data
// format (needed for the range check of untyped loads), everything else 0.
constexpr int BUF_DWORD3 = 0x00020000;

template <int DT, int NW> struct Row {
    static constexpr int EPW = DT == TWELL_BF16 ? 2 : 1; // elements per word
    int ndw, base, lane;

    DEVI Row(int dm, int lane_, int part)
        : ndw(DT == TWELL_BF16 ? dm / 2 : dm), base(part * NW * 64), lane(lane_) {}

    DEVI bool in(int c) const { return base + c * 64 + lane < ndw; }
    DEVI int word(int c) const { return base + c * 64 + lane; }

    // Words of row r of a [rows][d_model] matrix. The row index must be the
    // same in every lane: the loads go through a buffer descriptor built in
    // scalar registers for this row (and part), so every load needs only the
    // lane's byte offset plus an immediate, and lanes past the end of the row
    // read 0 from the descriptor's range check (no branches, no clamping).
    DEVI void load_w(const uint8_t *m, int r, uint32_t (&w)[NW]) const
    {
        const size_t row = (size_t)__builtin_amdgcn_readfirstlane(r) * ndw + base;
        const int bytes = ndw > base ? (ndw - base) * 4 : 0;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(m + row * 4), (short)0, bytes, BUF_DWORD3);
        // the lane's byte offset is redefined here (an empty asm, no code), so
        // that it is not hoisted out of a caller's loop: each load then folds
        // c * 256 into its immediate offset instead of holding NW offsets in
        // vector registers across the loop
        int off = lane * 4;
        asm volatile("" : "+v"(off));
#pragma unroll
        for (int c = 0; c < NW; ++c)
            w[c] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + c * 256, 0, 0);
    }

    DEVI void widen(uint32_t w, float (&f)[EPW]) const
    {
        if constexpr (EPW == 2) {
            f[0] = bf16_lo(w);
            f[1] = bf16_hi(w);
        } else {
            f[0] = __uint_as_float(w);
        }
    }

    DEVI void load_f(const uint8_t *m, int r, float (&f)[NW][EPW]) const
    {
        uint32_t w[NW];
        load_w(m, r, w);
#pragma unroll
        for (int c = 0; c < NW; ++c)
            widen(w[c], f[c]);
    }

    DEVI void zero_f(float (&f)[NW][EPW]) const
    {
#pragma unroll
        for (int c = 0; c < NW; ++c)
#pragma unroll
            for (int e = 0; e < EPW; ++e)
                f[c][e] = 0.f;
    }

    // this lane's share of the dot product of a float row with a stored row
    DEVI float dot(const float (&f)[NW][EPW], const uint32_t (&w)[NW]) const
    {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < NW; ++c) {
            float v[EPW];
            widen(w[c], v);
#pragma unroll
            for (int e = 0; e < EPW; ++e)
                s += f[c][e] * v[e];
        }
        return s;
    }

    // this lane's share of the dot product of two stored rows (bf16 words go
    // through the two-way bf16 dot instruction with float32 accumulation)
    DEVI float dotw(const uint32_t (&a)[NW], const uint32_t (&b)[NW]) const
    {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < NW; ++c) {
            if constexpr (EPW == 2)
                s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a[c]),
                                                    __builtin_bit_cast(bf16x2_t, b[c]), s, false);
            else
                s += __uint_as_float(a[c]) * __uint_as_float(b[c]);
        }
        return s;
    }

    // acc += a * (stored row)
    DEVI void axpy(float (&acc)[NW][EPW], float a, const uint32_t (&w)[NW]) const
    {
#pragma unroll
        for (int c = 0; c < NW; ++c) {
            float v[EPW];
            widen(w[c], v);
#pragma unroll
            for (int e = 0; e < EPW; ++e)
                acc[c][e] += a * v[e];
        }
    }

    // row r of a [rows][d_model] float32 matrix += f: every word's current
    // value is requested before any is added
    DEVI void add_store_f(float *y, int r, const float (&f)[NW][EPW]) const
    {
        float *p = y + (size_t)r * ndw * EPW;
        float cur[NW][EPW];
#pragma unroll
        for (int c = 0; c < NW; ++c) {
            const int w = in(c) ? word(c) : 0;
            if constexpr (EPW == 2) {
                const float2 v = *(const float2 *)(p + (size_t)w * 2);
                cur[c][0] = v.x;
                cur[c][1] = v.y;
            } else {
                cur[c][0] = p[w];
            }
        }
#pragma unroll
        for (int c = 0; c < NW; ++c) {
            if (!in(c))
                continue;
            if constexpr (EPW == 2)
                *(float2 *)(p + (size_t)word(c) * 2) =
                    make_float2(cur[c][0] + f[c][0], cur[c][1] + f[c][1]);
            else
                p[word(c)] = cur[c][0] + f[c][0];
        }
    }

    // row r of a [rows][d_model] float32 matrix
    DEVI void store_f(float *y, int r, const float (&f)[NW][EPW]) const
    {
        float *p = y + (size_t)r * ndw * EPW;
#pragma unroll
        for (int c = 0; c < NW; ++c) {
            if (!in(c))
                continue;
            if constexpr (EPW == 2)
                *(float2 *)(p + (size_t)word(c) * 2) = make_float2(f[c][0], f[c][1]);
            else
                p[word(c)] = f[c][0];
        }
    }
};

// Words per lane covering a whole row, rounded up to a power of two.
template <int DT> inline int row_nw(int dm)
{
    const int ndw = DT == TWELL_BF16 ? dm / 2 : dm;
    const int nw = (ndw + 63) / 64;
    int p = 1;
    while (p < nw)
        p <<= 1;
    return p;
}

// Number of parts of nwp words per lane that cover a row.
template <int DT> inline int row_parts(int dm, int nwp)
{
    const int ndw = DT == TWELL_BF16 ? dm / 2 : dm;
    return (ndw + nwp * 64 - 1) / (nwp * 64);
}
