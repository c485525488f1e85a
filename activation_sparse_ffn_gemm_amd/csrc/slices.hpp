// Slice-major copies of weight rows for the two-pass (XCD-local) gathers.
//
// MI355X hands workgroup b to XCD b % 8, and each XCD has its own 4 MB L2.
// A pass whose XCD k reads only the k-th eighth of every weight row (its
// "slice") keeps an eighth of the weights in each L2 instead of all of them
// everywhere. The slices are copied into their own arrays first so that a
// gathered row's slice is one run of whole 128-byte lines:
//   slice k holds words [k sww, k sww + sww) of every row (fewer in the last
//   slices), each row's slice padded to swp words (a multiple of 32).
// With NSRC = 2 two matrices are interleaved per row: row i of slice k holds
// the first matrix's slice, then the second's (2 swp words).
#pragma once

#include "common.hpp"

struct Slices {
    int ndw, sww, swp;
    DEVI int valid(int k) const { return max(0, min(sww, ndw - k * sww)); }
};

inline Slices slices(int dt, int dm)
{
    Slices s;
    s.ndw = dt == TWELL_BF16 ? dm / 2 : dm;
    s.sww = (s.ndw + NXCD - 1) / NXCD;
    s.swp = (s.sww + 31) / 32 * 32;
    return s;
}

constexpr int RL_ROWS = 8; // weight rows per workgroup of the copy

// Workgroups needed for the copy (a multiple of 8, so that the workgroups
// after them keep b % 8 as their XCD)
inline int copy_groups(int dff) { return ((dff + RL_ROWS - 1) / RL_ROWS + NXCD - 1) / NXCD * NXCD; }

// Workgroup b of NTH threads copies rows [b RL_ROWS, (b+1) RL_ROWS) of a (and
// b) into the slice-major array dst (padding words set to 0).
template <int NSRC, int NTH>
DEVI void copy_slices_rows(int b, const uint32_t *__restrict__ a, const uint32_t *__restrict__ bm,
                           uint32_t *__restrict__ dst, int dff, Slices sl)
{
    const int rw = NSRC * sl.swp; // words of one row of one slice
    const int per = NXCD * rw;
    for (int q = threadIdx.x; q < RL_ROWS * per; q += NTH) {
        const int i = b * RL_ROWS + q / per;
        if (i >= dff)
            break;
        const int k = (q % per) / rw, r = q % rw, m = r / sl.swp, w = r % sl.swp;
        const int srcw = k * sl.sww + w;
        const uint32_t *src = m == 0 ? a : bm;
        const uint32_t v = src[(size_t)i * sl.ndw + min(srcw, sl.ndw - 1)];
        dst[((size_t)k * dff + i) * rw + r] = (w < sl.sww && srcw < sl.ndw) ? v : 0u;
    }
}
