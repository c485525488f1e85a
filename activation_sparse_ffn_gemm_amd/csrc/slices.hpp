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
// b) into the slice-major array dst (padding words set to 0), 16 bytes per
// lane: with d_model % 64 == 0, ndw, sww and swp are multiples of 4 words, so
// a 4-word group is wholly inside or wholly outside a slice.
template <int NSRC, int NTH>
DEVI void copy_slices_rows(int b, const uint32_t *__restrict__ a, const uint32_t *__restrict__ bm,
                           uint32_t *__restrict__ dst, int dff, Slices sl)
{
    const int sw4 = sl.swp / 4, ss4 = sl.sww / 4, nd4 = sl.ndw / 4;
    const int rw = NSRC * sw4; // 4-word groups of one row of one slice
    const int per = NXCD * rw;
    const int nq = min(RL_ROWS, dff - b * RL_ROWS) * per;
    constexpr int U = 4; // independent loads in flight per thread
    for (int q0 = threadIdx.x; q0 < nq; q0 += U * NTH) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = min(q0 + u * NTH, nq - 1);
            const int i = b * RL_ROWS + q / per;
            const int k = (q % per) / rw, r = q % rw, m = r / sw4, w = r % sw4;
            const int src4 = k * ss4 + w;
            const uint32_t *src = m == 0 ? a : bm;
            v[u] = *(const uint4 *)(src + ((size_t)i * nd4 + min(src4, nd4 - 1)) * 4);
            if (w >= ss4 || src4 >= nd4)
                v[u] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + u * NTH;
            if (q < nq) {
                const int i = b * RL_ROWS + q / per;
                const int k = (q % per) / rw, r = q % rw;
                *(uint4 *)(dst + (((size_t)k * dff + i) * rw + r) * 4) = v[u];
            }
        }
    }
}
