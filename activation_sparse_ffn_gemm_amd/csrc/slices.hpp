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
// When a row is eight whole runs of 128-byte lines (ndw a multiple of 256
// words: d_model % 512 == 0 in bf16, % 256 in f32), a slice already is one
// run of whole lines in place ("direct"), and the forward's down pass reads
// wd as stored: no copy is made.
#pragma once

#include "common.hpp"
#include "rows.hpp"

struct Slices {
    int ndw, sww, swp;
    bool direct;
    DEVI int valid(int k) const { return max(0, min(sww, ndw - k * sww)); }
};

inline Slices slices(int dt, int dm)
{
    Slices s;
    s.ndw = dt == TWELL_BF16 ? dm / 2 : dm;
    s.sww = (s.ndw + NXCD - 1) / NXCD;
    s.swp = (s.sww + 31) / 32 * 32;
    s.direct = s.ndw % (NXCD * 32) == 0;
    return s;
}

// Where a pass finds slice k of row c of one or two matrices: row c of slice
// k of matrix a starts at word a + k kstride + c rowb / 4 (b likewise), and a
// lane's word offsets within it are clamped to [0, lim).
struct SliceSrc {
    const uint32_t *a, *b;
    size_t kstride;
    int rowb, lim;
};

// the weights as stored (Slices::direct)
inline SliceSrc slice_src_direct(const void *a, const void *b, const Slices &sl)
{
    return SliceSrc{(const uint32_t *)a, (const uint32_t *)b, (size_t)sl.sww, sl.ndw * 4, sl.sww};
}

// a slice-major copy of NSRC matrices (copy_slices_rows)
inline SliceSrc slice_src_copy(const uint32_t *w, int nsrc, int dff, const Slices &sl)
{
    return SliceSrc{w, w + sl.swp, (size_t)dff * nsrc * sl.swp, nsrc * sl.swp * 4, sl.swp};
}

// Bytes of a slice-major copy of NSRC matrices (0 when the slices are read in place)
inline size_t slice_copy_bytes(int nsrc, int dff, const Slices &sl)
{
    return sl.direct ? 0 : (size_t)NXCD * dff * nsrc * sl.swp * 4;
}

// Buffer descriptor over rows 0 .. dff - 1 of one matrix's slice k, from
// its base (range: the last row's lim words; loads past it read 0)
DEVI __amdgpu_buffer_rsrc_t slice_rsrc(const uint32_t *base, int dff, const SliceSrc &s)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0,
                                             (dff - 1) * s.rowb + s.lim * 4, BUF_DWORD3);
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
