// Host interface of the dense products over the hybrid's backup rows
// (backup.hip), and the device helper that finishes them: the split-K
// partials of y_O / dx_O are summed, in split order, by the ELL row kernels.
#pragma once

#include "common.hpp"

// Float32 partials part[S][R][d_model] of the backup rows' y_O or dx_O
// (part == nullptr: the hybrid has no backup capacity).
struct BkPart {
    const float *part;
    int S, R;
};

size_t bk_workspace(int dt, int dm, int dff, int max_ovf, bool bwd);
BkPart bk_part(int dt, int dm, int dff, int max_ovf, bool bwd, const void *ws);
// The forward's backup products (A, then the split-K partials of y_O); with
// out_rows, a third launch sums each backup row's partials into its y row
// (otherwise the ELL rows' kernel does, through bk_finish_row).
void launch_bk_fwd(twell_dtype dt, const void *x, const hybrid_t *h, const void *wu,
                   const void *wd, int dm, float *y, void *ws, bool out_rows, Timer &tm,
                   hipStream_t s);

// The backward's products run as extra workgroups of the ELL passes' launches
// (bwd.hip; device side in backup_tiles.hpp): their operands in the
// workspace, and their workgroup counts (all zero without backup capacity).
struct BkBwd {
    uint8_t *inter; // a, du, dg: [3][NH][R][d_ff] (NH = 2 halves hi, lo for bf16)
    uint8_t *xo;    // x_O, dy_O: [2][R][d_model]
    float *part;    // split-K partials of dx_O: [S][R][d_model]
    int R, S;
    int n_ud, n_dx, n_dw; // u/da tiles, dx_O tiles, dW tiles
};
BkBwd bk_bwd(int dt, int dm, int dff, int max_ovf, void *ws);

// Row `slot` of the backup: words [base, min(base + 64 NW, end, ndw)) of a
// d_model row (EPW floats each, lane l owning words base + 64 c + l) of sum
// over s of part[s][slot] into out_row. The S loads of a word go out together.
template <int NW, int EPW>
DEVI void bk_finish_row(const BkPart &bp, int slot, int ndw, int base, int end, int lane,
                        float *out_row)
{
    const size_t stride = (size_t)bp.R * ndw * EPW;
    const float *src = bp.part + (size_t)slot * ndw * EPW;
#pragma unroll
    for (int c = 0; c < NW; ++c) {
        const int w = base + c * 64 + lane;
        if (w >= ndw || w >= end)
            continue;
        float acc[EPW];
#pragma unroll
        for (int e = 0; e < EPW; ++e)
            acc[e] = 0.f;
        for (int s0 = 0; s0 < bp.S; s0 += 8) {
            float v[8][EPW];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const size_t o = (size_t)min(s0 + u, bp.S - 1) * stride + (size_t)w * EPW;
                if constexpr (EPW == 2) {
                    const float2 f = *(const float2 *)(src + o);
                    v[u][0] = f.x;
                    v[u][1] = f.y;
                } else {
                    v[u][0] = src[o];
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < bp.S)
#pragma unroll
                    for (int e = 0; e < EPW; ++e)
                        acc[e] += v[u][e];
        }
        if constexpr (EPW == 2)
            *(float2 *)(out_row + (size_t)w * 2) = make_float2(acc[0], acc[1]);
        else
            out_row[w] = acc[0];
    }
}

// ---- the backup rows' x and dy rows gathered into xo [2][R][d_model] (x_O,
// then dy_O; rows at or past n_ovf zero) by extra workgroups of an earlier
// launch (the ELL masks): the dW products take them, K-major, as the operand
// contracted over the rows.
struct BkGather {
    uint8_t *xo;
    int R, blocks;
};
BkGather bk_gather(int dt, int dm, int dff, int max_ovf, void *ws);
constexpr int GROWS = 4; // rows per workgroup of the gather
inline int bk_gather_blocks(int R) { return 2 * R / GROWS; }

// Block b (< bk_gather_blocks) of the gather, NTH threads, 16 bytes per lane.
// Nothing is written when the hybrid holds no backup rows.
template <int DT, int NTH>
DEVI void bk_gather_block(int b, const BkGather &g, const uint8_t *__restrict__ x,
                          const uint8_t *__restrict__ dy, const int32_t *__restrict__ ovf_rows,
                          const int32_t *__restrict__ n_ovf_p, int max_ovf, int dm)
{
    constexpr int esz = sizeof(typename elem<DT>::storage);
    const int n = min(*n_ovf_p, max_ovf);
    if (n <= 0)
        return;
    const int per = g.R / GROWS, z = b / per, r0 = (b % per) * GROWS;
    const size_t rowb = (size_t)dm * esz;
    const int c16 = (int)(rowb / 16); // d_model % 64 == 0: whole 16-byte chunks
    const uint8_t *src = z ? dy : x;
    uint8_t *dst = g.xo + (size_t)z * g.R * rowb;
    for (int q = threadIdx.x; q < GROWS * c16; q += NTH) {
        const int r = r0 + q / c16, c = q % c16;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < n)
            v = *(const uint4 *)(src + (size_t)ovf_rows[r] * rowb + (size_t)c * 16);
        *(uint4 *)(dst + (size_t)r * rowb + (size_t)c * 16) = v;
    }
}
