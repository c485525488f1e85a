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
void launch_bk_fwd(twell_dtype dt, const void *x, const hybrid_t *h, const void *wu,
                   const void *wd, int dm, float *y, void *ws, Timer &tm, hipStream_t s);
void launch_bk_ud(twell_dtype dt, const void *x, const void *dy, const hybrid_t *h,
                  const void *wu, const void *wd, int dm, float l1, void *ws, Timer &tm,
                  hipStream_t s);
void launch_bk_dxdw(twell_dtype dt, const hybrid_t *h, int dm, float *dx, float *dwd, float *dwu,
                    float *dwg, void *ws, Timer &tm, hipStream_t s);

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

// ---- transposed copies for the backward's backup products, made by extra
// workgroups of an earlier launch (the ELL masks) at full occupancy.
constexpr int TT = 64; // transpose tile (elements per side)
template <int DT> using Store = typename elem<DT>::storage;


// One TT x TT tile of out[c][r] = in[src(r)][c] for c < cols and r < rows_out,
// src(r) = r, or gather[r] for r < n_valid and a zero row past it (gather
// non-null). NTH threads; lds: TT x (TT + 8) elements.
template <typename T, int NTH = 256>
DEVI void transpose_tile(const T *__restrict__ in, T *__restrict__ out, int cols, int rows_out,
                         const int32_t *__restrict__ gather, int n_valid, int bx, int by,
                         uint8_t *lds)
{
    constexpr int V = 16 / sizeof(T), TP = TT + 8; // elements per 16-byte chunk, LDS pitch
    T(*tile)[TP] = (T(*)[TP])lds;
    const int c0 = bx * TT, r0 = by * TT, tid = threadIdx.x;
    if (gather && r0 >= (n_valid + TT - 1) / TT * TT)
        return; // never read: the products stop at the padded row count
    constexpr int CPR = TT / V; // chunks per tile row
    for (int q = tid; q < TT * CPR; q += NTH) {
        const int r = q / CPR, cc = q % CPR, gr = r0 + r, gc = c0 + cc * V;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (gr < n_valid && gc < cols) {
            const int sr = gather ? gather[gr] : gr;
            v = *(const uint4 *)(in + (size_t)sr * cols + gc);
        }
        const T *e = (const T *)&v;
#pragma unroll
        for (int k = 0; k < V; ++k)
            tile[r][cc * V + k] = e[k];
    }
    __syncthreads();
    for (int q = tid; q < TT * CPR; q += NTH) {
        const int c = q / CPR, rc = q % CPR, gc = c0 + c, gr = r0 + rc * V;
        if (gc >= cols || gr >= rows_out)
            continue;
        T e[V];
#pragma unroll
        for (int k = 0; k < V; ++k)
            e[k] = tile[rc * V + k][c];
        *(uint4 *)(out + (size_t)gc * rows_out + gr) = *(const uint4 *)e;
    }
    __syncthreads(); // lds is reused by the workgroup's next tile
}

// Tiles of a weight transpose [dff][dm] -> [dm][dff]
DEVI int wt_tiles(int dm, int dff) { return (dm / TT) * (dff / TT); }
template <int DT, int NTH = 256>
DEVI void weight_t_tile(const void *w, void *wt, int dm, int dff, int b, uint8_t *lds)
{
    const int nx = dm / TT;
    transpose_tile<Store<DT>, NTH>((const Store<DT> *)w, (Store<DT> *)wt, dm, dff, nullptr, dff,
                                   b % nx, b / nx, lds);
}


// Where the backward's transposed copies go: W_u^T, W_g^T ([dm][dff] each) at
// wt; x_O^T, dy_O^T ([dm][R] each) at xt; `blocks` workgroups make them.
struct BkXpose {
    uint8_t *wt, *xt;
    int R, blocks;
};
BkXpose bk_xpose(int dt, int dm, int dff, int max_ovf, void *ws);
inline int bk_xpose_blocks(int dm, int dff, int R)
{
    return 2 * (dm / TT) * (dff / TT) + 2 * (dm / TT) * (R / TT);
}

// Block b (< bk_xpose_blocks) of those copies; lds: TT x (TT + 8) elements.
// Nothing is copied when the hybrid holds no backup rows.
template <int DT>
DEVI void bk_xpose_block(int b, const BkXpose &xp, const uint8_t *x, const uint8_t *dy,
                         const uint8_t *wu, const uint8_t *wg, const int32_t *ovf_rows,
                         const int32_t *n_ovf_p, int max_ovf, int dm, int dff, uint8_t *lds)
{
    using T = Store<DT>;
    const int n = min(*n_ovf_p, max_ovf);
    if (n <= 0)
        return;
    const int nw = (dm / TT) * (dff / TT);
    if (b < 2 * nw) { // W_u^T, W_g^T
        const int z = b / nw;
        weight_t_tile<DT>(z ? wg : wu, (T *)xp.wt + (size_t)z * dm * dff, dm, dff, b % nw, lds);
        return;
    }
    b -= 2 * nw; // x_O^T, dy_O^T: [dm][R]
    const int ng = (dm / TT) * (xp.R / TT), z = b / ng, q = b % ng, gx = dm / TT;
    transpose_tile<T>((const T *)(z ? dy : x), (T *)xp.xt + (size_t)z * dm * xp.R, dm, xp.R,
                      ovf_rows, n, q % gx, q / gx, lds);
}
