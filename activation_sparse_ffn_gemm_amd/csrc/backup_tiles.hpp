// Device side of the dense products over the hybrid's backup rows (the
// products themselves are described in backup.hip): the tile routines and the
// backward's blocks. The forward's products have launches of their own
// (backup.hip); the backward's run as extra workgroups of the ELL passes'
// launches (bwd.hip), so that a layer without backup rows pays no launch for
// them.
#pragma once

#include "ntgemm.hpp"
#include "backup.hpp"

namespace bk {

// Tiles of 128 x 128, four waves of 64 x 64 each:
//   CU  the u/da products (short K = d_model; one workgroup of two four-wave
//       groups per CU): 64-byte K steps, four resident;
//   CY  y_O, the forward's split-K product (two workgroups per CU): 128-byte
//       K steps, two resident;
//   DX  the backward's dx_O and dW products (five workgroups per CU): 64-byte
//       K steps, two resident (measured against three resident, three
//       workgroups per CU: 141 -> 132 us at the 1.5B skewed layer; these
//       tiles have short K, and more tiles in flight hide their fill and
//       drain better than a deeper pipeline).
using CU = ng::Cfg<128, 128, 2, 2>;
using CY = ng::Cfg<128, 128, 2, 2, 2, 128>;
using DX = ng::Cfg<128, 128, 2, 2, 2, 64>;
constexpr int TILE = 128; // u/da tiles

template <int DT> using Store = typename elem<DT>::storage;

// ---------------------------------------------------------------- products
DEVI int n_rows(const int32_t *n_ovf_p, int max_ovf) { return min(*n_ovf_p, max_ovf); }

// u (and da) of one tile of backup rows x neurons on eight waves in two
// groups of four, each group on its own CU::LDS bytes of L:
//   fwd (BWD = false): the groups sum the two halves of K of u; epilogue
//                      A = h u -> a [R][dff] (hi, lo)
//   bwd (BWD = true):  group 0 runs u = x_O W_u, group 1 da = dy_O W_d^T;
//                      epilogue a, du, dg -> [R][dff] (hi, lo each)
// Each wave's sub-tile has two 32-row block rows (mi = 0, 1): group g runs
// the epilogue of block row g, so the groups swap the other block row's
// accumulators through LDS first (in the forward u = first half + second
// half, in that order). A workgroup of one group would leave one wave per
// SIMD, too few to cover the MFMA and LDS latencies; these products have few
// tiles, so the second group is not taken from other tiles.
constexpr int UD_NT = 2 * CU::NT;
static_assert(CU::MI == 2, "one block row per group");
template <int DT> constexpr int ud_lds()
{
    constexpr int P = TILE * (int)sizeof(Store<DT>) + 16;
    return 2 * CU::LDS > TILE * P ? 2 * CU::LDS : TILE * P;
}
static_assert(2 * CU::LDS >= 2 * CU::NWV * CU::NI * 16 * 64 * 4, "accumulator exchange");

template <int DT, bool BWD>
DEVI void ud_tile(const uint8_t *__restrict__ x, const uint8_t *__restrict__ dy,
                  const int32_t *__restrict__ ovf_rows, int n, const uint8_t *__restrict__ wu,
                  const uint8_t *__restrict__ wd, int dm, int dff, int R,
                  const void *__restrict__ dense, float l1, void *__restrict__ inter, int bx,
                  int by, uint8_t *L)
{
    using E = elem<DT>;
    constexpr int esz = sizeof(typename E::storage);
    constexpr int NH = DT == TWELL_BF16 ? 2 : 1; // arrays per intermediate
    constexpr int NI = CU::NI;
    constexpr int P = TILE * esz + 16;          // row pitch (bytes) of a staged tile in LDS
    const int m0 = by * TILE, i0 = bx * TILE;
    if (m0 >= n)
        return;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int grp = wave / CU::NWV, wg = wave % CU::NWV;
    const int wm = wg / CU::WGN, wn = wg % CU::WGN, lane = threadIdx.x & 63;
    const size_t rowbytes = (size_t)dm * esz;
    const int nk = (int)(rowbytes / CU::ROWB); // even: d_model % 64 == 0
    auto off = [](int kt) { return ng::StepOff{(size_t)kt * CU::ROWB, (size_t)kt * CU::ROWB}; };
    const uint8_t *src = BWD && grp ? dy : x, *w = BWD && grp ? wd : wu;
    auto rowa = [&](int r) { return src + (size_t)ovf_rows[min(m0 + r, n - 1)] * rowbytes; };
    auto rowb = [&](int r) { return w + (size_t)(i0 + r) * rowbytes; };
    const int kt0 = BWD ? 0 : grp * (nk / 2), kt1 = BWD ? nk : kt0 + nk / 2;
    // the stored h of this wave's epilogue elements (block row grp), requested
    // before the K loop: their latency then overlaps the first K step's loads
    // instead of following the accumulator swap
    const int mi = grp;
    typename E::storage hraw[NI][16];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int m = m0 + ng::acc_row<CU>(wm, mi, e, lane);
            const int i = i0 + ng::acc_col<CU>(wn, ni, lane);
            hraw[ni][e] = m < n ? ((const typename E::storage *)dense)[(size_t)m * dff + i]
                                : typename E::storage(0);
        }
    ng::Acc<CU> acc; // group 0: u (fwd: its first K half); group 1: da (fwd: u, second half)
    ng::mainloop<CU, DT>(L + grp * CU::LDS, rowa, rowb, off, kt0, kt1, acc, grp * CU::NWV);
    // swap: group g stores block row 1 - g of its accumulators in exchange
    // area g, lane-major per (wave, block column, element group), then reads
    // block row g of the other group's from area 1 - g
    float4 *X = (float4 *)L;
    auto xi = [&](int area, int ni, int eg) {
        return (((area * CU::NWV + wg) * NI + ni) * 4 + eg) * 64 + lane;
    };
    float own[NI][16], oth[NI][16];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            own[ni][e] = grp ? acc.v[1][ni][e] : acc.v[0][ni][e];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int eg = 0; eg < 4; ++eg) {
            const int mo = 1 - grp;
            X[xi(grp, ni, eg)] =
                make_float4(mo ? acc.v[1][ni][4 * eg] : acc.v[0][ni][4 * eg],
                            mo ? acc.v[1][ni][4 * eg + 1] : acc.v[0][ni][4 * eg + 1],
                            mo ? acc.v[1][ni][4 * eg + 2] : acc.v[0][ni][4 * eg + 2],
                            mo ? acc.v[1][ni][4 * eg + 3] : acc.v[0][ni][4 * eg + 3]);
        }
    __syncthreads();
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int eg = 0; eg < 4; ++eg) {
            const float4 v = X[xi(1 - grp, ni, eg)];
            oth[ni][4 * eg] = v.x;
            oth[ni][4 * eg + 1] = v.y;
            oth[ni][4 * eg + 2] = v.z;
            oth[ni][4 * eg + 3] = v.w;
        }
    __syncthreads(); // L is free again
    // block row grp of this wave: u and (bwd) da of each element
    const size_t plane = (size_t)R * dff; // elements per intermediate array
    float hv[NI][16];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if constexpr (DT == TWELL_BF16)
                hv[ni][e] = bf16_to_f32(hraw[ni][e]);
            else
                hv[ni][e] = hraw[ni][e];
        }
    // own / oth become a and (bwd) du, hv becomes dg
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float h = hv[ni][e];
            if constexpr (!BWD) {
                const float u = grp ? oth[ni][e] + own[ni][e] : own[ni][e] + oth[ni][e];
                own[ni][e] = h * u; // A
            } else {
                const float u = grp ? oth[ni][e] : own[ni][e];
                const float da = grp ? own[ni][e] : oth[ni][e];
                const float du = da * h, dg = h != 0.f ? da * u + l1 : 0.f;
                own[ni][e] = h * u; // a
                oth[ni][e] = du;
                hv[ni][e] = dg;
            }
        }
    constexpr int PLANE = TILE * P;
    constexpr int CPR = TILE * esz / 16; // 16-byte chunks per tile row
    {
        // A (fwd) or a, du and dg (bwd) as [R][dff] (planes hi, lo of each for
        // bf16): each plane's tile goes through LDS as [m][i], then the
        // workgroup stores it along i, 16 bytes per lane. QR planes per round.
        constexpr int NR = (BWD ? 3 : 1) * NH;
        constexpr int FIT = ud_lds<DT>() / PLANE;
        constexpr int QR = FIT >= 3 && NR % 3 == 0 ? 3 : (FIT >= 2 && NR % 2 == 0 ? 2 : 1);
        static_assert(NR % QR == 0 && QR * PLANE <= ud_lds<DT>(), "LDS rounds");
#pragma unroll 1
        for (int qb = 0; qb < NR; qb += QR) {
#pragma unroll
            for (int qq = 0; qq < QR; ++qq) {
                const int q = qb + qq, which = q / NH, part = q % NH; // bwd: a, du, dg
                uint8_t *Lq = L + qq * PLANE;
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int r = ng::acc_row<CU>(wm, mi, e, lane);
                        const int c = ng::acc_col<CU>(wn, ni, lane);
                        const float v = !BWD || which == 0
                                            ? own[ni][e]
                                            : (which == 1 ? oth[ni][e] : hv[ni][e]);
                        if constexpr (DT == TWELL_BF16) {
                            const uint32_t hl = f32_to_bf16_hilo(v);
                            *(uint16_t *)(Lq + r * P + c * 2) =
                                (uint16_t)(part == 0 ? hl : hl >> 16);
                        } else {
                            *(float *)(Lq + r * P + c * 4) = v;
                        }
                    }
            }
            __syncthreads();
#pragma unroll
            for (int qq = 0; qq < QR; ++qq) {
                uint8_t *base = (uint8_t *)inter + (size_t)(qb + qq) * plane * esz;
                const uint8_t *Lq = L + qq * PLANE;
                for (int t = threadIdx.x; t < TILE * CPR; t += UD_NT) {
                    const int r = t / CPR, ch = t % CPR;
                    *(uint4 *)(base + ((size_t)(m0 + r) * dff + i0) * esz + ch * 16) =
                        *(const uint4 *)(Lq + r * P + ch * 16);
                }
            }
            __syncthreads();
        }
    }
}

// One tile of partial rows x weights over a K split: part[sp][m][d] = sum
// over the split's K steps of a_q[m][.] . w_q[.][d], for NSEG segments of
// d_ff each. Segment q reads A array q (arrays `R dff` elements apart, K
// along their rows) and weight matrix w0 (q >> BSHIFT == 0) or w1, stored
// [d_ff][d_model], i.e. K-major: read through the transposing LDS loads.
template <class C, int DT, int NSEG, int BSHIFT>
DEVI void rowsw_tile(const uint8_t *__restrict__ a, const uint8_t *__restrict__ w0,
                     const uint8_t *__restrict__ w1, int n, int dm, int dff, int R, int S,
                     float *__restrict__ part, int bx, int by, int sp, uint8_t *L)
{
    using E = elem<DT>;
    constexpr int esz = sizeof(typename E::storage);
    constexpr int KS = C::ROWB / esz; // K per step
    static_assert(C::BM == C::BN, "square tiles");
    const int m0 = by * C::BM, d0 = bx * C::BN;
    if (m0 >= n)
        return;
    const size_t rowbytes = (size_t)dff * esz, plane = (size_t)R * dff * esz,
                 wrow = (size_t)dm * esz;
    const int spseg = dff / KS, nk = NSEG * spseg;
    const int kt0 = (int)((long)nk * sp / S), kt1 = (int)((long)nk * (sp + 1) / S);
    auto rowa = [&](int r) { return a + (size_t)(m0 + r) * rowbytes; };
    auto rowb = [&](int r) { return w0 + (size_t)r * wrow + (size_t)d0 * esz; };
    const ptrdiff_t w01 = w1 - w0;
    auto off = [&](int kt) {
        const int q = kt / spseg, kk = kt % spseg;
        return ng::StepOff{q * plane + (size_t)kk * C::ROWB,
                           (size_t)((q >> BSHIFT) ? w01 : 0) + (size_t)kk * KS * wrow};
    };
    ng::Acc<C> acc;
    ng::mainloop_mixed<C, DT, ng::KC, ng::KM>(L, rowa, rowb, off, kt0, kt1, acc, 1 << 30,
                                               dm - d0);
    const int lane = threadIdx.x & 63, wm = ng::wave_m<C>(), wn = ng::wave_n<C>();
    float *p = part + (size_t)sp * R * dm;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                // rows past n are padding rows of the R-row partial (never
                // read): only the column needs a test, no branch per row
                const int m = m0 + ng::acc_row<C>(wm, mi, e, lane);
                const int d = d0 + ng::acc_col<C>(wn, ni, lane);
                if (d < dm)
                    p[(size_t)m * dm + d] = acc.v[mi][ni][e];
            }
}

// One tile of dW[i][d] = sum_m it[m][i] xo[m][d] over the backup rows, z = 0,
// 1, 2: (dW_d, a, dy_O), (dW_u, du, x_O), (dW_g, dg, x_O); hi and lo segments
// for bf16. Both operands run along the rows m, the contraction index: both
// are read K-major. Rows at or past n hold zeros in both (the u/da epilogue
// stores its whole tiles, the gather zero rows), so whole K steps are safe.
template <class C, int DT>
DEVI void dw_tile(const uint8_t *__restrict__ it, const uint8_t *__restrict__ xo, int n, int dm,
                  int dff, int R, float *__restrict__ dwd, float *__restrict__ dwu,
                  float *__restrict__ dwg, int bx, int by, int z, uint8_t *L)
{
    using E = elem<DT>;
    constexpr int esz = sizeof(typename E::storage);
    constexpr int NH = DT == TWELL_BF16 ? 2 : 1;
    constexpr int KS = C::ROWB / esz; // rows per K step
    if (n <= 0)
        return;
    const int d0 = bx * C::BN, i0 = by * C::BM;
    const size_t plane = (size_t)R * dff * esz, irow = (size_t)dff * esz,
                 xrow = (size_t)dm * esz;
    const uint8_t *ta = it + (size_t)z * NH * plane;             // a / du / dg, hi first
    const uint8_t *tx = xo + (size_t)(z == 0 ? 1 : 0) * R * xrow; // dy_O or x_O
    float *out = z == 0 ? dwd : (z == 1 ? dwu : dwg);
    const int spseg = (n + KS - 1) / KS, nk = NH * spseg;
    auto rowa = [&](int r) { return ta + (size_t)r * irow + (size_t)i0 * esz; };
    auto rowb = [&](int r) { return tx + (size_t)r * xrow + (size_t)d0 * esz; };
    auto off = [&](int kt) {
        const int q = kt / spseg, kk = kt % spseg;
        return ng::StepOff{q * plane + (size_t)kk * KS * irow, (size_t)kk * KS * xrow};
    };
    ng::Acc<C> acc;
    ng::mainloop_mixed<C, DT, ng::KM, ng::KM>(L, rowa, rowb, off, 0, nk, acc, dff - i0, dm - d0);
    // the tile is the backup rows' share of dW, written whole: the ELL rows'
    // share is added to it by the neuron pass, which runs next
    const int lane = threadIdx.x & 63, wm = ng::wave_m<C>(), wn = ng::wave_n<C>();
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int i = i0 + ng::acc_row<C>(wm, mi, e, lane);
                const int d = d0 + ng::acc_col<C>(wn, ni, lane);
                if (i < dff && d < dm)
                    out[(size_t)i * dm + d] = acc.v[mi][ni][e];
            }
}

// ---------------------------------------------------------------- backward blocks
// Block b (< n_ud) of the u/da tiles (UD_NT threads, ud_lds bytes of L).
template <int DT>
DEVI void ud_block(int b, const BkBwd &p, const uint8_t *__restrict__ x,
                   const uint8_t *__restrict__ dy, const int32_t *__restrict__ ovf_rows,
                   const int32_t *__restrict__ n_ovf_p, int max_ovf,
                   const uint8_t *__restrict__ wu, const uint8_t *__restrict__ wd, int dm,
                   int dff, const void *__restrict__ dense, float l1, uint8_t *L)
{
    const int n = n_rows(n_ovf_p, max_ovf);
    if (n <= 0)
        return;
    const int nx = dff / TILE;
    ud_tile<DT, true>(x, dy, ovf_rows, n, wu, wd, dm, dff, p.R, dense, l1, p.inter, b % nx,
                      b / nx, L);
}

// Block b (< n_dx + n_dw) of the dx_O tiles (K split), then of the dW tiles
// (DX::NT threads, DX::LDS bytes of L).
template <int DT>
DEVI void dxdw_block(int b, const BkBwd &p, const uint8_t *__restrict__ wu,
                     const uint8_t *__restrict__ wg, const int32_t *__restrict__ n_ovf_p,
                     int max_ovf, int dm, int dff, float *__restrict__ dwd,
                     float *__restrict__ dwu, float *__restrict__ dwg, uint8_t *L)
{
    constexpr int NH = DT == TWELL_BF16 ? 2 : 1;
    const int n = n_rows(n_ovf_p, max_ovf);
    if (n <= 0)
        return;
    const int nd = (dm + DX::BN - 1) / DX::BN;
    if (b < p.n_dx) {
        // segments (du hi, du lo, dg hi, dg lo) against (W_u, W_u, W_g, W_g),
        // or (du, dg) against (W_u, W_g); du is plane NH of inter (after a)
        const int mt = p.R / DX::BM;
        const size_t plane = (size_t)p.R * dff * sizeof(Store<DT>);
        rowsw_tile<DX, DT, 2 * NH, NH == 2 ? 1 : 0>(p.inter + NH * plane, wu, wg, n, dm, dff,
                                                     p.R, p.S, p.part, b % nd, (b / nd) % mt,
                                                     b / (nd * mt), L);
        return;
    }
    b -= p.n_dx;
    const int ni = (dff + DX::BM - 1) / DX::BM;
    dw_tile<DX, DT>(p.inter, p.xo, n, dm, dff, p.R, dwd, dwu, dwg, b % nd, (b / nd) % ni,
                    b / (nd * ni), L);
}

} // namespace bk
