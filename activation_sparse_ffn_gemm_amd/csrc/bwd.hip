// Backward of y = (h (.) x W_u) W_d on the pattern P of a hybrid ELL + dense
// backup ("Sparser, Faster, Lighter Transformer Language Models", summary page
// section 2.B.3: sparse-to-dense and dense-to-sparse products in the backward,
// no dense work on zeros; overflow rows live in a dense backup).
//
// With u = x W_u and da = dy W_d^T sampled on P, a = h u, du = da h and
// dg = da u + l1 (l1: weight of an activation penalty l1 * sum(h) in the
// loss, whose gradient is l1 on P):
//   dx = du W_u^T + dg W_g^T,  dW_d = a^T dy,  dW_u = x^T du,  dW_g = x^T dg.
//
// ELL rows (gathers, fp32 accumulation, no atomics, deterministic):
//   1. masks:  per block of 64 rows and per neuron, a 64-bit mask of the
//      rows holding that neuron; its popcount is the block's count;
//   2. scans:  per neuron, the prefix of those counts over blocks, and per
//      group of 64 neurons the prefix of the neurons' totals inside the
//      group and the group's total. Entry (t, i) then sits at (totals of the
//      groups before i's) + (i's prefix in its group) + prefix[i][block(t)]
//      + popcount(mask bits below t): the column-major order of the entries,
//      rows ascending inside a column;
//   3. fill: each ELL slot writes its row index at its column-major position;
//   4. neuron pass (dense-to-sparse, then sparse^T-to-dense): a wave per
//      neuron keeps its wu_t and wd rows in registers and walks its entries in
//      row order; per entry it gathers x[t] and dy[t] once, computes
//      u = x[t] . wu_t[i] and da = dy[t] . wd[i], then a, du, dg, adds
//      a dy[t], du x[t], dg x[t] to its three dW rows, and keeps du, dg for
//      the dx pass. Every dW row is written once (zero rows for unused
//      neurons), added to the backup rows' share when there are backup rows;
//   5. dx (sparse-to-dense): a wave per (row, part of d_model) sums
//      du wu_t[i] + dg wg_t[i] over the row's entries.
// Rows are gathered with 4-byte lanes (rows.hpp).
// Backup rows (dense MFMA, fp32 accumulation; the tiles live in
// backup_tiles.hpp):
//   6. U/DA: u and da of every backup row and neuron, then a, du, dg (dg zero
//      where h is zero), as extra workgroups of the scans launch;
//   7. DX:   dx of backup rows = [du | dg] [W_u ; W_g]^T as split-K partials,
//      summed into their rows by the dx pass;
//   8. DW:   dW = [a | du | dg]^T [dy | x | x] over the backup rows, written
//      before the neuron pass, which adds the ELL rows' share (a two-term
//      sum, so its value does not depend on the order of the two passes).
// DX and DW ride on the fill launch, and the x and dy rows of the backup rows
// are gathered once by extra workgroups of the masks launch: five launches in
// all, with or without backup rows; no operand is transposed.
#include "backup_tiles.hpp"
#include "rows.hpp"
#include "slices.hpp"

namespace {

constexpr int NT = 256;
constexpr int BR = 64;    // rows per mask block (one bit each)
constexpr int CH = 1024;  // neurons per workgroup of the mask launch (8 KB of LDS)

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

// The dx pass gathers two weight rows per entry. With many tokens and
// weights well beyond one XCD's L2 it runs XCD-local (slices.hpp): XCD k sums
// the k-th slice of d_model of the wu_t and wg_t rows from an interleaved
// slice-major copy that the masks launch makes on the side: an entry's two
// slices are then one run of lines. (Reading the slices in place, where they
// are runs of whole lines, saves the copy's 12 us at the 1.5B shape but makes
// the dx pass 16 us slower: each XCD's slices are then 512-byte runs at a
// 4 KB stride in two matrices.)
inline bool dx_split(int dt, int T, int dm, int dff)
{
    return T >= 1024 && (size_t)dff * dm * (dt == TWELL_BF16 ? 2 : 4) >= ((size_t)16 << 20);
}

struct Layout {
    size_t coef, masks, cnt, lp, gt, csc, backup, wsl, total;
    int nblk;
    bool split;
};

Layout layout(int dt, int T, int dm, int dff, int K, int max_ovf)
{
    Layout L;
    L.nblk = (T + BR - 1) / BR;
    L.split = dx_split(dt, T, dm, dff);
    size_t o = 0;
    L.coef = o;   o += up256((size_t)2 * T * K * 4); // du, dg per ELL slot
    L.masks = o;  o += up256((size_t)L.nblk * dff * 8);
    L.cnt = o;    o += up256((size_t)L.nblk * dff * 4);
    L.lp = o;     o += up256((size_t)dff * 4);
    L.gt = o;     o += up256((size_t)(dff + 63) / 64 * 4);
    L.csc = o;    o += up256((size_t)T * K * 4);
    L.backup = o; o += up256(bk_workspace(dt, dm, dff, max_ovf, true));
    L.wsl = o;    o += L.split ? up256((size_t)NXCD * dff * 2 * slices(dt, dm).swp * 4) : 0;
    L.total = o;
    return L;
}

// ------------------------------------------------------------ 1. masks
// One workgroup per (block of 64 rows, chunk of CH neurons): the masks of the
// chunk are built in LDS, then written once, coalesced, with their popcounts:
// masks and cnt are both [nblk][dff]. Wave w takes the block's rows w, w + 4,
// ..., lane s reading ELL slot s of each (stored slots only): the sixteen
// rows' loads go out together.
DEVI void ell_mask_block(
    const int32_t *__restrict__ row_nnz, const int32_t *__restrict__ row_slot,
    const int16_t *__restrict__ ell_col, int T, int K, int dff,
    uint64_t *__restrict__ masks, int32_t *__restrict__ cnt, int b, int chunk,
    unsigned long long *m)
{
    constexpr int NWV = NT / 64, RPW = BR / NWV;
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int c0 = chunk * CH, c1 = min(dff, c0 + CH);
    const int r0 = b * BR, nr = min(T - r0, BR);
    for (int i = threadIdx.x; i < c1 - c0; i += NT)
        m[i] = 0ull;
    // lane j < RPW: stored entries of the wave's row wv + NWV j (none for
    // backup rows and rows past T)
    int rn = 0;
    if (lane < RPW) {
        const int r = wv + NWV * lane;
        if (r < nr && row_slot[r0 + r] < 0)
            rn = min(row_nnz[r0 + r], K);
    }
    __syncthreads();
    for (int s0 = 0; __ballot(rn > s0) != 0ull; s0 += 64) {
        int c[RPW];
#pragma unroll
        for (int j = 0; j < RPW; ++j)
            c[j] = s0 + lane < bcast(rn, j)
                       ? ell_col[(size_t)(r0 + wv + NWV * j) * K + s0 + lane] : -1;
        // corrupt columns fall outside every chunk: skipped here, reported
        // by the fill
#pragma unroll
        for (int j = 0; j < RPW; ++j)
            if (c[j] >= c0 && c[j] < c1)
                atomicOr(&m[c[j] - c0], 1ull << (wv + NWV * j));
    }
    __syncthreads();
    for (int i = threadIdx.x; i < c1 - c0; i += NT) {
        masks[(size_t)b * dff + c0 + i] = m[i];
        cnt[(size_t)b * dff + c0 + i] = __popcll(m[i]);
    }
}

// ------------------------------------------------------------ 2. scans
// One workgroup per group of 64 neurons (a lane each); its NTH / 64 waves take
// a share of the blocks each. Pass 1 sums each wave's counts, the waves' sums
// are combined in LDS, pass 2 rewrites the counts as exclusive prefixes over
// the blocks (in place). The last wave holds the neurons' totals: it stores
// their inclusive prefix inside the group (lp) and the group's total (gt).
// A neuron's entries then start at the sum of gt over the groups before its
// own plus lp of the neuron before it in its group (no scan over all
// neurons, and no launch for one: the fill and the neuron pass add the few
// group totals themselves). Loads are unconditional (indices clamped,
// values masked) so each pass keeps U loads in flight per lane.
template <int NTH>
DEVI void blk_prefix_block(int g, int32_t *__restrict__ cnt, int nblk, int dff,
                           int32_t *__restrict__ lp, int32_t *__restrict__ gt, int (*tot)[64])
{
    constexpr int U = 8, NWV = NTH / 64;
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int i = g * 64 + lane, ic = min(i, dff - 1);
    const int per = (nblk + NWV - 1) / NWV;
    const int b0 = min(nblk, wv * per), b1 = min(nblk, b0 + per);
    int run = 0;
    for (int b = b0; b < b1; b += U) {
        int v[U];
#pragma unroll
        for (int q = 0; q < U; ++q)
            v[q] = cnt[(size_t)min(b + q, b1 - 1) * dff + ic];
#pragma unroll
        for (int q = 0; q < U; ++q)
            run += b + q < b1 ? v[q] : 0;
    }
    tot[wv][lane] = run;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wv; ++w)
        base += tot[w][lane];
    if (wv == NWV - 1) {
        const int incl = wave_incl_scan(i < dff ? base + run : 0, lane);
        if (i < dff)
            lp[i] = incl;
        if (lane == 63)
            gt[g] = incl;
    }
    run = base;
    for (int b = b0; b < b1; b += U) {
        int v[U];
#pragma unroll
        for (int q = 0; q < U; ++q)
            v[q] = cnt[(size_t)min(b + q, b1 - 1) * dff + ic];
#pragma unroll
        for (int q = 0; q < U; ++q)
            if (b + q < b1 && i < dff) {
                cnt[(size_t)(b + q) * dff + i] = run;
                run += v[q];
            }
    }
}

// ------------------------------------------------------------ 3. fill
// Each stored ELL slot writes its index t K + s at its column-major position.
// Wave w of workgroup b takes rows FILL_ROWS b + FR w .. + FR - 1 (one 64-row
// block), lane s slot s of each, all the rows' loads in flight together; wave
// 0 first scans the group totals into LDS (gpre).
constexpr int FR = 4;                   // rows per wave of the fill
constexpr int FILL_ROWS = FR * NT / 64; // rows per workgroup of the fill
static_assert(BR % FR == 0, "a wave's rows share one mask block");
DEVI void csc_fill_block(
    int b, const int32_t *__restrict__ row_nnz, const int32_t *__restrict__ row_slot,
    const int16_t *__restrict__ ell_col, int T, int K, int dff,
    const uint64_t *__restrict__ masks, const int32_t *__restrict__ blkpre,
    const int32_t *__restrict__ lp, const int32_t *__restrict__ gt, int32_t *__restrict__ csc,
    int32_t *__restrict__ status, int *gpre)
{
    const int lane = threadIdx.x & 63, wv = wave_id();
    if (wv == 0) { // exclusive prefix of the group totals
        const int ng = (dff + 63) / 64;
        int run = 0;
        for (int g0 = 0; g0 < ng; g0 += 64) {
            const int g = g0 + lane;
            const int v = g < ng ? gt[g] : 0;
            const int incl = wave_incl_scan(v, lane);
            if (g < ng)
                gpre[g] = run + incl - v;
            run += bcast(incl, 63);
        }
    }
    const int t0 = b * FILL_ROWS + wv * FR, blk = t0 / BR;
    int nn = 0; // lane j < FR: stored entries of row t0 + j (none for backup rows)
    if (lane < FR && t0 + lane < T && row_slot[t0 + lane] < 0)
        nn = min(row_nnz[t0 + lane], K);
    __syncthreads();
    const size_t mb = (size_t)blk * dff;
    for (int s0 = 0; __ballot(nn > s0) != 0ull; s0 += 64) {
        const int s = s0 + lane;
        int c[FR];
#pragma unroll
        for (int j = 0; j < FR; ++j)
            c[j] = s < bcast(nn, j) ? ell_col[(size_t)(t0 + j) * K + s] : -1;
        int pre[FR];
        unsigned long long mk[FR];
        bool in[FR];
#pragma unroll
        for (int j = 0; j < FR; ++j) {
            in[j] = s < bcast(nn, j);
            // a corrupt entry is skipped (the masks skip it too) and reported
            if (in[j] && (c[j] < 0 || c[j] >= dff)) {
                raise_status(status, TWELL_DEV_BAD_INDEX);
                in[j] = false;
            }
            pre[j] = 0;
            mk[j] = 0ull;
            if (in[j]) {
                pre[j] = blkpre[mb + c[j]] + ((c[j] & 63) ? lp[c[j] - 1] : 0);
                mk[j] = masks[mb + c[j]];
            }
        }
#pragma unroll
        for (int j = 0; j < FR; ++j)
            if (in[j]) {
                const unsigned long long below = (1ull << ((t0 + j) % BR)) - 1ull;
                csc[gpre[c[j] >> 6] + pre[j] + __popcll(mk[j] & below)] = (t0 + j) * K + s;
            }
    }
}

// ------------------------------------------------------------ 4. neuron pass
// NW words per lane cover the whole row (dots); the wave accumulates the NWP
// words of part `part` (PARTS = NW / NWP parts, one per blockIdx.y).
template <int DT, int NW, int NWP, int G, int S>
__global__ __launch_bounds__(64 * S) void bwd_neuron_kernel(
    const int32_t *__restrict__ lp, const int32_t *__restrict__ gt,
    const int32_t *__restrict__ csc, const void *__restrict__ ell_val, int T, int K, int dff,
    const uint8_t *__restrict__ x,
    const uint8_t *__restrict__ dy, const uint8_t *__restrict__ wu, const uint8_t *__restrict__ wd,
    int dm, float l1, float *__restrict__ coef, float *__restrict__ dwg, float *__restrict__ dwu,
    float *__restrict__ dwd, const int32_t *__restrict__ n_ovf_p, int max_ovf)
{
    using E = elem<DT>;
    using R = Row<DT, NW>;
    // the backup rows' dense products have written their share of dW when the
    // hybrid holds backup rows: this pass adds the ELL rows' share to it
    const bool add = T > 0 && max_ovf > 0 && min(*n_ovf_p, max_ovf) > 0;
    using RP = Row<DT, NWP>;
    constexpr int EPW = R::EPW;
    constexpr int PL = NWP * 64 * EPW; // elements of one part of a row
    __shared__ __attribute__((aligned(16))) float red[S > 1 ? S : 1][S > 1 ? PL : 4];
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int i = blockIdx.x, part = blockIdx.y;
    const R geo(dm, lane, 0);
    const RP pgeo(dm, lane, part);
    const long TK = (long)T * K;
    uint32_t wuw[NW], wdw[NW];
    geo.load_w(wu, i, wuw);
    geo.load_w(wd, i, wdw);
    float ad[NWP][EPW], au[NWP][EPW], ag[NWP][EPW];
    pgeo.zero_f(ad);
    pgeo.zero_f(au);
    pgeo.zero_f(ag);
    // The neuron's entries are dealt to the S waves round-robin (entry p0 + w,
    // p0 + w + S, ...), so the chain of dependent gathers each wave walks is
    // 1/S of the list; the S partial dW rows are summed in LDS below.
    // the neuron's entries [p0, p1) of the column-major list: the totals of
    // the groups of 64 neurons before its own, plus its group's prefix
    int gs = 0;
    for (int j = lane; j < (i >> 6); j += 64)
        gs += gt[j];
    const int base = bcast(wave_incl_scan(gs, lane), 63);
    const int p0 = base + ((i & 63) ? lp[i - 1] : 0), p1 = base + lp[i];
    for (int pb = p0 + wv; pb < p1; pb += 64 * S) {
        // lane L prefetches this wave's entry pb + S L: its ELL slot, row and h
        const int p = pb + S * lane;
        int idx = -1;
        float h = 0.f;
        if (p < p1) {
            idx = csc[p];
            if (idx >= 0 && idx < TK)
                h = E::load1(ell_val, idx);
            else
                idx = -1;
        }
        const int tt = idx >= 0 ? idx / K : 0;
        const int m = min(64, (p1 - pb + S - 1) / S);
        // stream the m entries through G register buffers: the x and dy rows
        // of entry e + G are requested as soon as entry e has been used
        uint32_t vx[G][NW], vd[G][NW];
        auto fetch = [&](int e, uint32_t (&xr)[NW], uint32_t (&dr)[NW]) {
            const int tr = bcast(tt, min(e, m - 1));
            geo.load_w(x, tr, xr);
            geo.load_w(dy, tr, dr);
        };
#pragma unroll
        for (int g = 0; g < G; ++g)
            fetch(g, vx[g], vd[g]);
        for (int e0 = 0; e0 < m; e0 += G) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int e = e0 + g;
                const float u = wave_sum(geo.dotw(vx[g], wuw));
                const float da = wave_sum(geo.dotw(vd[g], wdw));
                if (e < m) { // uniform
                    const float hh = bcast(h, e);
                    const float a = hh * u, du = da * hh, dg = hh != 0.f ? da * u + l1 : 0.f;
                    // the lane that owns this entry keeps du, dg for the dx pass
                    if (lane == e && idx >= 0) {
                        coef[idx] = du;
                        coef[TK + idx] = dg;
                    }
                    // this wave's part of the row: words c = part * NWP + c2
                    // (static indices; the part test is uniform across the wave)
#pragma unroll
                    for (int c = 0; c < NW; ++c) {
                        if (c / NWP != part)
                            continue;
                        const int c2 = c % NWP;
                        float xv[EPW], dv[EPW];
                        geo.widen(vx[g][c], xv);
                        geo.widen(vd[g][c], dv);
#pragma unroll
                        for (int q = 0; q < EPW; ++q) {
                            ad[c2][q] += a * dv[q];
                            au[c2][q] += du * xv[q];
                            ag[c2][q] += dg * xv[q];
                        }
                    }
                }
                fetch(e + G, vx[g], vd[g]);
            }
        }
    }
    // sum the S partial rows in a fixed order (wave 0 first) and write each
    // dW row once; element q of the part is word q / EPW, half q % EPW
    const int n_el = dm - part * PL < PL ? dm - part * PL : PL;
    auto reduce_store = [&](const float (&acc)[NWP][EPW], float *out) {
#pragma unroll
        for (int c = 0; c < NWP; ++c)
#pragma unroll
            for (int e = 0; e < EPW; ++e)
                red[wv][(c * 64 + lane) * EPW + e] = acc[c][e];
        __syncthreads();
        float *o = out + (size_t)i * dm + (size_t)part * PL;
        for (int q = 4 * threadIdx.x; q < n_el; q += 4 * 64 * S) {
            float4 sum = *(const float4 *)&red[0][q];
#pragma unroll
            for (int w = 1; w < S; ++w) {
                const float4 v = *(const float4 *)&red[w][q];
                sum.x += v.x;
                sum.y += v.y;
                sum.z += v.z;
                sum.w += v.w;
            }
            if (add) {
                const float4 b = *(const float4 *)(o + q);
                sum = make_float4(b.x + sum.x, b.y + sum.y, b.z + sum.z, b.w + sum.w);
            }
            *(float4 *)(o + q) = sum;
        }
        __syncthreads();
    };
    if constexpr (S == 1) {
        if (add) {
            pgeo.add_store_f(dwd, i, ad);
            pgeo.add_store_f(dwu, i, au);
            pgeo.add_store_f(dwg, i, ag);
        } else {
            pgeo.store_f(dwd, i, ad);
            pgeo.store_f(dwu, i, au);
            pgeo.store_f(dwg, i, ag);
        }
    } else {
        reduce_store(ad, dwd);
        reduce_store(au, dwu);
        reduce_store(ag, dwg);
    }
}

// ------------------------------------------------------------ 5. dx
template <int DT, int NW, int G>
__global__ __launch_bounds__(NT) void bwd_dx_kernel(
    const int32_t *__restrict__ row_nnz, const int32_t *__restrict__ row_slot,
    const int16_t *__restrict__ ell_col, const float *__restrict__ coef, int T, int K, int dff,
    const uint8_t *__restrict__ wu, const uint8_t *__restrict__ wg, int dm,
    float *__restrict__ dx, BkPart bp, int max_ovf)
{
    using R = Row<DT, NW>;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (NT / 64) + wave_id();
    if (t >= T)
        return;
    const R geo(dm, lane, blockIdx.y);
    const int slot = row_slot[t];
    if (slot >= 0) { // a backup row: dx is the sum of the dense product's partials
        if (bp.part && slot < max_ovf)
            bk_finish_row<NW, R::EPW>(bp, slot, geo.ndw, geo.base, geo.ndw, lane,
                                          dx + (size_t)t * dm);
        return;
    }
    const size_t TK = (size_t)T * K, rb = (size_t)t * K;
    float acc[NW][R::EPW];
    geo.zero_f(acc);
    const int n = min(row_nnz[t], K);
    for (int s0 = 0; s0 < n; s0 += 64) {
        // each lane fetches one entry, then the wave walks them in order
        const int s = s0 + lane;
        int ci = 0;
        float cu = 0.f, cg = 0.f;
        if (s < n) {
            ci = ell_col[rb + s];
            cu = coef[rb + s];
            cg = coef[TK + rb + s];
            if (ci < 0 || ci >= dff) {
                ci = 0;
                cu = cg = 0.f;
            }
        }
        const int m = min(64, n - s0);
        // stream the m entries through G register buffers: the rows of entry
        // e + G are requested as soon as entry e has been used
        uint32_t vu[G][NW], vg[G][NW];
        auto fetch = [&](int e, uint32_t (&u)[NW], uint32_t (&g)[NW]) {
            const int c = bcast(ci, min(e, m - 1));
            geo.load_w(wu, c, u);
            geo.load_w(wg, c, g);
        };
#pragma unroll
        for (int g = 0; g < G; ++g)
            fetch(g, vu[g], vg[g]);
        for (int e0 = 0; e0 < m; e0 += G) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int e = e0 + g;
                if (e < m) { // uniform
                    geo.axpy(acc, bcast(cu, e), vu[g]);
                    geo.axpy(acc, bcast(cg, e), vg[g]);
                }
                fetch(e + G, vu[g], vg[g]);
            }
        }
    }
    geo.store_f(dx, t, acc);
}

// ------------------------------------------------------------ masks launch
// Work that only has to be done before later passes rides on the masks
// launch: workgroups b < n_mask build masks; the next n_copy copy wu_t and
// wg_t into the dx pass's interleaved slice-major array; the rest gather the
// backup rows' x and dy rows for the dW products.
template <int DT>
__global__ __launch_bounds__(NT) void mask_kernel(
    const int32_t *__restrict__ row_nnz, const int32_t *__restrict__ row_slot,
    const int16_t *__restrict__ ell_col, int T, int K, int dff, uint64_t *__restrict__ masks,
    int32_t *__restrict__ cnt, int n_chunk, int n_mask, int n_copy,
    const uint32_t *__restrict__ wu, const uint32_t *__restrict__ wg, uint32_t *__restrict__ wsl,
    Slices sl, BkGather bg, const uint8_t *__restrict__ x, const uint8_t *__restrict__ dy,
    const int32_t *__restrict__ ovf_rows, const int32_t *__restrict__ n_ovf_p, int max_ovf,
    int dm)
{
    __shared__ unsigned long long lds[CH];
    int b = blockIdx.x;
    if (b < n_mask) {
        ell_mask_block(row_nnz, row_slot, ell_col, T, K, dff, masks, cnt, b / n_chunk,
                       b % n_chunk, lds);
        return;
    }
    b -= n_mask;
    if (b < n_copy) {
        copy_slices_rows<2, NT>(b, wu, wg, wsl, dff, sl);
        return;
    }
    bk_gather_block<DT, NT>(b - n_copy, bg, x, dy, ovf_rows, n_ovf_p, max_ovf, dm);
}

// ------------------------------------------------------------ scans launch
// Workgroups g < n_grp run the block scans of neuron group g; the rest are the
// backup rows' u/da tiles, which need nothing from the masks launch.
template <int DT>
__global__ __launch_bounds__(bk::UD_NT, 1) void prefix_ud_kernel(
    int32_t *__restrict__ cnt, int nblk, int dff, int32_t *__restrict__ lp,
    int32_t *__restrict__ gt, int n_grp, BkBwd bw, const uint8_t *__restrict__ x,
    const uint8_t *__restrict__ dy, const int32_t *__restrict__ ovf_rows,
    const int32_t *__restrict__ n_ovf_p, int max_ovf, const uint8_t *__restrict__ wu,
    const uint8_t *__restrict__ wd, int dm, const void *__restrict__ dense, float l1)
{
    __shared__ __attribute__((aligned(16))) uint8_t L[bk::ud_lds<DT>()];
    if ((int)blockIdx.x < n_grp) {
        blk_prefix_block<bk::UD_NT>(blockIdx.x, cnt, nblk, dff, lp, gt, (int (*)[64])L);
        return;
    }
    bk::ud_block<DT>(blockIdx.x - n_grp, bw, x, dy, ovf_rows, n_ovf_p, max_ovf, wu, wd, dm, dff,
                     dense, l1, L);
}

// ------------------------------------------------------------ fill launch
// Workgroups b < n_fill fill the CSC list; the rest are the backup rows' dx_O
// and dW tiles (their dW tiles write dW, to which the neuron pass adds the
// ELL rows' share; the dx pass sums their dx partials).
template <int DT>
__global__ __launch_bounds__(NT, 5) void fill_dxdw_kernel(
    const int32_t *__restrict__ row_nnz, const int32_t *__restrict__ row_slot,
    const int16_t *__restrict__ ell_col, int T, int K, int dff,
    const uint64_t *__restrict__ masks, const int32_t *__restrict__ blkpre,
    const int32_t *__restrict__ lp, const int32_t *__restrict__ gt, int32_t *__restrict__ csc,
    int32_t *__restrict__ status, int n_fill, BkBwd bw, const uint8_t *__restrict__ wu,
    const uint8_t *__restrict__ wg, const int32_t *__restrict__ n_ovf_p, int max_ovf, int dm,
    float *__restrict__ dwd, float *__restrict__ dwu, float *__restrict__ dwg)
{
    static_assert(bk::DX::NT == NT, "one workgroup size for both");
    static_assert(bk::DX::LDS >= 512 * 4, "group offsets of d_ff <= 32768");
    __shared__ __attribute__((aligned(16))) uint8_t L[bk::DX::LDS];
    if ((int)blockIdx.x < n_fill) {
        csc_fill_block(blockIdx.x, row_nnz, row_slot, ell_col, T, K, dff, masks, blkpre, lp, gt,
                       csc, status, (int *)L);
        return;
    }
    bk::dxdw_block<DT>(blockIdx.x - n_fill, bw, wu, wg, n_ovf_p, max_ovf, dm, dff, dwd, dwu, dwg,
                       L);
}

// ------------------------------------------------------------ 5'. dx, XCD-local
// XCD k (workgroup b % 8) sums slice k of dx[t] for four tokens per workgroup:
// per entry the slices of wu_t[i] and wg_t[i] (adjacent in the copy) with
// the entry's du and dg. Backup rows get the sum of their dense product's
// partials for the slice.
template <int DT, int SPL, int G>
__global__ __launch_bounds__(NT) void bwd_dxs_kernel(
    SliceSrc src, int dff, Slices sl, const int32_t *__restrict__ row_nnz,
    const int32_t *__restrict__ row_slot, const int16_t *__restrict__ ell_col,
    const float *__restrict__ coef, int T, int K, int dm, float *__restrict__ dx, BkPart bp,
    int max_ovf)
{
    constexpr int EPW = DT == TWELL_BF16 ? 2 : 1;
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int k = blockIdx.x % NXCD;
    const int t = (blockIdx.x / NXCD) * (NT / 64) + wv;
    const int nk = sl.valid(k);
    if (t >= T || nk == 0)
        return;
    const int slot = row_slot[t];
    if (slot >= 0) {
        if (bp.part && slot < max_ovf)
            bk_finish_row<SPL, EPW>(bp, slot, sl.ndw, k * sl.sww, k * sl.sww + nk, lane,
                                    dx + (size_t)t * dm);
        return;
    }
    const int n = min(row_nnz[t], K);
    const size_t TK = (size_t)T * K, rb = (size_t)t * K;
    // one descriptor over this XCD's slice of every wu_t row, one over wg_t's;
    // a lane's word offsets are clamped to the slice, words past nk are never
    // stored
    const int rowb = src.rowb;
    const __amdgpu_buffer_rsrc_t rs_u = slice_rsrc(src.a + (size_t)k * src.kstride, dff, src);
    const __amdgpu_buffer_rsrc_t rs_g = slice_rsrc(src.b + (size_t)k * src.kstride, dff, src);
    int offq[SPL];
#pragma unroll
    for (int q = 0; q < SPL; ++q)
        offq[q] = min(q * 64 + lane, src.lim - 1) * 4;
    float acc[SPL][EPW];
#pragma unroll
    for (int q = 0; q < SPL; ++q)
#pragma unroll
        for (int e = 0; e < EPW; ++e)
            acc[q][e] = 0.f;
    for (int eb = 0; eb < n; eb += 64) {
        const int m = min(64, n - eb), s = eb + lane;
        int ci = 0;
        float cu = 0.f, cg = 0.f;
        if (lane < m) {
            ci = ell_col[rb + s];
            cu = coef[rb + s];
            cg = coef[TK + rb + s];
            if (ci < 0 || ci >= dff) {
                ci = 0;
                cu = cg = 0.f;
            }
        }
        // the row's two slices (W_u's, then W_g's)
        uint32_t vu[G][SPL], vg[G][SPL];
        auto fetch = [&](int e, uint32_t (&u)[SPL], uint32_t (&g)[SPL]) {
            const int rc = bcast(ci, min(e, m - 1)) * rowb;
#pragma unroll
            for (int q = 0; q < SPL; ++q) {
                u[q] = __builtin_amdgcn_raw_buffer_load_b32(rs_u, rc + offq[q], 0, 0);
                g[q] = __builtin_amdgcn_raw_buffer_load_b32(rs_g, rc + offq[q], 0, 0);
            }
        };
#pragma unroll
        for (int g = 0; g < G; ++g)
            fetch(g, vu[g], vg[g]);
        for (int e0 = 0; e0 < m; e0 += G) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int e = e0 + g;
                if (e < m) { // uniform
                    const float a = bcast(cu, e), b = bcast(cg, e);
#pragma unroll
                    for (int q = 0; q < SPL; ++q) {
                        if constexpr (EPW == 2) {
                            acc[q][0] += a * bf16_lo(vu[g][q]);
                            acc[q][1] += a * bf16_hi(vu[g][q]);
                            acc[q][0] += b * bf16_lo(vg[g][q]);
                            acc[q][1] += b * bf16_hi(vg[g][q]);
                        } else {
                            acc[q][0] += a * __uint_as_float(vu[g][q]);
                            acc[q][0] += b * __uint_as_float(vg[g][q]);
                        }
                    }
                }
                fetch(e + G, vu[g], vg[g]);
            }
        }
    }
    float *row = dx + (size_t)t * dm + (size_t)k * sl.sww * EPW;
#pragma unroll
    for (int q = 0; q < SPL; ++q) {
        const int w = q * 64 + lane;
        if (w < nk) {
            if constexpr (EPW == 2)
                *(float2 *)(row + 2 * w) = make_float2(acc[q][0], acc[q][1]);
            else
                row[w] = acc[q][0];
        }
    }
}

template <int DT, int NW>
void launch_all(const void *x, const void *dy, const hybrid_t *h, const void *wg, const void *wu,
                const void *wd, int dm, float l1, float *dx, float *dwg, float *dwu, float *dwd,
                uint8_t *ws, int32_t *status, Timer &tm, hipStream_t s)
{
    const int T = h->T, K = h->K, dff = h->d_ff;
    const Layout L = layout(DT, T, dm, dff, K, h->max_ovf);
    float *coef = (float *)(ws + L.coef);
    uint64_t *masks = (uint64_t *)(ws + L.masks);
    int32_t *cnt = (int32_t *)(ws + L.cnt), *lp = (int32_t *)(ws + L.lp);
    int32_t *gt = (int32_t *)(ws + L.gt);
    int32_t *csc = (int32_t *)(ws + L.csc);
    const uint8_t *xb = (const uint8_t *)x, *dyb = (const uint8_t *)dy;
    const int rgroups = (T + NT / 64 - 1) / (NT / 64);
    constexpr int NWN = NW < 16 ? NW : 16;          // neuron pass: accumulated words per lane
    // entries in flight per wave (neuron pass, dx pass): one beyond the
    // narrowest rows, since resident waves hide the gathers' latency better
    // than a second register buffer does; waves sharing one neuron's entries
    // (narrow rows only: wide rows leave no registers for it)
    constexpr int GN = 1;
    constexpr int GD = NW <= 4 ? 4 : 1;
    constexpr int NSPLIT = NW <= 8 ? 4 : 1;
    constexpr int NWP = NW < ACC_NW ? NW : ACC_NW; // dx pass: words per lane of one part
    const int parts = row_parts<DT>(dm, NWP);

    const Slices sl = slices(DT, dm);
    uint32_t *wsl = (uint32_t *)(ws + L.wsl);
    if (T > 0) {
        const int n_chunk = (dff + CH - 1) / CH, n_mask = L.nblk * n_chunk;
        const int n_copy = L.split ? copy_groups(dff) : 0;
        const BkGather bg = bk_gather(DT, dm, dff, h->max_ovf, ws + L.backup);
        hipLaunchKernelGGL((mask_kernel<DT>), dim3(n_mask + n_copy + bg.blocks), dim3(NT), 0, s,
                           h->row_nnz, h->row_slot, h->ell_col, T, K, dff, masks, cnt, n_chunk,
                           n_mask, n_copy, (const uint32_t *)wu, (const uint32_t *)wg, wsl, sl,
                           bg, xb, dyb, h->ovf_rows, h->n_ovf, h->max_ovf, dm);
        tm.mark("mask_kernel");
    }
    // the backup rows' products (none without backup capacity or rows)
    const BkBwd bw = T > 0 ? bk_bwd(DT, dm, dff, h->max_ovf, ws + L.backup) : BkBwd{};
    const int n_grp = (dff + 63) / 64;
    hipLaunchKernelGGL((prefix_ud_kernel<DT>), dim3(n_grp + bw.n_ud), dim3(bk::UD_NT), 0, s, cnt,
                       L.nblk, dff, lp, gt, n_grp, bw, xb, dyb, h->ovf_rows, h->n_ovf, h->max_ovf,
                       (const uint8_t *)wu, (const uint8_t *)wd, dm, h->dense, l1);
    tm.mark("prefix_ud_kernel");
    const int n_fill = (T + FILL_ROWS - 1) / FILL_ROWS;
    if (n_fill + bw.n_dx + bw.n_dw > 0) {
        hipLaunchKernelGGL((fill_dxdw_kernel<DT>), dim3(n_fill + bw.n_dx + bw.n_dw), dim3(NT), 0,
                           s, h->row_nnz, h->row_slot, h->ell_col, T, K, dff, masks, cnt, lp, gt,
                           csc, status, n_fill, bw, (const uint8_t *)wu, (const uint8_t *)wg,
                           h->n_ovf, h->max_ovf, dm, dwd, dwu, dwg);
        tm.mark("fill_dxdw_kernel");
    }
    hipLaunchKernelGGL((bwd_neuron_kernel<DT, NW, NWN, GN, NSPLIT>), dim3(dff, NW / NWN),
                       dim3(64 * NSPLIT), 0, s, lp, gt, csc, h->ell_val, T, K, dff, xb, dyb,
                       (const uint8_t *)wu, (const uint8_t *)wd, dm, l1, coef, dwg, dwu, dwd,
                       h->n_ovf, h->max_ovf);
    tm.mark("bwd_neuron_kernel");
    if (T > 0) {
        const BkPart bp = bk_part(DT, dm, dff, h->max_ovf, true, ws + L.backup);
        if (L.split) {
            const SliceSrc src = slice_src_copy(wsl, 2, dff, sl);
            const int spl = (sl.sww + 63) / 64;
            const dim3 grid(rgroups * NXCD);
            if (spl <= 1)
                hipLaunchKernelGGL((bwd_dxs_kernel<DT, 1, 8>), grid, dim3(NT), 0, s, src, dff, sl,
                                   h->row_nnz, h->row_slot, h->ell_col, coef, T, K, dm, dx, bp,
                                   h->max_ovf);
            else if (spl == 2)
                hipLaunchKernelGGL((bwd_dxs_kernel<DT, 2, 4>), grid, dim3(NT), 0, s, src, dff, sl,
                                   h->row_nnz, h->row_slot, h->ell_col, coef, T, K, dm, dx, bp,
                                   h->max_ovf);
            else
                hipLaunchKernelGGL((bwd_dxs_kernel<DT, 4, 2>), grid, dim3(NT), 0, s, src, dff, sl,
                                   h->row_nnz, h->row_slot, h->ell_col, coef, T, K, dm, dx, bp,
                                   h->max_ovf);
            tm.mark("bwd_dxs_kernel");
        } else {
            hipLaunchKernelGGL((bwd_dx_kernel<DT, NWP, GD>), dim3(rgroups, parts), dim3(NT), 0, s,
                               h->row_nnz, h->row_slot, h->ell_col, coef, T, K, dff,
                               (const uint8_t *)wu, (const uint8_t *)wg, dm, dx, bp, h->max_ovf);
            tm.mark("bwd_dx_kernel");
        }
    }
}

template <int DT>
void launch_dt(const void *x, const void *dy, const hybrid_t *h, const void *wg, const void *wu,
               const void *wd, int dm, float l1, float *dx, float *dwg, float *dwu, float *dwd,
               uint8_t *ws, int32_t *status, Timer &tm, hipStream_t s)
{
#define TW_CASE(N) \
    case N: launch_all<DT, N>(x, dy, h, wg, wu, wd, dm, l1, dx, dwg, dwu, dwd, ws, status, tm, s); break;
    switch (row_nw<DT>(dm)) {
        TW_CASE(1) TW_CASE(2) TW_CASE(4) TW_CASE(8) TW_CASE(16)
    default: launch_all<DT, 32>(x, dy, h, wg, wu, wd, dm, l1, dx, dwg, dwu, dwd, ws, status, tm, s);
    }
#undef TW_CASE
}

} // namespace

size_t bwd_workspace_layout(int dt, int T, int dm, int dff, int K, int max_ovf)
{
    return layout(dt, T, dm, dff, K, max_ovf).total;
}

hipError_t launch_bwd(twell_dtype dt, const void *x, const void *dy, const hybrid_t *h,
                      const void *wg_t, const void *wu_t, const void *wd, int dm, float l1,
                      float *dx, float *dwg_t, float *dwu_t, float *dwd, void *ws,
                      int32_t *status, twell_timing_t *timing, hipStream_t s)
{
    Timer tm(timing, s);
    if (dt == TWELL_BF16)
        launch_dt<TWELL_BF16>(x, dy, h, wg_t, wu_t, wd, dm, l1, dx, dwg_t, dwu_t, dwd,
                              (uint8_t *)ws, status, tm, s);
    else
        launch_dt<TWELL_F32>(x, dy, h, wg_t, wu_t, wd, dm, l1, dx, dwg_t, dwu_t, dwd,
                             (uint8_t *)ws, status, tm, s);
    return hipGetLastError();
}
