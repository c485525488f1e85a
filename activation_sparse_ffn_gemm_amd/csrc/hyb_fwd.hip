// Training forward over the hybrid layout ("Sparser, Faster, Lighter
// Transformer Language Models", summary page section 2.B.3: the hybrid
// ELL + dense-backup layout carries the training forward as well as the
// backward).
//
// y[t] = sum over row t's entries (i, h) of  a * wd[i],  a = h * (x[t] . wu_t[i]).
//
// ELL rows (few nonzeros): a wave per row gathers one wu_t row and one wd row
// per entry, as the TwELL forward does, several entries in flight.
// Backup rows (many nonzeros, dense): two MFMA products over the rows'
// stored h (backup.hip),
//   A = h (.) (x_O W_u)   [n_ovf x d_ff],   y_O = A W_d   [n_ovf x d_model],
// with A kept as a float32 intermediate (for bf16 inputs as a hi/lo bf16 pair,
// so the second product keeps about 16 significant bits of A).
//
// Small layers: the backup products first, then the ELL rows' kernel, which
// also stores each backup row's y (the sum of the products' split-K partials).
// Large layers (the XCD-split ELL passes): the two parts write disjoint rows
// of y and read only what the conversion wrote, so the backup products and a
// launch that sums their partials into the backup rows' y run on a second
// stream of the device, beside the ELL passes (MFMA-bound tiles beside
// gathers bound by memory requests); the call's stream waits for them before
// its next work. The fork and join cost about 15 us of host time and more
// than two empty launches on the device, which a small layer does not win
// back. Under graph capture, and when per-kernel timing is asked for, all
// kernels run in order on the call's stream.
#include "backup.hpp"
#include "rows.hpp"
#include "side.hpp"


bool hyb_use_split(int dt, int T, int dm, int dff);
size_t hyb_split_workspace(int dt, int T, int dm, int dff, int K);
void launch_hyb_split(twell_dtype dt, const void *x, const hybrid_t *h, const void *wu,
                      const void *wd, int dm, float *y, void *ws, int32_t *status, Timer &tm,
                      hipStream_t s);

namespace {

constexpr int NT = 256; // 4 waves = 4 rows per workgroup

// ---------------------------------------------------------------- ELL rows
template <int DT, int NW, int NWP, int G>
__global__ __launch_bounds__(NT) void hfwd_ell_kernel(
    const uint8_t *__restrict__ x, const int32_t *__restrict__ row_nnz,
    const int32_t *__restrict__ row_slot, const int16_t *__restrict__ ell_col,
    const void *__restrict__ ell_val, int T, int K, int dff, const uint8_t *__restrict__ wu,
    const uint8_t *__restrict__ wd, int dm, float *__restrict__ y, BkPart bp, int max_ovf,
    int32_t *__restrict__ status)
{
    using E = elem<DT>;
    using R = Row<DT, NW>;   // whole row, for the up dot product
    using RP = Row<DT, NWP>; // this wave's part of the row, for the down projection
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (NT / 64) + wave_id();
    if (t >= T)
        return;
    const R geo(dm, lane, 0);
    const RP part(dm, lane, blockIdx.y);
    const int slot = row_slot[t];
    if (slot >= 0) { // a backup row: y is the sum of the dense product's partials
        if (bp.part && slot < max_ovf)
            bk_finish_row<NWP, RP::EPW>(bp, slot, part.ndw, part.base, part.ndw, lane,
                                        y + (size_t)t * dm);
        return;
    }
    uint32_t xw[NW];
    geo.load_w(x, t, xw);
    float acc[NWP][RP::EPW];
    part.zero_f(acc);
    const int n = min(row_nnz[t], K);
    const size_t rb = (size_t)t * K;
    for (int s0 = 0; s0 < n; s0 += 64) {
        // lane e holds entry s0 + e; the wave then walks them in order
        const int s = s0 + lane;
        int ci = 0;
        float hv = 0.f;
        if (s < n) {
            ci = ell_col[rb + s];
            hv = E::load1(ell_val, rb + s);
            if (ci < 0 || ci >= dff) { // corrupt entry: skipped and reported
                raise_status(status, TWELL_DEV_BAD_INDEX);
                ci = 0;
                hv = 0.f;
            }
        }
        const int m = min(64, n - s0);
        // stream the m entries through G register buffers: the rows of entry
        // e + G are requested as soon as entry e has been used
        uint32_t vu[G][NW], vd[G][NWP];
        auto fetch = [&](int e, uint32_t (&u)[NW], uint32_t (&d)[NWP]) {
            const int c = bcast(ci, min(e, m - 1));
            geo.load_w(wu, c, u);
            part.load_w(wd, c, d);
        };
#pragma unroll
        for (int g = 0; g < G; ++g)
            fetch(g, vu[g], vd[g]);
        for (int e0 = 0; e0 < m; e0 += G) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int e = e0 + g;
                const float u = wave_sum(geo.dotw(xw, vu[g]));
                if (e < m) // uniform
                    part.axpy(acc, bcast(hv, e) * u, vd[g]);
                fetch(e + G, vu[g], vd[g]);
            }
        }
    }
    part.store_f(y, t, acc);
}

template <int DT, int NW>
void launch_nw(const void *x, const hybrid_t *h, const void *wu, const void *wd, int dm, float *y,
               uint8_t *ws, int32_t *status, Timer &tm, hipStream_t s)
{
    const int T = h->T, dff = h->d_ff;
    if (!hyb_use_split(DT, T, dm, dff)) {
        launch_bk_fwd((twell_dtype)DT, x, h, wu, wd, dm, y, ws, false, tm, s);
        const BkPart bp = bk_part(DT, dm, dff, h->max_ovf, false, ws);
        constexpr int NWP = NW < 16 ? NW : 16;
        constexpr int G = NW <= 4 ? 4 : 1; // entries in flight per wave (occupancy first)
        const int parts = row_parts<DT>(dm, NWP);
        hipLaunchKernelGGL((hfwd_ell_kernel<DT, NW, NWP, G>),
                           dim3((T + NT / 64 - 1) / (NT / 64), parts), dim3(NT), 0, s,
                           (const uint8_t *)x, h->row_nnz, h->row_slot, h->ell_col, h->ell_val, T,
                           h->K, dff, (const uint8_t *)wu, (const uint8_t *)wd, dm, y, bp,
                           h->max_ovf, status);
        tm.mark("hfwd_ell_kernel");
        return;
    }
    // many tokens, large weights: XCD-local ELL passes on s; fork: the backup
    // products on the side stream after everything already on s; join: s
    // waits for them after its own kernels
    SideStream *ss = h->max_ovf > 0 && T > 0 && !tm.t ? side_stream(s) : nullptr;
    std::unique_lock<std::mutex> lk;
    if (ss && !side_fork(ss, s, lk))
        ss = nullptr;
    launch_bk_fwd((twell_dtype)DT, x, h, wu, wd, dm, y, ws, true, tm, ss ? ss->s : s);
    const bool marked = ss && side_mark(ss, 1);
    const size_t off = (bk_workspace(DT, dm, dff, h->max_ovf, false) + 255) & ~(size_t)255;
    launch_hyb_split((twell_dtype)DT, x, h, wu, wd, dm, y, ws + off, status, tm, s);
    if (ss)
        side_wait(ss, 1, marked, s);
}

template <int DT>
void launch_dt(const void *x, const hybrid_t *h, const void *wu, const void *wd, int dm, float *y,
               uint8_t *ws, int32_t *status, Timer &tm, hipStream_t s)
{
#define TW_CASE(N) \
    case N: launch_nw<DT, N>(x, h, wu, wd, dm, y, ws, status, tm, s); break;
    switch (row_nw<DT>(dm)) {
        TW_CASE(1) TW_CASE(2) TW_CASE(4) TW_CASE(8) TW_CASE(16)
    default: launch_nw<DT, 32>(x, h, wu, wd, dm, y, ws, status, tm, s); break;
    }
#undef TW_CASE
}

} // namespace

// The backup rows' products (their intermediate A, W_d^T and the split-K
// partials of y_O).
size_t hyb_fwd_workspace(int dt, int T, int dm, int max_ovf, int dff, int K)
{
    const size_t bk = (bk_workspace(dt, dm, dff, max_ovf, false) + 255) & ~(size_t)255;
    return bk + (hyb_use_split(dt, T, dm, dff) ? hyb_split_workspace(dt, T, dm, dff, K) : 0);
}

hipError_t launch_hyb_fwd(twell_dtype dt, const void *x, const hybrid_t *h, const void *wu_t,
                          const void *wd, int dm, float *y, void *ws, int32_t *status,
                          twell_timing_t *timing, hipStream_t s)
{
    Timer tm(timing, s);
    if (dt == TWELL_BF16)
        launch_dt<TWELL_BF16>(x, h, wu_t, wd, dm, y, (uint8_t *)ws, status, tm, s);
    else
        launch_dt<TWELL_F32>(x, h, wu_t, wd, dm, y, (uint8_t *)ws, status, tm, s);
    return hipGetLastError();
}
