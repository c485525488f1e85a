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
// stored h,
//   A = h (.) (x_O W_u)   [n_ovf x d_ff],   y_O = A W_d   [n_ovf x d_model],
// with A kept as a float32 intermediate (for bf16 inputs as a hi/lo bf16 pair,
// so the second product keeps about 16 significant bits of A).
#include "mfma_tile.hpp"
#include "rows.hpp"

namespace {

constexpr int NT = 256; // 4 waves = 4 rows per workgroup

// ---------------------------------------------------------------- ELL rows
template <int DT, int NW, int NWP, int G>
__global__ __launch_bounds__(NT) void hfwd_ell_kernel(
    const uint8_t *__restrict__ x, const int32_t *__restrict__ row_nnz,
    const int32_t *__restrict__ row_slot, const int16_t *__restrict__ ell_col,
    const void *__restrict__ ell_val, int T, int K, int dff, const uint8_t *__restrict__ wu,
    const uint8_t *__restrict__ wd, int dm, float *__restrict__ y, int32_t *__restrict__ status)
{
    using E = elem<DT>;
    using R = Row<DT, NW>;   // whole row, for the up dot product
    using RP = Row<DT, NWP>; // this wave's part of the row, for the down projection
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
    if (t >= T || row_slot[t] >= 0)
        return; // a backup row's y comes from the dense products
    const R geo(dm, lane, 0);
    const RP part(dm, lane, blockIdx.y);
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

// ---------------------------------------------------------------- backup rows
// A = h (.) (x_O W_u) for one 128 x 128 tile (backup rows x neurons).
template <int DT>
__global__ __launch_bounds__(mt::NT, 2) void hfwd_a_kernel(
    const uint8_t *__restrict__ x, const int32_t *__restrict__ ovf_rows,
    const int32_t *__restrict__ n_ovf_p, int max_ovf, const uint8_t *__restrict__ wu, int dm,
    int dff, const void *__restrict__ dense, void *__restrict__ inter, size_t stride)
{
    using E = elem<DT>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[mt::TILE_LDS];
    mt::Tiles As = (mt::Tiles)lds, Bs = As + 2;
    const int n_ovf = min(*n_ovf_p, max_ovf);
    const int m0 = blockIdx.y * mt::TILE, n0 = blockIdx.x * mt::TILE;
    if (m0 >= n_ovf)
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const size_t rowbytes = (size_t)dm * sizeof(typename E::storage);
    const int nk = (int)(rowbytes / mt::ROWB);
    int src[4]; // token row of each staged A row (-1 past n_ovf)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid + mt::NT * i) >> 3;
        src[i] = m0 + r < n_ovf ? ovf_rows[m0 + r] : -1;
    }
    auto load_a = [&](mt::Stage &st, int kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = (tid + mt::NT * i) & 7;
            st.v[i] = src[i] >= 0 ? ldg16(x + (size_t)src[i] * rowbytes + (size_t)kt * mt::ROWB + c * 16)
                                  : make_uint4(0, 0, 0, 0);
        }
    };
    auto load_b = [&](mt::Stage &st, int kt) {
        mt::load_k(st, [&](int r) { return wu + (size_t)(n0 + r) * rowbytes + (size_t)kt * mt::ROWB; },
                   tid);
    };
    auto put = [&](uint8_t *S, const mt::Stage &st) { mt::store_k(S, st, tid); };
    mt::Acc au;
    mt::zero(au);
    mt::gemm<DT>(au, As, Bs, nk, load_a, put, load_b, put, wm, wn, lane);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + mt::acc_row(wm, mi, e, lane);
                if (m >= n_ovf)
                    continue;
                const size_t o = (size_t)m * dff + n0 + mt::acc_col(wn, ni, lane);
                mt::put_inter<DT>(inter, stride, 0, o, E::load1(dense, o) * au[mi][ni][e]);
            }
}

// y_O = A W_d for one 128 x 128 tile (backup rows x model columns), written to
// the rows' places in y.
template <int DT>
__global__ __launch_bounds__(mt::NT, 2) void hfwd_y_kernel(
    const void *__restrict__ inter, size_t stride, const int32_t *__restrict__ ovf_rows,
    const int32_t *__restrict__ n_ovf_p, int max_ovf, const uint8_t *__restrict__ wd, int dm,
    int dff, float *__restrict__ y)
{
    using E = elem<DT>;
    constexpr int esz = sizeof(typename E::storage);
    constexpr int KE = mt::ROWB / esz;
    constexpr int NSEG = DT == TWELL_BF16 ? 2 : 1; // (A hi, A lo) or A
    __shared__ __attribute__((aligned(16))) uint8_t lds[mt::TILE_LDS];
    mt::Tiles As = (mt::Tiles)lds, Bs = As + 2;
    const int n_ovf = min(*n_ovf_p, max_ovf);
    const int m0 = blockIdx.y * mt::TILE, n0 = blockIdx.x * mt::TILE;
    if (m0 >= n_ovf)
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const size_t rowbytes = (size_t)dm * esz;
    const int spseg = dff / KE; // K steps per segment
    const uint8_t *ibase = (const uint8_t *)inter;
    auto load_a = [&](mt::Stage &st, int kt) {
        const int seg = kt / spseg, k0 = (kt % spseg) * KE;
        const uint8_t *arr = ibase + (size_t)seg * stride * esz;
        mt::load_k(st, [&](int r) {
            return m0 + r < n_ovf ? arr + ((size_t)(m0 + r) * dff + k0) * esz : (const uint8_t *)nullptr;
        }, tid);
    };
    auto load_b = [&](mt::Stage &st, int kt) {
        const int k0 = (kt % spseg) * KE;
        mt::load_mn<DT>(st, [&](int kk) { return wd + (size_t)(k0 + kk) * rowbytes + (size_t)n0 * esz; },
                        [&](int r0) { return n0 + r0 < dm; }, tid);
    };
    auto put_a = [&](uint8_t *S, const mt::Stage &st) { mt::store_k(S, st, tid); };
    auto put_b = [&](uint8_t *S, const mt::Stage &st) { mt::store_mn<DT>(S, st, tid); };
    mt::Acc acc;
    mt::zero(acc);
    mt::gemm<DT>(acc, As, Bs, NSEG * spseg, load_a, put_a, load_b, put_b, wm, wn, lane);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int m = m0 + mt::acc_row(wm, mi, e, lane);
            if (m >= n_ovf)
                continue;
            const size_t yrow = (size_t)ovf_rows[m] * dm;
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int n = n0 + mt::acc_col(wn, ni, lane);
                if (n < dm)
                    y[yrow + n] = acc[mi][ni][e];
            }
        }
}

size_t pad_rows(int max_ovf) { return (size_t)(max_ovf + mt::TILE - 1) / mt::TILE * mt::TILE; }

template <int DT, int NW>
void launch_nw(const void *x, const hybrid_t *h, const void *wu, const void *wd, int dm, float *y,
               uint8_t *ws, int32_t *status, Timer &tm, hipStream_t s)
{
    const int T = h->T, dff = h->d_ff;
    if (h->max_ovf > 0) {
        const size_t stride = pad_rows(h->max_ovf) * dff;
        const int mt_tiles = (int)(pad_rows(h->max_ovf) / mt::TILE);
        hipLaunchKernelGGL((hfwd_a_kernel<DT>), dim3(dff / mt::TILE, mt_tiles), dim3(mt::NT), 0, s,
                           (const uint8_t *)x, h->ovf_rows, h->n_ovf, h->max_ovf,
                           (const uint8_t *)wu, dm, dff, h->dense, ws, stride);
        tm.mark("hfwd_a_kernel");
        hipLaunchKernelGGL((hfwd_y_kernel<DT>), dim3((dm + mt::TILE - 1) / mt::TILE, mt_tiles),
                           dim3(mt::NT), 0, s, ws, stride, h->ovf_rows, h->n_ovf, h->max_ovf,
                           (const uint8_t *)wd, dm, dff, y);
        tm.mark("hfwd_y_kernel");
    }
    constexpr int NWP = NW < 16 ? NW : 16;
    constexpr int G = NW <= 4 ? 4 : (NW <= 16 ? 2 : 1); // entries in flight per wave
    const int parts = row_parts<DT>(dm, NWP);
    hipLaunchKernelGGL((hfwd_ell_kernel<DT, NW, NWP, G>), dim3((T + NT / 64 - 1) / (NT / 64), parts),
                       dim3(NT), 0, s, (const uint8_t *)x, h->row_nnz, h->row_slot, h->ell_col,
                       h->ell_val, T, h->K, dff, (const uint8_t *)wu, (const uint8_t *)wd, dm, y,
                       status);
    tm.mark("hfwd_ell_kernel");
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

// A's float32 intermediate: a hi/lo pair of bf16 arrays or one float32 array,
// each [rows of the backup, padded to whole tiles][d_ff].
size_t hyb_fwd_workspace(int max_ovf, int dff) { return 4 * pad_rows(max_ovf) * (size_t)dff; }

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
