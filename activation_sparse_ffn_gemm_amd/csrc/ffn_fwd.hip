// Fused up and down projections over the TwELL nonzeros ("Sparser, Faster,
// Lighter Transformer Language Models", summary page section 2.B.2: one kernel
// applies the up and down projections to the nonzero gate entries only).
//
// y[t] = sum over stored (i, h) of row t of  a * wd[i],  a = h * (x[t] . wu_t[i]).
//
// One wave64 owns one token (and, for wide rows, one part of d_model for the
// output): x[t] and the float32 accumulator of y[t] stay in registers, the
// row's entries are staged in LDS in ascending column order, and per nonzero
// the wave gathers one wu_t row (the up column) and one wd row (the down
// row), each a contiguous d_model vector read with 4-byte lanes (rows.hpp),
// several nonzeros in flight at once. a is never written to memory.
#include "rows.hpp"

namespace {

constexpr int NT = 256;   // 4 waves = 4 tokens per workgroup
constexpr int LIST = 256; // entries staged in LDS per pass

// Stage the stored entries of row t, tiles [j0, j1), into LDS: element e of
// the list is (slot within the row = j * W + s, column, value). Calls fn(ne)
// after each pass of up to LIST entries, with the list visible to the wave.
// A lane reads the slots of one tile, 8 independent loads at a time. With
// VALS false only slots and columns are staged (val is not read).
template <int DT, bool VALS, class Fn>
DEVI void for_row_entries(const int32_t *count, const int16_t *col, const void *val, int t,
                          int nt, int W, int j0, int j1, int dff, int lane, int *lslot,
                          int *lcol, float *lval, int32_t *status, Fn fn)
{
    using E = elem<DT>;
    for (int jb = j0; jb < j1; jb += 64) {
        const int j = jb + lane;
        const int n = j < j1 ? min(count[(size_t)t * nt + j], W) : 0;
        const int incl = wave_incl_scan(n, lane);
        const int excl = incl - n;
        const int tot = __shfl(incl, 63, 64);
        const size_t src = ((size_t)t * nt + j) * W;
        for (int p0 = 0; p0 < tot; p0 += LIST) {
            for (int s0 = max(0, p0 - excl); s0 < n && excl + s0 < p0 + LIST; s0 += 8) {
                // branch-free: every lane issues its 8 (or 16) loads before any
                // is used; slots past the tile's width re-read its last slot
                int c[8];
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const size_t q = src + min(s0 + u, W - 1);
                    c[u] = col[q];
                    v[u] = VALS ? E::load1(val, q) : 0.f;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (s0 + u >= n)
                        c[u] = 0, v[u] = 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int e = excl + s0 + u - p0;
                    if (s0 + u < n && e < LIST) {
                        if (c[u] < 0 || c[u] >= dff) { // corrupt entry: skipped and reported
                            raise_status(status, TWELL_DEV_BAD_INDEX);
                            c[u] = 0;
                            v[u] = 0.f;
                        }
                        lslot[e] = j * W + s0 + u;
                        lcol[e] = c[u];
                        lval[e] = v[u];
                    }
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            fn(min(LIST, tot - p0));
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// ---------------------------------------------------------------- fused
template <int DT, int NW, int NWP, int G>
__global__ __launch_bounds__(NT) void ffn_fwd_kernel(
    const uint8_t *__restrict__ x, const int32_t *__restrict__ count,
    const int16_t *__restrict__ col, const void *__restrict__ val, int T, int nt, int W,
    const uint8_t *__restrict__ wu, const uint8_t *__restrict__ wd, int dm,
    float *__restrict__ y, int32_t *__restrict__ status)
{
    using R = Row<DT, NW>;   // whole row, for the up dot product
    using RP = Row<DT, NWP>; // this wave's part of the row, for the down projection
    __shared__ int lslot[NT / 64][LIST], lcol[NT / 64][LIST];
    __shared__ float lval[NT / 64][LIST];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = blockIdx.x * (NT / 64) + wv;
    if (t >= T)
        return;
    const R geo(dm, lane, 0);
    const RP part(dm, lane, blockIdx.y);
    uint32_t xw[NW];
    geo.load_w(x, t, xw);
    float acc[NWP][RP::EPW];
    part.zero_f(acc);
    for_row_entries<DT, true>(count, col, val, t, nt, W, 0, nt, nt * TWELL_TILE_C, lane,
                              lslot[wv], lcol[wv], lval[wv], status, [&](int ne) {
        // Stream the staged entries through G register buffers: the rows of
        // entry e + G are requested as soon as entry e has been used, so G
        // entries' gathers stay in flight while the wave computes. Requests
        // past the list re-read its last entry and are not used.
        uint32_t vu[G][NW], vd[G][NWP];
        auto fetch = [&](int e, uint32_t (&u)[NW], uint32_t (&d)[NWP]) {
            const int ci = lcol[wv][min(e, ne - 1)];
            geo.load_w(wu, ci, u);
            part.load_w(wd, ci, d);
        };
#pragma unroll
        for (int g = 0; g < G; ++g)
            fetch(g, vu[g], vd[g]);
        for (int e0 = 0; e0 < ne; e0 += G) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int e = e0 + g;
                const float u = wave_sum(geo.dotw(xw, vu[g]));
                if (e < ne) // uniform
                    part.axpy(acc, lval[wv][e] * u, vd[g]);
                fetch(e + G, vu[g], vd[g]);
            }
        }
    });
    part.store_f(y, t, acc);
}

template <int DT, int NW>
void launch_nw(const void *x, const twell_t *h, const void *wu, const void *wd, int dm, float *y,
               int32_t *status, hipStream_t s)
{
    constexpr int NWP = NW < 16 ? NW : 16; // whole rows up to d_model 2048 (bf16)
    constexpr int G = NW <= 4 ? 4 : (NW <= 16 ? 2 : 1); // entries in flight per wave
    const int parts = row_parts<DT>(dm, NWP);
    const int groups = (h->T + NT / 64 - 1) / (NT / 64);
    hipLaunchKernelGGL((ffn_fwd_kernel<DT, NW, NWP, G>), dim3(groups, parts), dim3(NT), 0, s,
                       (const uint8_t *)x, h->count, h->col, h->val, h->T,
                       h->d_ff / TWELL_TILE_C, h->width, (const uint8_t *)wu,
                       (const uint8_t *)wd, dm, y, status);
}

template <int DT>
void launch_dt(const void *x, const twell_t *h, const void *wu, const void *wd, int dm, float *y,
               int32_t *status, hipStream_t s)
{
    switch (row_nw<DT>(dm)) {
    case 1: launch_nw<DT, 1>(x, h, wu, wd, dm, y, status, s); break;
    case 2: launch_nw<DT, 2>(x, h, wu, wd, dm, y, status, s); break;
    case 4: launch_nw<DT, 4>(x, h, wu, wd, dm, y, status, s); break;
    case 8: launch_nw<DT, 8>(x, h, wu, wd, dm, y, status, s); break;
    case 16: launch_nw<DT, 16>(x, h, wu, wd, dm, y, status, s); break;
    default: launch_nw<DT, 32>(x, h, wu, wd, dm, y, status, s); break;
    }
}

} // namespace

size_t fwd_workspace(int, int, int) { return 0; }

hipError_t launch_ffn_fwd(twell_dtype dt, const void *x, const twell_t *h, const void *wu_t,
                          const void *wd, int dm, float *y, void *, int32_t *status,
                          twell_timing_t *timing, hipStream_t s)
{
    Timer tm(timing, s);
    if (dt == TWELL_BF16)
        launch_dt<TWELL_BF16>(x, h, wu_t, wd, dm, y, status, s);
    else
        launch_dt<TWELL_F32>(x, h, wu_t, wd, dm, y, status, s);
    tm.mark("ffn_fwd_kernel");
    return hipGetLastError();
}
