// Up and down projections over the TwELL nonzeros only ("Sparser, Faster,
// Lighter Transformer Language Models", summary page section 2.B.2: the up
// and down projections applied to the nonzero gate entries, nothing else).
//
// y[t] = sum over stored (i, h) of row t of  a * wd[i],  a = h * (x[t] . wu_t[i]).
//
// Every gathered row is a contiguous d_model vector (wu_t and wd rows are
// both [d_ff][d_model]), read with 4-byte lanes through a per-row buffer
// descriptor (rows.hpp). Two designs:
//
// Many tokens and large weights: two passes, each giving every XCD a working set
// that stays in its own 4 MB L2 (workgroup b runs on XCD b % 8):
//   up:   XCD k owns the neuron tiles [k nt / 8, (k+1) nt / 8). A wave per
//         token holds x[t] in registers, gathers the wu_t rows of its
//         entries in those tiles and writes a = h u for each, with the entry's
//         column, into the token's compact entry list (entries of all tiles in
//         column order, so each XCD's share is one contiguous run). When a
//         slice of a wd row is not a run of whole 128-byte lines in place,
//         extra workgroups copy wd into a slice-major layout (slices.hpp).
//   down: XCD k owns the k-th eighth of the d_model columns. A wave per token
//         walks the token's compact list and gathers, per entry, only the
//         slice of the wd row (in place, or in that copy), accumulating
//         y[t]'s slice.
// Otherwise: one fused pass, a wave per token doing both projections, a is
// never written to memory.
#include "backup.hpp"
#include "rows.hpp"
#include "slices.hpp"

namespace {

constexpr int NT = 256;       // 4 waves = 4 tokens per workgroup
constexpr int LIST = 256;     // entries staged in LDS per pass
// The two-pass design pays for its extra traffic (x read by every XCD, the
// wd copy, the entry lists) only with many tokens and weights well beyond
// one XCD's L2; otherwise the fused pass is faster.
constexpr int SPLIT_T = 1024;                 // tokens
constexpr size_t SPLIT_W = (size_t)16 << 20;  // bytes of one weight matrix

inline bool use_split(int dt, int T, int dm, int dff)
{
    return T >= SPLIT_T && (size_t)dff * dm * (dt == TWELL_BF16 ? 2 : 4) >= SPLIT_W;
}

// Stage the stored entries of row t, tiles [j0, j1), into LDS: element e of
// the list is (column, value). Calls fn(p0, ne) after each pass of up to LIST
// entries, p0 being the index of the pass's first entry among the range's
// entries (in column order). A lane reads the slots of one tile, 4
// independent loads at a time (most tiles hold one or two entries; eight at a
// time cost the fused 0.5B pass a wave per SIMD), through buffer descriptors
// over row t's slots: 32-bit offsets instead of 64-bit addresses keep the
// staging's registers few (measured: the 1.5B up pass about 10% faster).
// Slots past a tile's count (the next tile's, or past the row: 0 from the
// range check) are read but never used. With VALS false val is not read.
template <int DT, bool VALS, class Fn>
DEVI void for_row_entries(const int32_t *count, const int16_t *col, const void *val, int t,
                          int nt, int W, int j0, int j1, int dff, int lane, int *lcol, float *lval,
                          int32_t *status, Fn fn)
{
    constexpr int VB = DT == TWELL_BF16 ? 2 : 4; // bytes of one stored value
    const size_t slot0 = (size_t)__builtin_amdgcn_readfirstlane(t) * nt * W;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(col + slot0), (short)0, nt * W * 2, BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const uint8_t *)val + slot0 * VB), (short)0, nt * W * VB, BUF_DWORD3);
    int done = 0; // entries of earlier 64-tile chunks
    for (int jb = j0; jb < j1; jb += 64) {
        const int j = jb + lane;
        const int n = j < j1 ? min(count[(size_t)t * nt + j], W) : 0;
        const int incl = wave_incl_scan(n, lane);
        const int excl = incl - n;
        const int tot = __shfl(incl, 63, 64);
        for (int p0 = 0; p0 < tot; p0 += LIST) {
            for (int s0 = max(0, p0 - excl); s0 < n && excl + s0 < p0 + LIST; s0 += 4) {
                // branch-free: every lane issues its loads before any is used
                const int q = j * W + s0;
                int c[4];
                float v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    c[u] = (int16_t)__builtin_amdgcn_raw_buffer_load_b16(rc, (q + u) * 2, 0, 0);
                    if constexpr (!VALS)
                        v[u] = 0.f;
                    else if constexpr (DT == TWELL_BF16)
                        v[u] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rv, (q + u) * 2, 0, 0));
                    else
                        v[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rv, (q + u) * 4, 0, 0));
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int e = excl + s0 + u - p0;
                    if (s0 + u < n && e < LIST) {
                        if (c[u] < 0 || c[u] >= dff) { // corrupt entry: skipped and reported
                            raise_status(status, TWELL_DEV_BAD_INDEX);
                            c[u] = 0;
                            v[u] = 0.f;
                        }
                        lcol[e] = c[u];
                        lval[e] = v[u];
                    }
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            fn(done + p0, min(LIST, tot - p0));
            __builtin_amdgcn_wave_barrier();
        }
        done += tot;
    }
}

// Stored entries of row t in tiles [0, j) (.x) and in all tiles (.y).
DEVI int2 row_counts(const int32_t *count, int t, int nt, int W, int j, int lane)
{
    int below = 0, all = 0;
    for (int jb = 0; jb < nt; jb += 64) {
        const int jj = jb + lane;
        const int n = jj < nt ? min(count[(size_t)t * nt + jj], W) : 0;
        below += __shfl(wave_incl_scan(jj < j ? n : 0, lane), 63, 64);
        all += __shfl(wave_incl_scan(n, lane), 63, 64);
    }
    return make_int2(below, all);
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
    __shared__ int lcol[NT / 64][LIST];
    __shared__ float lval[NT / 64][LIST];
    const int lane = threadIdx.x & 63, wv = wave_id();
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
                              lcol[wv], lval[wv], status, [&](int, int ne) {
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

// ---------------------------------------------------------------- split
// Workspace of the two-pass design: slice-major wd (if copied), then the compact entry
// lists (a as float32, columns as int16) and their lengths.
struct FwdLayout {
    size_t wds, ac, cc, rn, total;
    int cap;
};

inline size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

inline FwdLayout fwd_layout(int dt, int T, int dm, int dff, int W)
{
    FwdLayout L;
    const Slices sl = slices(dt, dm);
    L.cap = dff / TWELL_TILE_C * W;
    size_t o = 0;
    L.wds = o; o += up256(slice_copy_bytes(1, dff, sl));
    L.ac = o;  o += up256((size_t)T * L.cap * 4);
    L.cc = o;  o += up256((size_t)T * L.cap * 2);
    L.rn = o;  o += up256((size_t)T * 4);
    L.total = o;
    return L;
}

DEVI void copy_slices(int b, const uint32_t *__restrict__ wd, uint32_t *__restrict__ wds, int dff,
                      Slices sl)
{
    copy_slices_rows<1, NT>(b, wd, nullptr, wds, dff, sl);
}

template <int DT, int NW, int G>
__global__ __launch_bounds__(NT) void fwd_up_kernel(
    const uint8_t *__restrict__ x, const int32_t *__restrict__ count,
    const int16_t *__restrict__ col, const void *__restrict__ val, int T, int nt, int W,
    const uint8_t *__restrict__ wu, int dm, int n_copy, const uint32_t *__restrict__ wd,
    uint32_t *__restrict__ wds, int dff, Slices sl, float *__restrict__ ac,
    int16_t *__restrict__ cc, int32_t *__restrict__ rn, int cap, int32_t *__restrict__ status)
{
    using R = Row<DT, NW>;
    __shared__ int lcol[NT / 64][LIST];
    __shared__ float lval[NT / 64][LIST];
    const int lane = threadIdx.x & 63, wv = wave_id();
    int b = blockIdx.x;
    if (b < n_copy) {
        copy_slices(b, wd, wds, dff, sl);
        return;
    }
    b -= n_copy; // n_copy is a multiple of 8: b % 8 is still the XCD
    const int k = b % NXCD;
    const int t = (b / NXCD) * (NT / 64) + wv;
    if (t >= T)
        return;
    // x[t] is requested first: its latency then overlaps the count scan and
    // the staging of the entry list instead of delaying the first dot product
    const R geo(dm, lane, 0);
    uint32_t xw[NW];
    geo.load_w(x, t, xw);
    const int j0 = k * nt / NXCD, j1 = (k + 1) * nt / NXCD;
    const int2 cnt = row_counts(count, t, nt, W, j0, lane);
    if (k == 0 && lane == 0)
        rn[t] = cnt.y;
    if (j0 >= j1)
        return;
    float *arow = ac + (size_t)t * cap + cnt.x;
    int16_t *crow = cc + (size_t)t * cap + cnt.x;
    for_row_entries<DT, true>(count, col, val, t, nt, W, j0, j1, dff, lane, lcol[wv], lval[wv],
                              status, [&](int p0, int ne) {
        for (int eb = 0; eb < ne; eb += 64) {
            const int m = min(64, ne - eb);
            // stream the m entries through G register buffers; lane e keeps
            // entry e's a and writes it, with its column, at the end
            uint32_t vu[G][NW];
            auto fetch = [&](int e, uint32_t (&u)[NW]) {
                geo.load_w(wu, lcol[wv][eb + min(e, m - 1)], u);
            };
#pragma unroll
            for (int g = 0; g < G; ++g)
                fetch(g, vu[g]);
            float mine = 0.f;
            for (int e0 = 0; e0 < m; e0 += G) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int e = e0 + g;
                    const float u = wave_sum(geo.dotw(xw, vu[g]));
                    if (lane == e && e < m)
                        mine = lval[wv][eb + e] * u;
                    fetch(e + G, vu[g]);
                }
            }
            if (lane < m) {
                arow[p0 + eb + lane] = mine;
                crow[p0 + eb + lane] = (int16_t)lcol[wv][eb + lane];
            }
        }
    });
}

// Up pass over a hybrid's ELL rows (the forward over the hybrid): XCD k takes
// the entries whose column lies in its neuron tiles (k = 0 also takes corrupt
// columns, which are reported and get a = 0), so every slot of every ELL row
// gets its a = h u written exactly once, in place: ac[t][s] beside
// ell_col[t][s], which the down pass reads as the entry list. Backup rows are
// left to the dense products.
template <int DT, int NW, int G>
__global__ __launch_bounds__(NT) void hfwd_up_kernel(
    const uint8_t *__restrict__ x, const int32_t *__restrict__ row_nnz,
    const int32_t *__restrict__ row_slot, const int16_t *__restrict__ ell_col,
    const void *__restrict__ ell_val, int T, int K, int nt, const uint8_t *__restrict__ wu,
    int dm, int n_copy, const uint32_t *__restrict__ wd, uint32_t *__restrict__ wds, int dff,
    Slices sl, float *__restrict__ ac, int32_t *__restrict__ status)
{
    using E = elem<DT>;
    using R = Row<DT, NW>;
    __shared__ int lcol[NT / 64][64];
    __shared__ int lslot[NT / 64][64];
    __shared__ float lval[NT / 64][64];
    const int lane = threadIdx.x & 63, wv = wave_id();
    int b = blockIdx.x;
    if (b < n_copy) {
        copy_slices(b, wd, wds, dff, sl);
        return;
    }
    b -= n_copy; // n_copy is a multiple of 8: b % 8 is still the XCD
    const int k = b % NXCD;
    const int t = (b / NXCD) * (NT / 64) + wv;
    if (t >= T || row_slot[t] >= 0)
        return;
    const int c0 = (k * nt / NXCD) * TWELL_TILE_C, c1 = ((k + 1) * nt / NXCD) * TWELL_TILE_C;
    const int n = min(row_nnz[t], K);
    const size_t rb = (size_t)t * K;
    const R geo(dm, lane, 0);
    uint32_t xw[NW];
    bool have_x = false;
    const uint64_t below = (1ull << lane) - 1ull;
    for (int s0 = 0; s0 < n; s0 += 64) {
        const int s = s0 + lane;
        int c = 0;
        float h = 0.f;
        bool mine = false;
        if (s < n) {
            c = ell_col[rb + s];
            h = E::load1(ell_val, rb + s);
            const bool bad = c < 0 || c >= dff;
            mine = bad ? k == 0 : (c >= c0 && c < c1);
            if (mine && bad) {
                raise_status(status, TWELL_DEV_BAD_INDEX);
                c = 0;
                h = 0.f;
            }
        }
        const uint64_t msk = __ballot(mine);
        const int m = __popcll(msk);
        if (m == 0) // uniform
            continue;
        if (!have_x) {
            geo.load_w(x, t, xw);
            have_x = true;
        }
        if (mine) {
            const int r = __popcll(msk & below);
            lcol[wv][r] = c;
            lslot[wv][r] = s;
            lval[wv][r] = h;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // stream the m entries through G register buffers; lane e keeps entry
        // e's a and writes it at the end
        uint32_t vu[G][NW];
        auto fetch = [&](int e, uint32_t (&u)[NW]) { geo.load_w(wu, lcol[wv][min(e, m - 1)], u); };
#pragma unroll
        for (int g = 0; g < G; ++g)
            fetch(g, vu[g]);
        float a = 0.f;
        for (int e0 = 0; e0 < m; e0 += G) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int e = e0 + g;
                const float u = wave_sum(geo.dotw(xw, vu[g]));
                if (lane == e && e < m)
                    a = lval[wv][e] * u;
                fetch(e + G, vu[g]);
            }
        }
        if (lane < m)
            ac[rb + lslot[wv][lane]] = a;
        __builtin_amdgcn_wave_barrier(); // the lists are rewritten by the next chunk
    }
}

// Down pass: y[t][slice k] from the token's (a, column) list. For the forward
// over a hybrid (row_slot non-null) the list is the ELL row itself; backup
// rows are skipped (their y rows come from the dense products).
template <int DT, int SPL, int G>
__global__ __launch_bounds__(NT) void fwd_down_kernel(
    SliceSrc src, int dff, Slices sl, const float *__restrict__ ac,
    const int16_t *__restrict__ cc, const int32_t *__restrict__ rn, int cap, int T, int dm,
    float *__restrict__ y, const int32_t *__restrict__ row_slot)
{
    constexpr int EPW = DT == TWELL_BF16 ? 2 : 1;
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int k = blockIdx.x % NXCD;
    const int t = (blockIdx.x / NXCD) * (NT / 64) + wv;
    const int nk = sl.valid(k);
    if (t >= T || nk == 0 || (row_slot && row_slot[t] >= 0))
        return;
    const int n = min(rn[t], cap);
    const float *arow = ac + (size_t)t * cap;
    const int16_t *crow = cc + (size_t)t * cap;
    // one descriptor over this XCD's slice of every wd row; a lane's word
    // offsets are clamped to the slice (words past nk are never stored)
    const int rowb = src.rowb;
    const __amdgpu_buffer_rsrc_t rs_all = slice_rsrc(src.a + (size_t)k * src.kstride, dff, src);
    int offq[SPL];
#pragma unroll
    for (int q = 0; q < SPL; ++q)
        offq[q] = min(q * 64 + lane, src.lim - 1) * 4;
    float acc[SPL][EPW];
#pragma unroll
    for (int c = 0; c < SPL; ++c)
#pragma unroll
        for (int e = 0; e < EPW; ++e)
            acc[c][e] = 0.f;
    for (int eb = 0; eb < n; eb += 64) {
        const int m = min(64, n - eb);
        const int ci = lane < m ? crow[eb + lane] : 0;
        const float av = lane < m ? arow[eb + lane] : 0.f;
        uint32_t v[G][SPL];
        auto fetch = [&](int e, uint32_t (&w)[SPL]) {
            const int c = min(max(bcast(ci, min(e, m - 1)), 0), dff - 1);
#pragma unroll
            for (int q = 0; q < SPL; ++q)
                w[q] = __builtin_amdgcn_raw_buffer_load_b32(rs_all, c * rowb + offq[q], 0, 0);
        };
#pragma unroll
        for (int g = 0; g < G; ++g)
            fetch(g, v[g]);
        for (int e0 = 0; e0 < m; e0 += G) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int e = e0 + g;
                if (e < m) { // uniform
                    const float a = bcast(av, e);
#pragma unroll
                    for (int q = 0; q < SPL; ++q) {
                        if constexpr (EPW == 2) {
                            acc[q][0] += a * bf16_lo(v[g][q]);
                            acc[q][1] += a * bf16_hi(v[g][q]);
                        } else {
                            acc[q][0] += a * __uint_as_float(v[g][q]);
                        }
                    }
                }
                fetch(e + G, v[g]);
            }
        }
    }
    float *yrow = y + (size_t)t * dm + (size_t)k * sl.sww * EPW;
#pragma unroll
    for (int q = 0; q < SPL; ++q) {
        const int w = q * 64 + lane;
        if (w < nk) {
            if constexpr (EPW == 2)
                *(float2 *)(yrow + 2 * w) = make_float2(acc[q][0], acc[q][1]);
            else
                yrow[w] = acc[q][0];
        }
    }
}

template <int DT, int NW>
void launch_nw(const void *x, const twell_t *h, const void *wu, const void *wd, int dm, float *y,
               uint8_t *ws, int32_t *status, Timer &tm, hipStream_t s)
{
    const int T = h->T, nt = h->d_ff / TWELL_TILE_C, dff = h->d_ff;
    const int groups = (T + NT / 64 - 1) / (NT / 64);
    if (!use_split(DT, T, dm, dff)) {
        constexpr int NWP = NW < 16 ? NW : 16; // whole rows up to d_model 2048 (bf16)
        // entries in flight per wave: one for rows of 1 KB and more, where the
        // registers of a second would cost a wave per SIMD (the gathers are
        // latency-bound: resident waves hide more than deeper buffers)
        constexpr int G = NW <= 4 ? 4 : 1;
        const int parts = row_parts<DT>(dm, NWP);
        hipLaunchKernelGGL((ffn_fwd_kernel<DT, NW, NWP, G>), dim3(groups, parts), dim3(NT), 0, s,
                           (const uint8_t *)x, h->count, h->col, h->val, T, nt, h->width,
                           (const uint8_t *)wu, (const uint8_t *)wd, dm, y, status);
        tm.mark("ffn_fwd_kernel");
        return;
    }
    const Slices sl = slices(DT, dm);
    const FwdLayout L = fwd_layout(DT, T, dm, dff, h->width);
    uint32_t *wds = (uint32_t *)(ws + L.wds);
    float *ac = (float *)(ws + L.ac);
    int16_t *cc = (int16_t *)(ws + L.cc);
    int32_t *rn = (int32_t *)(ws + L.rn);
    const int n_copy = sl.direct ? 0 : copy_groups(dff);
    const SliceSrc src = sl.direct ? slice_src_direct(wd, nullptr, sl) : slice_src_copy(wds, 1, dff, sl);
    constexpr int GU = NW <= 8 ? 2 : 1; // entries in flight per wave (occupancy first)
    hipLaunchKernelGGL((fwd_up_kernel<DT, NW, GU>), dim3(n_copy + groups * NXCD), dim3(NT), 0, s,
                       (const uint8_t *)x, h->count, h->col, h->val, T, nt, h->width,
                       (const uint8_t *)wu, dm, n_copy, (const uint32_t *)wd, wds, dff, sl, ac,
                       cc, rn, L.cap, status);
    tm.mark("fwd_up_kernel");
    const int spl = (sl.sww + 63) / 64;
    if (spl <= 1)
        hipLaunchKernelGGL((fwd_down_kernel<DT, 1, 8>), dim3(groups * NXCD), dim3(NT), 0, s, src,
                           dff, sl, ac, cc, rn, L.cap, T, dm, y, nullptr);
    else if (spl == 2)
        hipLaunchKernelGGL((fwd_down_kernel<DT, 2, 8>), dim3(groups * NXCD), dim3(NT), 0, s, src,
                           dff, sl, ac, cc, rn, L.cap, T, dm, y, nullptr);
    else
        hipLaunchKernelGGL((fwd_down_kernel<DT, 4, 4>), dim3(groups * NXCD), dim3(NT), 0, s, src,
                           dff, sl, ac, cc, rn, L.cap, T, dm, y, nullptr);
    tm.mark("fwd_down_kernel");
}

template <int DT>
void launch_dt(const void *x, const twell_t *h, const void *wu, const void *wd, int dm, float *y,
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

// ---- the forward over a hybrid's ELL rows, two-pass form (hyb_fwd.hip)
bool hyb_use_split(int dt, int T, int dm, int dff) { return use_split(dt, T, dm, dff); }

// slice-major wd copy (unless read in place), then a per ELL slot (float32 [T][K])
size_t hyb_split_workspace(int dt, int T, int dm, int dff, int K)
{
    const Slices sl = slices(dt, dm);
    return up256(slice_copy_bytes(1, dff, sl)) + up256((size_t)T * K * 4);
}

namespace {
template <int DT, int NW>
void launch_hyb_split_nw(const void *x, const hybrid_t *h, const void *wu, const void *wd, int dm,
                         float *y, uint8_t *ws, int32_t *status, Timer &tm, hipStream_t s)
{
    const int T = h->T, dff = h->d_ff, nt = dff / TWELL_TILE_C;
    const int groups = (T + NT / 64 - 1) / (NT / 64);
    const Slices sl = slices(DT, dm);
    uint32_t *wds = (uint32_t *)ws;
    float *ac = (float *)(ws + up256(slice_copy_bytes(1, dff, sl)));
    const int n_copy = sl.direct ? 0 : copy_groups(dff);
    const SliceSrc src = sl.direct ? slice_src_direct(wd, nullptr, sl) : slice_src_copy(wds, 1, dff, sl);
    constexpr int GU = NW <= 8 ? 2 : 1;
    hipLaunchKernelGGL((hfwd_up_kernel<DT, NW, GU>), dim3(n_copy + groups * NXCD), dim3(NT), 0, s,
                       (const uint8_t *)x, h->row_nnz, h->row_slot, h->ell_col, h->ell_val, T,
                       h->K, nt, (const uint8_t *)wu, dm, n_copy, (const uint32_t *)wd, wds, dff,
                       sl, ac, status);
    tm.mark("hfwd_up_kernel");
    const int spl = (sl.sww + 63) / 64;
    if (spl <= 1)
        hipLaunchKernelGGL((fwd_down_kernel<DT, 1, 8>), dim3(groups * NXCD), dim3(NT), 0, s, src,
                           dff, sl, ac, h->ell_col, h->row_nnz, h->K, T, dm, y, h->row_slot);
    else if (spl == 2)
        hipLaunchKernelGGL((fwd_down_kernel<DT, 2, 8>), dim3(groups * NXCD), dim3(NT), 0, s, src,
                           dff, sl, ac, h->ell_col, h->row_nnz, h->K, T, dm, y, h->row_slot);
    else
        hipLaunchKernelGGL((fwd_down_kernel<DT, 4, 4>), dim3(groups * NXCD), dim3(NT), 0, s, src,
                           dff, sl, ac, h->ell_col, h->row_nnz, h->K, T, dm, y, h->row_slot);
    tm.mark("hfwd_down_kernel");
}
} // namespace

void launch_hyb_split(twell_dtype dt, const void *x, const hybrid_t *h, const void *wu,
                      const void *wd, int dm, float *y, void *ws, int32_t *status, Timer &tm,
                      hipStream_t s)
{
#define TW_CASE(D, N) \
    case N: launch_hyb_split_nw<D, N>(x, h, wu, wd, dm, y, (uint8_t *)ws, status, tm, s); break;
    if (dt == TWELL_BF16) {
        switch (row_nw<TWELL_BF16>(dm)) {
            TW_CASE(TWELL_BF16, 1) TW_CASE(TWELL_BF16, 2) TW_CASE(TWELL_BF16, 4)
            TW_CASE(TWELL_BF16, 8) TW_CASE(TWELL_BF16, 16)
        default: launch_hyb_split_nw<TWELL_BF16, 32>(x, h, wu, wd, dm, y, (uint8_t *)ws, status, tm, s);
        }
    } else {
        switch (row_nw<TWELL_F32>(dm)) {
            TW_CASE(TWELL_F32, 1) TW_CASE(TWELL_F32, 2) TW_CASE(TWELL_F32, 4)
            TW_CASE(TWELL_F32, 8) TW_CASE(TWELL_F32, 16)
        default: launch_hyb_split_nw<TWELL_F32, 32>(x, h, wu, wd, dm, y, (uint8_t *)ws, status, tm, s);
        }
    }
#undef TW_CASE
}

size_t dec_ffn_workspace(int dt, int T, int dm, int dff, int W);
hipError_t launch_dec_ffn(twell_dtype dt, const void *x, const twell_t *h, const void *wu_t,
                          const void *wd, int dm, float *y, void *ws, int32_t *status, Timer &tm,
                          hipStream_t s);

size_t fwd_workspace(int dt, int T, int dm, int dff, int W)
{
    if (T <= TWELL_DECODE_T)
        return dec_ffn_workspace(dt, T, dm, dff, W);
    return use_split(dt, T, dm, dff) ? fwd_layout(dt, T, dm, dff, W).total : 0;
}

hipError_t launch_ffn_fwd(twell_dtype dt, const void *x, const twell_t *h, const void *wu_t,
                          const void *wd, int dm, float *y, void *ws, int32_t *status,
                          twell_timing_t *timing, hipStream_t s)
{
    Timer tm(timing, s);
    if (h->T <= TWELL_DECODE_T) // few tokens: up and down over the whole chip
        return launch_dec_ffn(dt, x, h, wu_t, wd, dm, y, ws, status, tm, s);
    if (dt == TWELL_BF16)
        launch_dt<TWELL_BF16>(x, h, wu_t, wd, dm, y, (uint8_t *)ws, status, tm, s);
    else
        launch_dt<TWELL_F32>(x, h, wu_t, wd, dm, y, (uint8_t *)ws, status, tm, s);
    return hipGetLastError();
}
