// Backward of y = (h (.) x W_u) W_d on the pattern P of a hybrid ELL + dense
// backup ("Sparser, Faster, Lighter Transformer Language Models", summary page
// section 2.B.3: sparse-to-dense and dense-to-sparse products in the backward,
// no dense work on zeros; overflow rows live in a dense backup).
//
// With u = x W_u and da = dy W_d^T sampled on P, a = h u, du = da h, dg = da u:
//   dx = du W_u^T + dg W_g^T,  dW_d = a^T dy,  dW_u = x^T du,  dW_g = x^T dg.
//
// ELL rows (gathers, fp32 accumulation):
//   1. token pass: one wave per ELL row computes u and da for each entry
//      (dense-to-sparse dots with the entry's wu_t and wd rows), keeps the
//      entry's (a, du, dg) and accumulates dx[t] from the entry's wu_t and
//      wg_t rows (sparse-to-dense);
//   2. a stable column transpose of the ELL entries (per-block histograms,
//      a scan, and an in-order fill), so the weight gradients need no atomics
//      and sum each neuron's entries in ascending row order (deterministic);
//   3. neuron pass: one wave per neuron sums its entries' x and dy rows into
//      its dW rows, writing every row (zero for unused neurons).
// Backup rows (dense MFMA, fp32 accumulation):
//   4. U/DA: u and da of every backup row and neuron (two 128x128-tile GEMMs
//      over d_model), then a, du, dg (dg zero where h is zero);
//   5. DX:   dx of backup rows = [du | dg] [W_u ; W_g]^T, scattered to their rows;
//   6. DW:   dW += [a | du | dg]^T [dy | x | x] over the backup rows.
// For bf16 inputs, the fp32 intermediates a, du, dg enter the MFMA as a pair
// of bf16 (hi + lo, 16 significant bits), so products 5 and 6 run over a K
// twice as long; fp32 inputs use fp32 MFMA directly.
#include "mfma_tile.hpp"

namespace {

constexpr int NT = 256;
constexpr int TB = 64;     // rows per block of the column transpose
constexpr int CH = 16384;  // columns per LDS chunk of the transpose (64 KB of counters)

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
    size_t coef, cnt, colptr, csc, inter, total;
    int nblk, pad_ovf;
};

Layout layout(int T, int dff, int K, int max_ovf)
{
    Layout L;
    L.nblk = (T + TB - 1) / TB;
    L.pad_ovf = (max_ovf + mt::TILE - 1) / mt::TILE * mt::TILE;
    size_t o = 0;
    L.coef = o;   o += up256((size_t)3 * T * K * 4);
    L.cnt = o;    o += up256((size_t)L.nblk * dff * 4);
    L.colptr = o; o += up256((size_t)(dff + 1) * 4);
    L.csc = o;    o += up256((size_t)T * K * 4);
    L.inter = o;  o += up256((size_t)12 * L.pad_ovf * dff); // 6 bf16 or 3 f32 arrays
    L.total = o;
    return L;
}

// ------------------------------------------------------------ 1. ELL token pass
template <int DT, int NCH, int G>
__global__ __launch_bounds__(NT) void bwd_ell_kernel(
    const uint8_t *__restrict__ x, const uint8_t *__restrict__ dy,
    const int32_t *__restrict__ row_nnz, const int32_t *__restrict__ row_slot,
    const int16_t *__restrict__ ell_col, const void *__restrict__ ell_val, int T, int K, int dff,
    const uint8_t *__restrict__ wg, const uint8_t *__restrict__ wu, const uint8_t *__restrict__ wd,
    int dm, float *__restrict__ dx, float *__restrict__ coef, int32_t *__restrict__ status)
{
    using E = elem<DT>;
    constexpr int P = E::per16;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
    if (t >= T || row_slot[t] >= 0)
        return; // a backup row's dx comes from the dense products
    const size_t rowbytes = (size_t)dm * sizeof(typename E::storage);
    const size_t TK = (size_t)T * K;

    float xr[NCH][P], dr[NCH][P], acc[NCH][P];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const size_t off = (size_t)(c * 64 + lane) * 16;
        const bool in = off < rowbytes;
        E::widen(in ? ldg16(x + (size_t)t * rowbytes + off) : make_uint4(0, 0, 0, 0), xr[c]);
        E::widen(in ? ldg16(dy + (size_t)t * rowbytes + off) : make_uint4(0, 0, 0, 0), dr[c]);
#pragma unroll
        for (int k = 0; k < P; ++k)
            acc[c][k] = 0.f;
    }
    const int n = min(row_nnz[t], K);
    for (int s0 = 0; s0 < n; s0 += G) {
        int ci[G];
        float hv[G];
        bool ok[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int s = s0 + g;
            int c = 0;
            float h = 0.f;
            if (s < n) {
                c = ell_col[(size_t)t * K + s];
                h = E::load1(ell_val, (size_t)t * K + s);
                if (c < 0 || c >= dff) {
                    raise_status(status, TWELL_DEV_BAD_INDEX);
                    c = 0;
                    h = 0.f;
                }
            }
            ci[g] = c;
            hv[g] = h;
            ok[g] = s < n && h != 0.f;
        }
        uint4 vu[G][NCH], vd[G][NCH], vg[G][NCH];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const size_t off = (size_t)(c * 64 + lane) * 16;
                const bool in = ok[g] && off < rowbytes;
                const size_t ro = (size_t)ci[g] * rowbytes + off;
                vu[g][c] = in ? ldg16(wu + ro) : make_uint4(0, 0, 0, 0);
                vd[g][c] = in ? ldg16(wd + ro) : make_uint4(0, 0, 0, 0);
                vg[g][c] = in ? ldg16(wg + ro) : make_uint4(0, 0, 0, 0);
            }
        float pu[G], pd[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float su = 0.f, sd = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                float w1[P], w2[P];
                E::widen(vu[g][c], w1);
                E::widen(vd[g][c], w2);
#pragma unroll
                for (int k = 0; k < P; ++k) {
                    su += xr[c][k] * w1[k];
                    sd += dr[c][k] * w2[k];
                }
            }
            pu[g] = su;
            pd[g] = sd;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            pu[g] = wave_sum(pu[g]);
            pd[g] = wave_sum(pd[g]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int s = s0 + g;
            if (s >= n)
                continue;
            const float u = pu[g], da = pd[g], h = hv[g];
            const float a = ok[g] ? h * u : 0.f, du = ok[g] ? da * h : 0.f, dg = ok[g] ? da * u : 0.f;
            if (lane == 0) {
                const size_t e = (size_t)t * K + s;
                coef[e] = a;
                coef[TK + e] = du;
                coef[2 * TK + e] = dg;
            }
            if (ok[g]) {
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    float w1[P], w3[P];
                    E::widen(vu[g][c], w1);
                    E::widen(vg[g][c], w3);
#pragma unroll
                    for (int k = 0; k < P; ++k)
                        acc[c][k] += du * w1[k] + dg * w3[k];
                }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const size_t el = (size_t)(c * 64 + lane) * P;
        if (el < (size_t)dm) {
            float4 *d = (float4 *)(dx + (size_t)t * dm + el);
#pragma unroll
            for (int q = 0; q < P / 4; ++q)
                d[q] = make_float4(acc[c][4 * q], acc[c][4 * q + 1], acc[c][4 * q + 2], acc[c][4 * q + 3]);
        }
    }
}

// ------------------------------------------------------------ 2. column transpose
DEVI bool ell_row(const int32_t *row_slot, int t) { return row_slot[t] < 0; }

__global__ __launch_bounds__(NT) void csc_hist_kernel(
    const int32_t *__restrict__ row_nnz, const int32_t *__restrict__ row_slot,
    const int16_t *__restrict__ ell_col, int T, int K, int dff, int32_t *__restrict__ cnt)
{
    extern __shared__ int hist[];
    const int b = blockIdx.x, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c0 = blockIdx.y * CH, c1 = min(dff, c0 + CH);
    for (int i = threadIdx.x; i < c1 - c0; i += NT)
        hist[i] = 0;
    __syncthreads();
    for (int t = b * TB + wv; t < min(T, (b + 1) * TB); t += NT / 64) {
        if (!ell_row(row_slot, t))
            continue;
        const int n = min(row_nnz[t], K);
        for (int s = lane; s < n; s += 64) {
            const int c = ell_col[(size_t)t * K + s];
            if (c >= c0 && c < c1)
                atomicAdd(&hist[c - c0], 1);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < c1 - c0; i += NT)
        cnt[(size_t)b * dff + c0 + i] = hist[i];
}

// per column: exclusive prefix over blocks (in place); column totals to colptr
__global__ __launch_bounds__(NT) void csc_cols_kernel(int32_t *__restrict__ cnt, int nblk, int dff,
                                                      int32_t *__restrict__ colptr)
{
    const int i = blockIdx.x * NT + threadIdx.x;
    if (i >= dff)
        return;
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
        const int v = cnt[(size_t)b * dff + i];
        cnt[(size_t)b * dff + i] = run;
        run += v;
    }
    colptr[i] = run;
}

constexpr int SCAN_NT = 1024;

// in-place exclusive scan of colptr[0..dff); colptr[dff] = total
__global__ __launch_bounds__(SCAN_NT) void csc_colptr_kernel(int32_t *__restrict__ colptr, int dff)
{
    __shared__ int wsum[SCAN_NT / 64];
    __shared__ int carry;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (tid == 0)
        carry = 0;
    __syncthreads();
    for (int i0 = 0; i0 < dff; i0 += SCAN_NT) {
        const int i = i0 + tid;
        const int v = i < dff ? colptr[i] : 0;
        const int incl = wave_incl_scan(v, lane);
        if (lane == 63)
            wsum[wv] = incl;
        __syncthreads();
        int before = carry;
        for (int w = 0; w < wv; ++w)
            before += wsum[w];
        if (i < dff)
            colptr[i] = before + incl - v;
        __syncthreads();
        if (tid == SCAN_NT - 1)
            carry = before + incl;
        __syncthreads();
    }
    if (tid == 0)
        colptr[dff] = carry;
}

// one wave per block of TB rows, rows in ascending order: each entry goes to
// colptr[c] + (entries of column c in earlier blocks) + (earlier in this block)
__global__ __launch_bounds__(64) void csc_fill_kernel(
    const int32_t *__restrict__ row_nnz, const int32_t *__restrict__ row_slot,
    const int16_t *__restrict__ ell_col, int T, int K, int dff, const int32_t *__restrict__ cnt,
    const int32_t *__restrict__ colptr, int32_t *__restrict__ csc)
{
    extern __shared__ int cursor[];
    const int b = blockIdx.x, lane = threadIdx.x;
    const int c0 = blockIdx.y * CH, c1 = min(dff, c0 + CH);
    for (int i = lane; i < c1 - c0; i += 64)
        cursor[i] = 0;
    __syncthreads();
    for (int t = b * TB; t < min(T, (b + 1) * TB); ++t) {
        if (!ell_row(row_slot, t))
            continue;
        const int n = min(row_nnz[t], K);
        for (int s = lane; s < n; s += 64) {
            const int c = ell_col[(size_t)t * K + s];
            if (c >= c0 && c < c1) { // columns of a row are distinct, so lanes never collide
                const int r = cursor[c - c0];
                cursor[c - c0] = r + 1;
                csc[colptr[c] + cnt[(size_t)b * dff + c] + r] = t * K + s;
            }
        }
    }
}

// ------------------------------------------------------------ 3. neuron pass
template <int DT, int NCH>
__global__ __launch_bounds__(NT) void dw_ell_kernel(
    const uint8_t *__restrict__ x, const uint8_t *__restrict__ dy, int T, int K, int dff, int dm,
    const int32_t *__restrict__ colptr, const int32_t *__restrict__ csc,
    const float *__restrict__ coef, float *__restrict__ dwg, float *__restrict__ dwu,
    float *__restrict__ dwd)
{
    using E = elem<DT>;
    constexpr int P = E::per16;
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
    if (i >= dff)
        return;
    const size_t rowbytes = (size_t)dm * sizeof(typename E::storage);
    const long TK = (long)T * K;
    float ad[NCH][P], au[NCH][P], ag[NCH][P];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int k = 0; k < P; ++k)
            ad[c][k] = au[c][k] = ag[c][k] = 0.f;
    const int e1 = colptr[i + 1];
    for (int e = colptr[i]; e < e1; ++e) {
        const int idx = csc[e];
        if (idx < 0 || idx >= TK)
            continue;
        const int t = idx / K;
        const float a = coef[idx], du = coef[TK + idx], dg = coef[2 * TK + idx];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const size_t off = (size_t)(c * 64 + lane) * 16;
            if (off < rowbytes) {
                float xv[P], dv[P];
                E::widen(ldg16(x + (size_t)t * rowbytes + off), xv);
                E::widen(ldg16(dy + (size_t)t * rowbytes + off), dv);
#pragma unroll
                for (int k = 0; k < P; ++k) {
                    ad[c][k] += a * dv[k];
                    au[c][k] += du * xv[k];
                    ag[c][k] += dg * xv[k];
                }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const size_t el = (size_t)(c * 64 + lane) * P;
        if (el < (size_t)dm) {
            const size_t o = (size_t)i * dm + el;
#pragma unroll
            for (int q = 0; q < P / 4; ++q) {
                *(float4 *)(dwd + o + 4 * q) = make_float4(ad[c][4 * q], ad[c][4 * q + 1], ad[c][4 * q + 2], ad[c][4 * q + 3]);
                *(float4 *)(dwu + o + 4 * q) = make_float4(au[c][4 * q], au[c][4 * q + 1], au[c][4 * q + 2], au[c][4 * q + 3]);
                *(float4 *)(dwg + o + 4 * q) = make_float4(ag[c][4 * q], ag[c][4 * q + 1], ag[c][4 * q + 2], ag[c][4 * q + 3]);
            }
        }
    }
}

// ------------------------------------------------------------ 4-6. backup rows
// Intermediate arrays, each [pad_ovf][dff]: bf16 -> a_hi, a_lo, du_hi, du_lo,
// dg_hi, dg_lo; f32 -> a, du, dg.
template <int DT> DEVI void put_inter(void *inter, size_t stride, int q, size_t o, float v);
template <> DEVI void put_inter<TWELL_BF16>(void *inter, size_t stride, int q, size_t o, float v)
{
    uint16_t *p = (uint16_t *)inter;
    const uint16_t hi = f32_to_bf16(v);
    p[(2 * q) * stride + o] = hi;
    p[(2 * q + 1) * stride + o] = f32_to_bf16(v - bf16_to_f32(hi));
}
template <> DEVI void put_inter<TWELL_F32>(void *inter, size_t stride, int q, size_t o, float v)
{
    ((float *)inter)[q * stride + o] = v;
}

template <int DT>
__global__ __launch_bounds__(mt::NT, 2) void ovf_ud_kernel(
    const uint8_t *__restrict__ x, const uint8_t *__restrict__ dy,
    const int32_t *__restrict__ ovf_rows, const int32_t *__restrict__ n_ovf_p, int max_ovf,
    const uint8_t *__restrict__ wu, const uint8_t *__restrict__ wd, int dm, int dff,
    const void *__restrict__ dense, void *__restrict__ inter, size_t stride)
{
    using E = elem<DT>;
    const int n_ovf = min(*n_ovf_p, max_ovf);
    const int m0 = blockIdx.y * mt::TILE, n0 = blockIdx.x * mt::TILE;
    if (m0 >= n_ovf)
        return;
    __shared__ __attribute__((aligned(16))) uint8_t As[2][mt::TILE * mt::ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][mt::TILE * mt::ROWB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const size_t rowbytes = (size_t)dm * sizeof(typename E::storage);
    const int nk = (int)(rowbytes / mt::ROWB);
    int src[4]; // source row of each staged A row (-1 past n_ovf)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid + mt::NT * i) >> 3;
        src[i] = m0 + r < n_ovf ? ovf_rows[m0 + r] : -1;
    }
    auto gather_rows = [&](const uint8_t *base) {
        return [=](mt::Stage &st, int kt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = (tid + mt::NT * i) & 7;
                st.v[i] = src[i] >= 0 ? ldg16(base + (size_t)src[i] * rowbytes + (size_t)kt * mt::ROWB + c * 16)
                                      : make_uint4(0, 0, 0, 0);
            }
        };
    };
    auto weight_rows = [&](const uint8_t *base) {
        return [=](mt::Stage &st, int kt) {
            mt::load_k(st, [&](int r) { return base + (size_t)(n0 + r) * rowbytes + (size_t)kt * mt::ROWB; }, tid);
        };
    };
    auto put = [&](uint8_t *S, const mt::Stage &st) { mt::store_k(S, st, tid); };
    mt::Acc au, ad;
    mt::zero(au);
    mt::zero(ad);
    mt::gemm<DT>(au, As, Bs, nk, gather_rows(x), put, weight_rows(wu), put, wm, wn, lane);
    mt::gemm<DT>(ad, As, Bs, nk, gather_rows(dy), put, weight_rows(wd), put, wm, wn, lane);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + mt::acc_row(wm, mi, e, lane);
                if (m >= n_ovf)
                    continue;
                const int i = n0 + mt::acc_col(wn, ni, lane);
                const size_t o = (size_t)m * dff + i;
                const float h = E::load1(dense, o), u = au[mi][ni][e], da = ad[mi][ni][e];
                put_inter<DT>(inter, stride, 0, o, h * u);
                put_inter<DT>(inter, stride, 1, o, da * h);
                put_inter<DT>(inter, stride, 2, o, h != 0.f ? da * u : 0.f);
            }
}

template <int DT>
__global__ __launch_bounds__(mt::NT, 2) void ovf_dx_kernel(
    const void *__restrict__ inter, size_t stride, const int32_t *__restrict__ ovf_rows,
    const int32_t *__restrict__ n_ovf_p, int max_ovf, const uint8_t *__restrict__ wu,
    const uint8_t *__restrict__ wg, int dm, int dff, float *__restrict__ dx)
{
    using E = elem<DT>;
    constexpr int esz = sizeof(typename E::storage);
    constexpr int KE = mt::ROWB / esz;
    constexpr int NSEG = DT == TWELL_BF16 ? 4 : 2; // (du hi, du lo, dg hi, dg lo) or (du, dg)
    const int n_ovf = min(*n_ovf_p, max_ovf);
    const int m0 = blockIdx.y * mt::TILE, n0 = blockIdx.x * mt::TILE;
    if (m0 >= n_ovf)
        return;
    __shared__ __attribute__((aligned(16))) uint8_t As[2][mt::TILE * mt::ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][mt::TILE * mt::ROWB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const size_t rowbytes = (size_t)dm * esz;
    const int spseg = dff / KE; // K steps per segment
    const uint8_t *ibase = (const uint8_t *)inter;
    auto load_a = [&](mt::Stage &st, int kt) {
        const int seg = kt / spseg, k0 = (kt % spseg) * KE;
        const uint8_t *arr = ibase + (size_t)(NSEG == 4 ? 2 + seg : 1 + seg) * stride * esz;
        mt::load_k(st, [&](int r) {
            return m0 + r < n_ovf ? arr + ((size_t)(m0 + r) * dff + k0) * esz : (const uint8_t *)nullptr;
        }, tid);
    };
    auto load_b = [&](mt::Stage &st, int kt) {
        const int seg = kt / spseg, k0 = (kt % spseg) * KE;
        const uint8_t *w = seg < NSEG / 2 ? wu : wg;
        mt::load_mn<DT>(st, [&](int kk) { return w + (size_t)(k0 + kk) * rowbytes + (size_t)n0 * esz; },
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
            const size_t drow = (size_t)ovf_rows[m] * dm;
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int n = n0 + mt::acc_col(wn, ni, lane);
                if (n < dm)
                    dx[drow + n] = acc[mi][ni][e];
            }
        }
}

template <int DT>
__global__ __launch_bounds__(mt::NT, 2) void ovf_dw_kernel(
    const void *__restrict__ inter, size_t stride, const int32_t *__restrict__ ovf_rows,
    const int32_t *__restrict__ n_ovf_p, int max_ovf, const uint8_t *__restrict__ x,
    const uint8_t *__restrict__ dy, int dm, int dff, float *__restrict__ dwd,
    float *__restrict__ dwu, float *__restrict__ dwg)
{
    using E = elem<DT>;
    constexpr int esz = sizeof(typename E::storage);
    constexpr int KE = mt::ROWB / esz;
    constexpr int NSEG = DT == TWELL_BF16 ? 2 : 1; // hi, lo
    const int n_ovf = min(*n_ovf_p, max_ovf);
    if (n_ovf <= 0)
        return;
    __shared__ __attribute__((aligned(16))) uint8_t As[2][mt::TILE * mt::ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][mt::TILE * mt::ROWB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int z = blockIdx.z; // 0: dW_d from (a, dy); 1: dW_u from (du, x); 2: dW_g from (dg, x)
    const int i0 = blockIdx.y * mt::TILE, n0 = blockIdx.x * mt::TILE;
    const uint8_t *src = z == 0 ? dy : x;
    float *out = z == 0 ? dwd : (z == 1 ? dwu : dwg);
    const size_t rowbytes = (size_t)dm * esz;
    const int spseg = (n_ovf + KE - 1) / KE;
    const uint8_t *ibase = (const uint8_t *)inter;
    auto load_a = [&](mt::Stage &st, int kt) {
        const int seg = kt / spseg, k0 = (kt % spseg) * KE;
        const uint8_t *arr = ibase + (size_t)(NSEG * z + seg) * stride * esz;
        mt::load_mn<DT>(st, [&](int kk) {
            const int m = k0 + kk;
            return m < n_ovf ? arr + ((size_t)m * dff + i0) * esz : (const uint8_t *)nullptr;
        }, [&](int) { return true; }, tid);
    };
    auto load_b = [&](mt::Stage &st, int kt) {
        const int k0 = (kt % spseg) * KE;
        mt::load_mn<DT>(st, [&](int kk) {
            const int m = k0 + kk;
            return m < n_ovf ? src + (size_t)ovf_rows[m] * rowbytes + (size_t)n0 * esz
                             : (const uint8_t *)nullptr;
        }, [&](int r0) { return n0 + r0 < dm; }, tid);
    };
    auto put = [&](uint8_t *S, const mt::Stage &st) { mt::store_mn<DT>(S, st, tid); };
    mt::Acc acc;
    mt::zero(acc);
    mt::gemm<DT>(acc, As, Bs, NSEG * spseg, load_a, put, load_b, put, wm, wn, lane);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int i = i0 + mt::acc_row(wm, mi, e, lane);
                const int n = n0 + mt::acc_col(wn, ni, lane);
                if (n < dm)
                    out[(size_t)i * dm + n] += acc[mi][ni][e];
            }
}

template <int DT, int NCH>
hipError_t launch_nch(const void *x, const void *dy, const hybrid_t *h, const void *wg,
                      const void *wu, const void *wd, int dm, float *dx, float *dwg, float *dwu,
                      float *dwd, uint8_t *ws, int32_t *status, hipStream_t s)
{
    const int T = h->T, K = h->K, dff = h->d_ff;
    const Layout L = layout(T, dff, K, h->max_ovf);
    float *coef = (float *)(ws + L.coef);
    int32_t *cnt = (int32_t *)(ws + L.cnt), *colptr = (int32_t *)(ws + L.colptr);
    int32_t *csc = (int32_t *)(ws + L.csc);
    void *inter = ws + L.inter;
    const size_t stride = (size_t)L.pad_ovf * dff;
    const uint8_t *xb = (const uint8_t *)x, *dyb = (const uint8_t *)dy;
    constexpr int G = NCH <= 2 ? 2 : 1;
    const int nch = (dff + CH - 1) / CH;
    const size_t lds_hist = (size_t)min(dff, CH) * sizeof(int);

    if (T > 0) {
        hipLaunchKernelGGL((bwd_ell_kernel<DT, NCH, G>), dim3((T + 3) / 4), dim3(NT), 0, s, xb, dyb,
                           h->row_nnz, h->row_slot, h->ell_col, h->ell_val, T, K, dff,
                           (const uint8_t *)wg, (const uint8_t *)wu, (const uint8_t *)wd, dm, dx,
                           coef, status);
        hipLaunchKernelGGL(csc_hist_kernel, dim3(L.nblk, nch), dim3(NT), lds_hist, s, h->row_nnz,
                           h->row_slot, h->ell_col, T, K, dff, cnt);
    }
    hipLaunchKernelGGL(csc_cols_kernel, dim3((dff + NT - 1) / NT), dim3(NT), 0, s, cnt, L.nblk,
                       dff, colptr);
    hipLaunchKernelGGL(csc_colptr_kernel, dim3(1), dim3(SCAN_NT), 0, s, colptr, dff);
    if (T > 0)
        hipLaunchKernelGGL(csc_fill_kernel, dim3(L.nblk, nch), dim3(64), lds_hist, s, h->row_nnz,
                           h->row_slot, h->ell_col, T, K, dff, cnt, colptr, csc);
    hipLaunchKernelGGL((dw_ell_kernel<DT, NCH>), dim3((dff + 3) / 4), dim3(NT), 0, s, xb, dyb, T,
                       K, dff, dm, colptr, csc, coef, dwg, dwu, dwd);
    if (h->max_ovf > 0 && T > 0) {
        const int mt_tiles = L.pad_ovf / mt::TILE;
        hipLaunchKernelGGL((ovf_ud_kernel<DT>), dim3(dff / mt::TILE, mt_tiles), dim3(mt::NT), 0, s,
                           xb, dyb, h->ovf_rows, h->n_ovf, h->max_ovf, (const uint8_t *)wu,
                           (const uint8_t *)wd, dm, dff, h->dense, inter, stride);
        const int nt_dm = (dm + mt::TILE - 1) / mt::TILE;
        hipLaunchKernelGGL((ovf_dx_kernel<DT>), dim3(nt_dm, mt_tiles), dim3(mt::NT), 0, s, inter,
                           stride, h->ovf_rows, h->n_ovf, h->max_ovf, (const uint8_t *)wu,
                           (const uint8_t *)wg, dm, dff, dx);
        hipLaunchKernelGGL((ovf_dw_kernel<DT>), dim3(nt_dm, dff / mt::TILE, 3), dim3(mt::NT), 0, s,
                           inter, stride, h->ovf_rows, h->n_ovf, h->max_ovf, xb, dyb, dm, dff, dwd,
                           dwu, dwg);
    }
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const void *x, const void *dy, const hybrid_t *h, const void *wg,
                     const void *wu, const void *wd, int dm, float *dx, float *dwg, float *dwu,
                     float *dwd, uint8_t *ws, int32_t *status, hipStream_t s)
{
    const int nch = (dm * (int)sizeof(typename elem<DT>::storage) + 1023) / 1024;
#define TW_CASE(N) \
    case N: return launch_nch<DT, N>(x, dy, h, wg, wu, wd, dm, dx, dwg, dwu, dwd, ws, status, s);
    switch (nch) {
        TW_CASE(1) TW_CASE(2) TW_CASE(3) TW_CASE(4) TW_CASE(5) TW_CASE(6) TW_CASE(7)
    default: return launch_nch<DT, 8>(x, dy, h, wg, wu, wd, dm, dx, dwg, dwu, dwd, ws, status, s);
    }
#undef TW_CASE
}

} // namespace

size_t bwd_workspace_layout(int T, int dm, int dff, int K, int max_ovf, size_t *offsets)
{
    (void)dm;
    const Layout L = layout(T, dff, K, max_ovf);
    if (offsets) {
        offsets[0] = L.coef;
        offsets[1] = L.cnt;
        offsets[2] = L.colptr;
        offsets[3] = L.csc;
        offsets[4] = L.inter;
    }
    return L.total;
}

hipError_t launch_bwd(twell_dtype dt, const void *x, const void *dy, const hybrid_t *h,
                      const void *wg_t, const void *wu_t, const void *wd, int dm, float *dx,
                      float *dwg_t, float *dwu_t, float *dwd, void *ws, int32_t *status,
                      hipStream_t s)
{
    if (dt == TWELL_BF16)
        return launch_dt<TWELL_BF16>(x, dy, h, wg_t, wu_t, wd, dm, dx, dwg_t, dwu_t, dwd,
                                     (uint8_t *)ws, status, s);
    return launch_dt<TWELL_F32>(x, dy, h, wg_t, wu_t, wd, dm, dx, dwg_t, dwu_t, dwd,
                                (uint8_t *)ws, status, s);
}
