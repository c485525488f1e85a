// Fused up and down projections over the TwELL nonzeros ("Sparser, Faster,
// Lighter Transformer Language Models", summary page section 2.B.2: one
// kernel applies both projections, dot products only for nonzero entries).
//
// y[t] = sum over stored (i, h) of row t of  h * (x[t] . wu_t[i]) * wd[i].
//
// One wave64 owns one token: x[t] and the float32 accumulator y[t] live in
// registers (16-byte chunks, chunk c of lane l = elements (64 c + l) * P ..),
// the row's entries are staged in LDS in ascending column order, and entries
// are processed G at a time so 2 G weight rows are in flight per wave. Each
// entry gathers one contiguous wu_t row (the up column) and one wd row (the
// down row): both are coalesced 16-byte-per-lane reads.
#include "common.hpp"

namespace {

constexpr int NT = 256;   // 4 waves = 4 tokens per workgroup
constexpr int LIST = 256; // entries staged per pass

template <int DT, int NCH, int G>
__global__ __launch_bounds__(NT) void ffn_fwd_token_kernel(
    const uint8_t *__restrict__ x, const int32_t *__restrict__ count,
    const int16_t *__restrict__ col, const void *__restrict__ val, int T, int nt, int W,
    const uint8_t *__restrict__ wu, const uint8_t *__restrict__ wd, int dm, float *__restrict__ y,
    int32_t *__restrict__ status)
{
    using E = elem<DT>;
    constexpr int P = E::per16;
    constexpr int esz = sizeof(typename E::storage);
    __shared__ int lcol[NT / 64][LIST];
    __shared__ float lval[NT / 64][LIST];

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = blockIdx.x * (NT / 64) + wv;
    if (t >= T)
        return; // the whole wave leaves; no workgroup barrier below
    const size_t rowbytes = (size_t)dm * esz;

    float xr[NCH][P], yr[NCH][P];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const size_t off = (size_t)(c * 64 + lane) * 16;
        if (off < rowbytes)
            E::widen(ldg16(x + (size_t)t * rowbytes + off), xr[c]);
        else
#pragma unroll
            for (int k = 0; k < P; ++k)
                xr[c][k] = 0.f;
#pragma unroll
        for (int k = 0; k < P; ++k)
            yr[c][k] = 0.f;
    }

    for (int j0 = 0; j0 < nt; j0 += 64) {
        const int jj = j0 + lane;
        const int n = jj < nt ? min(count[(size_t)t * nt + jj], W) : 0;
        const int incl = wave_incl_scan(n, lane);
        const int excl = incl - n;
        const int tot = __shfl(incl, 63, 64);
        for (int p0 = 0; p0 < tot; p0 += LIST) {
            for (int s = 0; s < n; ++s) {
                const int e = excl + s - p0;
                if (e >= 0 && e < LIST) {
                    const size_t src = ((size_t)t * nt + jj) * W + s;
                    int c = col[src];
                    float v = E::load1(val, src);
                    if (c < 0 || c >= nt * TWELL_TILE_C) { // corrupt entry: skip it, report
                        raise_status(status, TWELL_DEV_BAD_INDEX);
                        c = 0;
                        v = 0.f;
                    }
                    lcol[wv][e] = c;
                    lval[wv][e] = v;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int ne = min(LIST, tot - p0);
            for (int e0 = 0; e0 < ne; e0 += G) {
                int ci[G];
                float hv[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int e = e0 + g < ne ? e0 + g : e0;
                    ci[g] = lcol[wv][e];
                    hv[g] = lval[wv][e];
                }
                uint4 vu[G][NCH], vd[G][NCH];
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int c = 0; c < NCH; ++c) {
                        const size_t off = (size_t)(c * 64 + lane) * 16;
                        if (off < rowbytes) {
                            vu[g][c] = ldg16(wu + (size_t)ci[g] * rowbytes + off);
                            vd[g][c] = ldg16(wd + (size_t)ci[g] * rowbytes + off);
                        } else {
                            vu[g][c] = make_uint4(0, 0, 0, 0);
                            vd[g][c] = make_uint4(0, 0, 0, 0);
                        }
                    }
                float d[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float s = 0.f;
#pragma unroll
                    for (int c = 0; c < NCH; ++c) {
                        float w[P];
                        E::widen(vu[g][c], w);
#pragma unroll
                        for (int k = 0; k < P; ++k)
                            s += xr[c][k] * w[k];
                    }
                    d[g] = s;
                }
#pragma unroll
                for (int g = 0; g < G; ++g)
                    d[g] = wave_sum(d[g]);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    if (e0 + g < ne && hv[g] != 0.f) {
                        const float a = hv[g] * d[g];
#pragma unroll
                        for (int c = 0; c < NCH; ++c) {
                            float w[P];
                            E::widen(vd[g][c], w);
#pragma unroll
                            for (int k = 0; k < P; ++k)
                                yr[c][k] += a * w[k];
                        }
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }

#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const size_t el = (size_t)(c * 64 + lane) * P;
        if (el < (size_t)dm) {
            float4 *dst = (float4 *)(y + (size_t)t * dm + el);
#pragma unroll
            for (int q = 0; q < P / 4; ++q)
                dst[q] = make_float4(yr[c][4 * q], yr[c][4 * q + 1], yr[c][4 * q + 2], yr[c][4 * q + 3]);
        }
    }
}

template <int DT, int NCH, int G>
hipError_t launch_nch(const void *x, const twell_t *h, const void *wu, const void *wd, int dm,
                      float *y, int32_t *status, hipStream_t s)
{
    dim3 grid((h->T + NT / 64 - 1) / (NT / 64));
    hipLaunchKernelGGL((ffn_fwd_token_kernel<DT, NCH, G>), grid, dim3(NT), 0, s,
                       (const uint8_t *)x, h->count, h->col, h->val, h->T, h->d_ff / TWELL_TILE_C,
                       h->width, (const uint8_t *)wu, (const uint8_t *)wd, dm, y, status);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const void *x, const twell_t *h, const void *wu, const void *wd, int dm,
                     float *y, int32_t *status, hipStream_t s)
{
    const int nch = (dm * (int)sizeof(typename elem<DT>::storage) + 1023) / 1024;
    switch (nch) {
    case 1: return launch_nch<DT, 1, 4>(x, h, wu, wd, dm, y, status, s);
    case 2: return launch_nch<DT, 2, 4>(x, h, wu, wd, dm, y, status, s);
    case 3: return launch_nch<DT, 3, 2>(x, h, wu, wd, dm, y, status, s);
    case 4: return launch_nch<DT, 4, 2>(x, h, wu, wd, dm, y, status, s);
    case 5: return launch_nch<DT, 5, 2>(x, h, wu, wd, dm, y, status, s);
    case 6: return launch_nch<DT, 6, 1>(x, h, wu, wd, dm, y, status, s);
    case 7: return launch_nch<DT, 7, 1>(x, h, wu, wd, dm, y, status, s);
    default: return launch_nch<DT, 8, 1>(x, h, wu, wd, dm, y, status, s);
    }
}

} // namespace

hipError_t launch_ffn_fwd(twell_dtype dt, const void *x, const twell_t *h, const void *wu_t,
                          const void *wd, int dm, float *y, int32_t *status, hipStream_t s)
{
    if (dt == TWELL_BF16)
        return launch_dt<TWELL_BF16>(x, h, wu_t, wd, dm, y, status, s);
    return launch_dt<TWELL_F32>(x, h, wu_t, wd, dm, y, status, s);
}
