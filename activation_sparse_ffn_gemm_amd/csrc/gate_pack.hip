// Gate matmul g = x W_g on MFMA with the TwELL packing of ReLU(g) in its
// epilogue ("Sparser, Faster, Lighter Transformer Language Models", summary
// page section 2.B.1; the dothoosh.com article: conversion moved into the
// matmul's epilogue, tiles matched to the matmul tile).
//
// One workgroup computes a 192-token x 256-neuron block of g: two TwELL
// column tiles for 192 rows, g never leaving the registers. Eight wave64s (two
// per SIMD, so one computes while the other waits on memory) split it 2 x 4;
// each wave owns 96 rows x 64 columns = 3 x 2 MFMA 32x32 blocks. The tile
// keeps 192 x 256 x 64 MACs per 56 KB K step (114 flop per byte of L2
// traffic) and, for 4096 tokens x 2816 neurons, gives 242 workgroups: one
// round on 256 CUs. K steps of 128 bytes per row (64 bf16 / 32 f32) go
// through double-buffered, XOR-swizzled LDS, the next step's global loads in
// flight during the current step's MFMAs.
//
// Epilogue, per row: one ballot per 32-column block gives the g > 0 mask;
// popcounts give the count in each wave's 64 columns, which the two waves of a
// TwELL tile exchange through LDS; each positive lane's slot is the number of
// positive columns before it, so entries land in ascending column order.
#include "mfma_tile.hpp"

namespace {

constexpr int BM = 192, BN = 256;
constexpr int ROWB = 128; // bytes of one LDS row per K step
constexpr int NT = 512;
constexpr int WM = 96, WN = 64, MI = 3, NI = 2; // per wave: 96 x 64 = 3 x 2 blocks of 32x32
constexpr int A_CH = BM * 8 / NT, B_CH = BN * 8 / NT; // 16-byte chunks per thread per step

template <int DT>
__global__ __launch_bounds__(NT, 1) void gate_pack_kernel(
    const uint8_t *__restrict__ x, const uint8_t *__restrict__ wg, int T, int dm, int dff, int W,
    int32_t *__restrict__ count, int16_t *__restrict__ col, void *__restrict__ val,
    int32_t *__restrict__ status)
{
    using E = elem<DT>;
    constexpr int esz = sizeof(typename E::storage);
    __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * ROWB];
    __shared__ int cnt_lds[BM][4];

    // XCD-aware tile order: workgroup b runs on XCD b % 8; XCD k takes the
    // k-th contiguous run of output tiles in M-major order, so its L2 holds a
    // few x row blocks and the W_g blocks they meet instead of all of both.
    const int n_nt = (dff + BN - 1) / BN, total = n_nt * ((T + BM - 1) / BM);
    const int per = (total + NXCD - 1) / NXCD;
    const int tile = (blockIdx.x % NXCD) * per + blockIdx.x / NXCD;
    if (tile >= total)
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int half = lane >> 5, l32 = lane & 31;
    const int m0 = (tile / n_nt) * BM, n0 = (tile % n_nt) * BN;
    const int nt = dff / TWELL_TILE_C;
    const size_t rowbytes = (size_t)dm * esz;

    // Two register stages: the global loads of step k + 2 are issued while
    // step k is computed, so each load has two steps of MFMA work to land.
    uint4 ra0[A_CH], rb0[B_CH], ra1[A_CH], rb1[B_CH];
    // Loads are branch-free (rows past the operand are clamped, then zeroed on
    // the way into LDS) so the compiler can keep two steps of loads in flight.
    const uint8_t *pa[A_CH], *pb[B_CH];
    bool oka[A_CH], okb[B_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int q = tid + NT * i, r = q >> 3, c = q & 7;
        oka[i] = m0 + r < T;
        pa[i] = x + (size_t)min(m0 + r, T - 1) * rowbytes + c * 16;
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
        const int q = tid + NT * i, r = q >> 3, c = q & 7;
        okb[i] = n0 + r < dff;
        pb[i] = wg + (size_t)min(n0 + r, dff - 1) * rowbytes + c * 16;
    }
    auto gload = [&](int kt, uint4 (&ra)[A_CH], uint4 (&rb)[B_CH]) {
        const size_t koff = (size_t)kt * ROWB;
#pragma unroll
        for (int i = 0; i < A_CH; ++i)
            ra[i] = ldg16(pa[i] + koff);
#pragma unroll
        for (int i = 0; i < B_CH; ++i)
            rb[i] = ldg16(pb[i] + koff);
    };
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    auto sstore = [&](int b, const uint4 (&ra)[A_CH], const uint4 (&rb)[B_CH]) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int q = tid + NT * i;
            *(uint4 *)(As[b] + mt::swz(q >> 3, q & 7)) = oka[i] ? ra[i] : z4;
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int q = tid + NT * i;
            *(uint4 *)(Bs[b] + mt::swz(q >> 3, q & 7)) = okb[i] ? rb[i] : z4;
        }
    };

    floatx16_t acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[mi][ni][e] = 0.f;

    auto compute = [&](int b) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint4 fa[MI], fb[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                fa[mi] = *(const uint4 *)(As[b] + mt::swz(wm * WM + mi * 32 + l32, 2 * g + half));
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                fb[ni] = *(const uint4 *)(Bs[b] + mt::swz(wn * WN + ni * 32 + l32, 2 * g + half));
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    mt::mma_group<DT>(acc[mi][ni], fa[mi], fb[ni]);
        }
    };
    // step kt: fetch step kt + 2 into `ld` (which held step kt, already in
    // LDS), compute step kt from LDS buffer b, then put step kt + 1 (held in
    // `st`) into the other LDS buffer
    auto iter = [&](int kt, int nk, int b, uint4 (&lda)[A_CH], uint4 (&ldb)[B_CH],
                    const uint4 (&sta)[A_CH], const uint4 (&stb)[B_CH]) {
        if (kt + 2 < nk)
            gload(kt + 2, lda, ldb);
        compute(b);
        if (kt + 1 < nk)
            sstore(b ^ 1, sta, stb);
        __syncthreads();
    };

    const int nk = (int)(rowbytes / ROWB);
    gload(0, ra0, rb0);
    sstore(0, ra0, rb0);
    if (nk > 1)
        gload(1, ra1, rb1);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        iter(kt, nk, 0, ra0, rb0, ra1, rb1);
        if (kt + 1 < nk)
            iter(kt + 1, nk, 1, ra1, rb1, ra0, rb0);
    }

    // ---- epilogue: waves wn and wn ^ 1 share TwELL tile j = n0/128 + wn/2
    // (columns 64 * (wn & 1) .. of it) for rows m0 + wm*96 .. +96.
    // Accumulator element e of lane l in a 32x32 block holds row
    // 8*(e/4) + 4*(l/32) + e%4 and column l%32 of that block.
    const int j = (n0 >> 7) + (wn >> 1);
    const bool tile_ok = j < nt;
    const uint32_t below = lanemask_lt32(l32);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = wm * WM + mi * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            const bool ok = tile_ok && m0 + row < T;
            int tot = 0;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                tot += __popc((uint32_t)(__ballot(ok && acc[mi][ni][e] > 0.f) >> (32 * half)));
            if (l32 == 0)
                cnt_lds[row][wn] = tot;
        }
    __syncthreads();
    if (!tile_ok)
        return;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = wm * WM + mi * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            const int t = m0 + row;
            const bool ok = t < T;
            uint32_t m[NI];
            int before[NI];
            int run = (wn & 1) ? cnt_lds[row][wn ^ 1] : 0;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                m[ni] = (uint32_t)(__ballot(ok && acc[mi][ni][e] > 0.f) >> (32 * half));
                before[ni] = run;
                run += __popc(m[ni]);
            }
            if (!ok)
                continue;
            const size_t rbase = ((size_t)t * nt + j) * W;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const float v = acc[mi][ni][e];
                if (v > 0.f) {
                    const int p = before[ni] + __popc(m[ni] & below);
                    if (p < W) {
                        col[rbase + p] = (int16_t)(n0 + wn * WN + ni * 32 + l32);
                        E::store1(val, rbase + p, v);
                    }
                }
            }
            if (l32 == 0 && (wn & 1) == 0) {
                const int tot = cnt_lds[row][wn] + cnt_lds[row][wn + 1];
                count[(size_t)t * nt + j] = tot;
                if (tot > W)
                    raise_status(status, TWELL_DEV_TILE_OVERFLOW);
            }
        }
}

} // namespace

hipError_t launch_gate_pack(twell_dtype dt, const void *x, const void *wg_t, int T, int dm,
                            const twell_t *o, int32_t *status, twell_timing_t *timing,
                            hipStream_t s)
{
    Timer tm(timing, s);
    const int total = ((o->d_ff + BN - 1) / BN) * ((T + BM - 1) / BM);
    dim3 grid((total + NXCD - 1) / NXCD * NXCD);
    if (dt == TWELL_BF16)
        hipLaunchKernelGGL(gate_pack_kernel<TWELL_BF16>, grid, dim3(NT), 0, s, (const uint8_t *)x,
                           (const uint8_t *)wg_t, T, dm, o->d_ff, o->width, o->count, o->col,
                           o->val, status);
    else
        hipLaunchKernelGGL(gate_pack_kernel<TWELL_F32>, grid, dim3(NT), 0, s, (const uint8_t *)x,
                           (const uint8_t *)wg_t, T, dm, o->d_ff, o->width, o->count, o->col,
                           o->val, status);
    tm.mark("gate_pack_kernel");
    return hipGetLastError();
}
