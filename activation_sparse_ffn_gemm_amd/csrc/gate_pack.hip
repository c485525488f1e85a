// Gate matmul g = x W_g on MFMA with the TwELL packing of ReLU(g) in its
// epilogue ("Sparser, Faster, Lighter Transformer Language Models", summary
// page section 2.B.1; the dothoosh.com article: conversion moved into the
// matmul's epilogue, tiles matched to the matmul tile).
//
// One workgroup computes a 128-token x 128-neuron block of g, i.e. exactly one
// TwELL column tile for 128 rows, so the packing needs no other workgroup and
// g never leaves the chip. Four wave64s split the block 2 x 2 (64 x 64 each,
// 2 x 2 MFMA 32x32 blocks). K steps of 128 bytes per row (64 bf16 / 32 f32)
// are staged through double-buffered, XOR-swizzled LDS.
//
// Epilogue: for every row, one ballot per 32-column MFMA block gives the
// g > 0 mask; popcounts give the row's count in each wave's 64 columns, which
// the two waves sharing a row exchange through LDS; a lane's slot is the
// number of positive columns before it (mbcnt-style popcount), so entries
// land in ascending column order.
#include "common.hpp"

namespace {

constexpr int BM = 128;
constexpr int BN = TWELL_TILE_C;
constexpr int ROWB = 128; // bytes of one LDS row per K step
constexpr int NT = 256;

// Byte offset of 16-byte chunk c of LDS row r. The XOR swizzle spreads the 8
// consecutive rows read by one pass of a fragment load over all bank groups.
DEVI int swz(int r, int c) { return r * ROWB + ((c ^ (r & 7)) << 4); }

template <int DT>
DEVI void mma_group(floatx16_t &acc, const uint4 &a, const uint4 &b);

template <>
DEVI void mma_group<TWELL_BF16>(floatx16_t &acc, const uint4 &a, const uint4 &b)
{
    // 8 bf16 of k per lane: the two lane halves hold k 0..7 and 8..15 of a 16-k step
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

template <>
DEVI void mma_group<TWELL_F32>(floatx16_t &acc, const uint4 &a, const uint4 &b)
{
    // 4 floats of k per lane; element m of both operands is the same k, so four
    // K=2 MFMAs cover the 8 k of this 16-byte group (any k order sums the same terms)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

template <int DT>
__global__ __launch_bounds__(NT, 2) void gate_pack_kernel(
    const uint8_t *__restrict__ x, const uint8_t *__restrict__ wg, int T, int dm, int dff, int W,
    int32_t *__restrict__ count, int16_t *__restrict__ col, void *__restrict__ val,
    int32_t *__restrict__ status)
{
    using E = elem<DT>;
    constexpr int esz = sizeof(typename E::storage);
    __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * ROWB];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * ROWB];
    __shared__ int cnt_lds[BM][2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int half = lane >> 5, l32 = lane & 31;
    const int j = blockIdx.x;
    const int m0 = blockIdx.y * BM, n0 = j * BN;
    const int nt = dff / BN;
    const size_t rowbytes = (size_t)dm * esz;

    uint4 ra[4], rb[4];
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + NT * i, r = q >> 3, c = q & 7;
            const size_t koff = (size_t)kt * ROWB + c * 16;
            ra[i] = (m0 + r < T) ? ldg16(x + (size_t)(m0 + r) * rowbytes + koff) : make_uint4(0, 0, 0, 0);
            rb[i] = ldg16(wg + (size_t)(n0 + r) * rowbytes + koff);
        }
    };
    auto sstore = [&](int b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + NT * i, r = q >> 3, c = q & 7;
            *(uint4 *)(As[b] + swz(r, c)) = ra[i];
            *(uint4 *)(Bs[b] + swz(r, c)) = rb[i];
        }
    };

    floatx16_t acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[mi][ni][e] = 0.f;

    const int nk = (int)(rowbytes / ROWB);
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int b = kt & 1;
        if (kt + 1 < nk)
            gload(kt + 1);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint4 fa[2], fb[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                fa[mi] = *(const uint4 *)(As[b] + swz(wm * 64 + mi * 32 + l32, 2 * g + half));
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                fb[ni] = *(const uint4 *)(Bs[b] + swz(wn * 64 + ni * 32 + l32, 2 * g + half));
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    mma_group<DT>(acc[mi][ni], fa[mi], fb[ni]);
        }
        if (kt + 1 < nk)
            sstore(b ^ 1);
        __syncthreads();
    }

    // ---- epilogue. Accumulator element e of lane l in a 32x32 block holds
    // row 8*(e/4) + 4*(l/32) + e%4 and column l%32 of that block.
    const uint32_t below = lanemask_lt32(l32);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = wm * 64 + mi * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            const bool ok = m0 + row < T;
            const uint64_t b0 = __ballot(ok && acc[mi][0][e] > 0.f);
            const uint64_t b1 = __ballot(ok && acc[mi][1][e] > 0.f);
            const uint32_t h0 = (uint32_t)(b0 >> (32 * half)), h1 = (uint32_t)(b1 >> (32 * half));
            if (l32 == 0)
                cnt_lds[row][wn] = __popc(h0) + __popc(h1);
        }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = wm * 64 + mi * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            const int t = m0 + row;
            const bool ok = t < T;
            const float v0 = acc[mi][0][e], v1 = acc[mi][1][e];
            const uint64_t b0 = __ballot(ok && v0 > 0.f);
            const uint64_t b1 = __ballot(ok && v1 > 0.f);
            const uint32_t h0 = (uint32_t)(b0 >> (32 * half)), h1 = (uint32_t)(b1 >> (32 * half));
            const int base = wn ? cnt_lds[row][0] : 0;
            const size_t rbase = ((size_t)t * nt + j) * W;
            if (ok && v0 > 0.f) {
                const int p = base + __popc(h0 & below);
                if (p < W) {
                    col[rbase + p] = (int16_t)(n0 + wn * 64 + l32);
                    E::store1(val, rbase + p, v0);
                }
            }
            if (ok && v1 > 0.f) {
                const int p = base + __popc(h0) + __popc(h1 & below);
                if (p < W) {
                    col[rbase + p] = (int16_t)(n0 + wn * 64 + 32 + l32);
                    E::store1(val, rbase + p, v1);
                }
            }
            if (ok && wn == 0 && l32 == 0) {
                const int tot = cnt_lds[row][0] + cnt_lds[row][1];
                count[(size_t)t * nt + j] = tot;
                if (tot > W)
                    raise_status(status, TWELL_DEV_TILE_OVERFLOW);
            }
        }
}

} // namespace

hipError_t launch_gate_pack(twell_dtype dt, const void *x, const void *wg_t, int T, int dm,
                            const twell_t *o, int32_t *status, hipStream_t s)
{
    dim3 grid(o->d_ff / BN, (T + BM - 1) / BM);
    if (dt == TWELL_BF16)
        hipLaunchKernelGGL(gate_pack_kernel<TWELL_BF16>, grid, dim3(NT), 0, s, (const uint8_t *)x,
                           (const uint8_t *)wg_t, T, dm, o->d_ff, o->width, o->count, o->col,
                           o->val, status);
    else
        hipLaunchKernelGGL(gate_pack_kernel<TWELL_F32>, grid, dim3(NT), 0, s, (const uint8_t *)x,
                           (const uint8_t *)wg_t, T, dm, o->d_ff, o->width, o->count, o->col,
                           o->val, status);
    return hipGetLastError();
}
