// Gate matmul g = x W_g on MFMA with the TwELL packing of ReLU(g) in its
// epilogue ("Sparser, Faster, Lighter Transformer Language Models", summary
// page section 2.B.1; the dothoosh.com article: conversion moved into the
// matmul's epilogue, tiles matched to the matmul tile).
//
// One workgroup computes a BM-token x 256-neuron block of g: two TwELL
// column tiles for BM rows, g never leaving the registers. Eight wave64s (two
// per SIMD) split it 2 x 4; each wave owns BM/2 rows x 64 columns of MFMA
// 32x32 blocks. BM = 192 for moderate token counts (4096 tokens x 2816
// neurons give 242 workgroups, one round on 256 CUs); BM = 256 once there are
// enough tiles for several rounds (fewer operand bytes per flop).
//
// The K loop is the shared LDS-DMA main loop (ntgemm.hpp): 128-byte K steps,
// two resident, loads straight from global memory to LDS, per-wave vmcnt
// waits, XOR-swizzled LDS rows.
//
// Epilogue, per row: one ballot per 32-column block gives the g > 0 mask;
// popcounts give the count in each wave's 64 columns, which the two waves of a
// TwELL tile exchange through LDS; each positive lane's slot is the number of
// positive columns before it, so entries land in ascending column order.
#include "ntgemm.hpp"

namespace {

// 128-byte K steps, two resident: one barrier per four MFMA groups
using C192 = ng::Cfg<192, 256, 2, 4, 2, 128>; // waves of 96 x 64 (3 x 2 blocks)
using C256 = ng::Cfg<256, 256, 2, 4, 2, 128>; // waves of 128 x 64 (4 x 2 blocks)
constexpr int GM = 8; // token tiles per group of the tile order

// bf16 epilogue. The K loop's LDS is free again: the tile's values go there
// as bf16 (round to nearest even, what TwELL stores), column-major, with one
// 32-bit g > 0 mask per row and 32-column block; then every thread packs one
// (row, TwELL tile) pair from LDS: count = popcounts of its four masks,
// entries = the set bits in ascending column order. Per lane this costs a
// few dozen instructions instead of a pass over every accumulator row.
//
// A column holds VS = BM + 4 values: the 32 lanes of a half-wave store 8 bytes
// each at 32 consecutive columns, and a column stride of VS / 2 = 2 x odd
// dwords sends them to 32 disjoint bank pairs (a stride of BM, a multiple of
// 64 dwords, would put all 32 on one bank).
template <class C> constexpr int vals_stride() { return C::BM + 4; }
static_assert(((C192::BM + 4) / 2) % 2 == 0 && ((C192::BM + 4) / 4) % 2 == 1, "odd stride");
static_assert(((C256::BM + 4) / 2) % 2 == 0 && ((C256::BM + 4) / 4) % 2 == 1, "odd stride");
template <class C> constexpr int vals_bytes() { return C::BN * vals_stride<C>() * 2; }
template <class C> constexpr int pack_lds() { return vals_bytes<C>() + C::BM * (C::BN / 32) * 4; }
template <class C> constexpr int kernel_lds()
{
    return pack_lds<C>() > C::LDS ? pack_lds<C>() : C::LDS;
}

// v_writelane through its compiler intrinsic (no HIP builtin for it here):
// lane `lane` of `old` becomes the wave-uniform `v`.
extern "C" __device__ int amdgcn_writelane_i32(int v, int lane, int old) __asm("llvm.amdgcn.writelane.i32");
DEVI uint32_t lane_write(uint32_t old, uint32_t v, int lane)
{
    return (uint32_t)amdgcn_writelane_i32((int)v, lane, (int)old);
}

template <class C>
DEVI void pack_bf16(const ng::Acc<C> &acc, uint8_t *lds, int m0, int n0, int T, int nt, int W,
                    int wm, int wn, int lane, int32_t *__restrict__ count,
                    int16_t *__restrict__ col, uint16_t *__restrict__ val,
                    int32_t *__restrict__ status)
{
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    constexpr int BM = C::BM, BN = C::BN, NBK = BN / 32, VS = vals_stride<C>();
    const int half = lane >> 5, l32 = lane & 31;
    uint16_t *vals = (uint16_t *)lds;                       // [BN][VS]
    uint32_t *masks = (uint32_t *)(lds + vals_bytes<C>()); // [BM][NBK]
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni) {
            const int c = wn * C::WN + ni * 32 + l32;
#pragma unroll
            for (int eg = 0; eg < 4; ++eg) { // rows r .. r+3, r = 8 eg + 4 half
                const int r = wm * C::WM + mi * 32 + 8 * eg + 4 * half;
                const bf16x2v p0 = {(__bf16)acc.v[mi][ni][4 * eg], (__bf16)acc.v[mi][ni][4 * eg + 1]};
                const bf16x2v p1 = {(__bf16)acc.v[mi][ni][4 * eg + 2], (__bf16)acc.v[mi][ni][4 * eg + 3]};
                *(uint2 *)(vals + (size_t)c * VS + r) =
                    make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
            }
        }
    // g > 0 masks: ballot i (over mi, e, ni in that order) covers rows r (lanes
    // 0-31) and r + 4 (lanes 32-63) of one 32-column block. The ballot stays
    // in scalar registers and its two words are written straight into lanes
    // 2 i and 2 i + 1 (mod 64) of a register (v_writelane), 32 ballots per
    // register, so a ballot costs one compare and two lane writes; each lane
    // then stores one row's word (four LDS stores per wave).
    constexpr int NBAL = C::MI * 16 * C::NI;
    static_assert(NBAL % 32 == 0, "whole registers of ballots");
    uint32_t mv[NBAL / 32];
#pragma unroll
    for (int q = 0; q < NBAL / 32; ++q)
        mv[q] = 0u;
    // rows of the tile past T get no bits: a wave-uniform mask per (mi, e)
    const int rlim = T - m0 - wm * C::WM; // rows r of this wave's block are valid if r < rlim
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r = mi * 32 + 8 * (e >> 2) + (e & 3);
            const uint32_t ok0 = r < rlim ? ~0u : 0u, ok1 = r + 4 < rlim ? ~0u : 0u;
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni) {
                const int i = (mi * 16 + e) * C::NI + ni;
                const uint64_t b = __ballot(acc.v[mi][ni][e] > 0.f);
                mv[i / 32] = lane_write(mv[i / 32], (uint32_t)b & ok0, 2 * (i % 32));
                mv[i / 32] = lane_write(mv[i / 32], (uint32_t)(b >> 32) & ok1, 2 * (i % 32) + 1);
                // keep each ballot next to its lane writes: hoisted together,
                // the ballots would not fit the scalar registers
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
    for (int q = 0; q < NBAL / 32; ++q) {
        const int i = q * 32 + lane / 2, ni = i % C::NI, e = (i / C::NI) % 16,
                  mi = i / (C::NI * 16);
        const int r = wm * C::WM + mi * 32 + 8 * (e >> 2) + 4 * (lane & 1) + (e & 3);
        masks[r * NBK + wn * (C::WN / 32) + ni] = mv[q];
    }
    __syncthreads();
    for (int q = threadIdx.x; q < BM * (BN / TWELL_TILE_C); q += C::NT) {
        const int r = q / (BN / TWELL_TILE_C), tl = q % (BN / TWELL_TILE_C);
        const int t = m0 + r, j = (n0 >> 7) + tl;
        if (t >= T || j >= nt)
            continue;
        const uint4 mk = *(const uint4 *)(masks + r * NBK + tl * 4);
        const uint32_t mm[4] = {mk.x, mk.y, mk.z, mk.w};
        const int n = __popc(mk.x) + __popc(mk.y) + __popc(mk.z) + __popc(mk.w);
        const size_t tj = (size_t)t * nt + j;
        count[tj] = n;
        if (n > W)
            raise_status(status, TWELL_DEV_TILE_OVERFLOW);
        int p = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t m = mm[k];
            while (m && p < W) {
                const int c = tl * TWELL_TILE_C + k * 32 + __ffs(m) - 1;
                m &= m - 1;
                col[tj * W + p] = (int16_t)(n0 + c);
                val[tj * W + p] = vals[(size_t)c * VS + r];
                ++p;
            }
        }
    }
}

// Generic epilogue (float32 values): per row, one ballot per 32-column block
// gives the g > 0 mask; popcounts give each wave's count in its 64 columns,
// which the two waves of a TwELL tile exchange through LDS; each positive
// lane's slot is the number of positive columns before it.
template <class C, int DT>
DEVI void pack_rows(const ng::Acc<C> &acc, int *cnt_lds, int m0, int n0, int T, int nt, int W,
                    int wm, int wn, int half, int l32, int32_t *__restrict__ count,
                    int16_t *__restrict__ col, void *__restrict__ val,
                    int32_t *__restrict__ status)
{
    static_assert(C::WN == 64, "two waves per TwELL tile");
    using E = elem<DT>;
    constexpr int WGN = C::WGN;
    const int lane = half * 32 + l32;
    const int j = (n0 >> 7) + (wn >> 1);
    const bool tile_ok = j < nt;
    const uint32_t below = lanemask_lt32(l32);
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = wm * C::WM + mi * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            const bool ok = tile_ok && m0 + row < T;
            int tot = 0;
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
                tot += __popc((uint32_t)(__ballot(ok && acc.v[mi][ni][e] > 0.f) >> (32 * half)));
            if (l32 == 0)
                cnt_lds[row * WGN + wn] = tot;
        }
    __syncthreads();
    if (!tile_ok)
        return;
    // the other wave of the TwELL tile counted columns 64 (wn ^ 1) .. of the
    // same rows: lane l fetches its counts for rows l, 64 + l, ... of this
    // wave's WM, and each row's value is then broadcast from its lane
    const int pw = wn ^ 1;
    constexpr int NPC = (C::WM + 63) / 64;
    int pc[NPC];
#pragma unroll
    for (int u = 0; u < NPC; ++u)
        pc[u] = cnt_lds[(wm * C::WM + min(64 * u + lane, C::WM - 1)) * WGN + pw];
    auto partner = [&](int r) { // r: compile-time row of this wave
        return __builtin_amdgcn_readlane(pc[r >> 6], r & 63);
    };
    const size_t rs = (size_t)nt * W; // slots per token row of TwELL
    const size_t rb = ((size_t)(m0 + wm * C::WM + 4 * half) * nt + j) * W;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r0 = mi * 32 + 8 * (e >> 2) + (e & 3); // this lane's row: r0 + 4 half
            const int t = m0 + wm * C::WM + r0 + 4 * half;
            const bool ok = t < T;
            const int prt = half ? partner(r0 + 4) : partner(r0);
            uint32_t m[C::NI];
            int before[C::NI];
            int run = (wn & 1) ? prt : 0;
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni) {
                m[ni] = (uint32_t)(__ballot(ok && acc.v[mi][ni][e] > 0.f) >> (32 * half));
                before[ni] = run;
                run += __popc(m[ni]);
            }
            if (!ok)
                continue;
            const size_t rbase = rb + (size_t)r0 * rs;
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni) {
                const float v = acc.v[mi][ni][e];
                if (v > 0.f) {
                    const int p = before[ni] + __popc(m[ni] & below);
                    if (p < W) {
                        col[rbase + p] = (int16_t)(n0 + wn * C::WN + ni * 32 + l32);
                        E::store1(val, rbase + p, v);
                    }
                }
            }
            if (l32 == 0 && (wn & 1) == 0) {
                // run = this wave's count of the row (it starts at 0)
                const int tot = run + prt;
                count[(size_t)t * nt + j] = tot;
                if (tot > W)
                    raise_status(status, TWELL_DEV_TILE_OVERFLOW);
            }
        }
}

template <class C, int DT>
__global__ __launch_bounds__(C::NT, 1) void gate_pack_kernel(
    const uint8_t *__restrict__ x, const uint8_t *__restrict__ wg, int T, int dm, int dff, int W,
    int32_t *__restrict__ count, int16_t *__restrict__ col, void *__restrict__ val,
    int32_t *__restrict__ status)
{
    using E = elem<DT>;
    constexpr int esz = sizeof(typename E::storage);
    __shared__ __attribute__((aligned(16))) uint8_t L[kernel_lds<C>()];
    __shared__ int cnt_lds[C::BM * C::WGN];
    // XCD-aware tile order: workgroup b runs on XCD b % 8; XCD k takes the
    // k-th contiguous run of a grouped tile order (GM token tiles x all neuron
    // tiles per group, token tile fastest), so the ~32 tiles an XCD runs at
    // once form a GM x (32 / GM) block whose x and W_g rows its L2 shares.
    const int n_nt = (dff + C::BN - 1) / C::BN, n_mt = (T + C::BM - 1) / C::BM;
    const int total = n_nt * n_mt;
    const int per = (total + NXCD - 1) / NXCD;
    const int q = (blockIdx.x % NXCD) * per + blockIdx.x / NXCD;
    if (q >= total)
        return;
    const int grp = q / (GM * n_nt), rows = min(GM, n_mt - grp * GM), r = q % (GM * n_nt);
    const int m0 = (grp * GM + r % rows) * C::BM, n0 = (r / rows) * C::BN;
    const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
    const int wm = ng::wave_m<C>(), wn = ng::wave_n<C>();
    const int nt = dff / TWELL_TILE_C;
    const size_t rowbytes = (size_t)dm * esz;
    // rows past an operand read a clamped row: they only feed outputs that
    // are not stored
    auto rowa = [&](int rr) { return x + (size_t)min(m0 + rr, T - 1) * rowbytes; };
    auto rowb = [&](int rr) { return wg + (size_t)min(n0 + rr, dff - 1) * rowbytes; };
    auto off = [](int kt) { return ng::StepOff{(size_t)kt * C::ROWB, (size_t)kt * C::ROWB}; };
    ng::Acc<C> acc;
    ng::mainloop<C, DT>(L, rowa, rowb, off, 0, (int)(rowbytes / C::ROWB), acc);
    // ---- epilogue. Accumulator element e of lane l in a 32x32 block holds
    // row 8*(e/4) + 4*(l/32) + e%4 and column l%32 of that block.
    if constexpr (DT == TWELL_BF16)
        pack_bf16<C>(acc, L, m0, n0, T, nt, W, wm, wn, lane, count, col, (uint16_t *)val, status);
    else
        pack_rows<C, DT>(acc, cnt_lds, m0, n0, T, nt, W, wm, wn, half, l32, count, col, val,
                         status);
}

template <class C>
void launch_cfg(twell_dtype dt, const void *x, const void *wg_t, int T, int dm,
                const twell_t *o, int32_t *status, hipStream_t s)
{
    const int total = ((o->d_ff + C::BN - 1) / C::BN) * ((T + C::BM - 1) / C::BM);
    const dim3 grid((total + NXCD - 1) / NXCD * NXCD);
    if (dt == TWELL_BF16)
        hipLaunchKernelGGL((gate_pack_kernel<C, TWELL_BF16>), grid, dim3(C::NT), 0, s,
                           (const uint8_t *)x, (const uint8_t *)wg_t, T, dm, o->d_ff, o->width,
                           o->count, o->col, o->val, status);
    else
        hipLaunchKernelGGL((gate_pack_kernel<C, TWELL_F32>), grid, dim3(C::NT), 0, s,
                           (const uint8_t *)x, (const uint8_t *)wg_t, T, dm, o->d_ff, o->width,
                           o->count, o->col, o->val, status);
}

} // namespace

hipError_t launch_dec_gate(twell_dtype dt, const void *x, const void *wg_t, int T, int dm,
                           const twell_t *o, void *ws, int32_t *status, Timer &tm, hipStream_t s);

hipError_t launch_gate_pack(twell_dtype dt, const void *x, const void *wg_t, int T, int dm,
                            const twell_t *o, void *ws, int32_t *status, twell_timing_t *timing,
                            hipStream_t s)
{
    Timer tm(timing, s);
    if (T <= TWELL_DECODE_T) // few tokens: the tile grid would leave the chip idle
        return launch_dec_gate(dt, x, wg_t, T, dm, o, ws, status, tm, s);
    // 256-token tiles once they fill the chip at least twice over
    const int t256 = ((o->d_ff + 255) / 256) * ((T + 255) / 256);
    if (t256 >= 512)
        launch_cfg<C256>(dt, x, wg_t, T, dm, o, status, s);
    else
        launch_cfg<C192>(dt, x, wg_t, T, dm, o, status, s);
    tm.mark("gate_pack_kernel");
    return hipGetLastError();
}
