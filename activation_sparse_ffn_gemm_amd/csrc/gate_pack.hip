// Gate matmul g = x W_g on MFMA with the TwELL packing of ReLU(g) in its
// epilogue ("Sparser, Faster, Lighter Transformer Language Models", summary
// page section 2.B.1; the dothoosh.com article: conversion moved into the
// matmul's epilogue, tiles matched to the matmul tile).
//
// One workgroup computes a 192-token x 256-neuron block of g: two TwELL
// column tiles for 192 rows, g never leaving the registers. Eight wave64s (two
// per SIMD) split it 2 x 4; each wave owns 96 rows x 64 columns = 3 x 2 MFMA
// 32x32 blocks. For 4096 tokens x 2816 neurons this gives 242 workgroups, one
// round on 256 CUs.
//
// Operands stream through LDS in K steps of 64 bytes per row (32 bf16 /
// 16 f32), NST steps resident at once: the loads of step k + NST - 1 are
// issued while step k is computed. The loads go straight from global memory
// to LDS (4 bytes per lane, no register staging); each wave waits only for its
// own loads of the step it is about to use, then a barrier covers the others'.
// LDS rows are XOR-swizzled in 16-byte chunks so that the 16 lanes a 128-bit
// fragment read serves per cycle hit 16 distinct groups of the 64 banks.
//
// Epilogue, per row: one ballot per 32-column block gives the g > 0 mask;
// popcounts give the count in each wave's 64 columns, which the two waves of a
// TwELL tile exchange through LDS; each positive lane's slot is the number of
// positive columns before it, so entries land in ascending column order.
#include "mfma_tile.hpp"

namespace {

constexpr int BM = 192, BN = 256;
constexpr int ROWB = 64; // bytes of one LDS row per K step
constexpr int NST = 4;   // K steps resident in LDS
constexpr int GM = 8;    // token tiles per group of the tile order
constexpr int WM = 96, WN = 64, MI = 3, NI = 2; // per wave: 96 x 64 = 3 x 2 blocks of 32x32
constexpr int WGM = BM / WM, WGN = BN / WN;     // waves along M and N
constexpr int NT = 64 * WGM * WGN;
constexpr int MINB = 1;  // workgroups per CU the register budget is sized for
constexpr int STAGE = (BM + BN) * ROWB; // bytes per K step
constexpr int BLK = 1024;               // bytes one wave's 16-byte-lane load writes: 16 rows
constexpr int NBLK = STAGE / BLK;       // blocks per K step
constexpr int NWV = NT / 64;
// blocks per wave: the first N_HI waves take WB_HI, the others WB_HI - 1
constexpr int WB_HI = (NBLK + NWV - 1) / NWV, N_HI = NBLK - (WB_HI - 1) * NWV;
static_assert(STAGE % BLK == 0 && BM % 16 == 0, "a block must not straddle the two operands");
static_assert(2 * WB_HI < 64, "loads in flight must fit the vmcnt counter");

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// One 16-byte-per-lane load from global memory straight into LDS: lane l's
// 16 bytes land at LDS byte lds + 16 l. Written as assembly so that the compiler, which
// would otherwise make every LDS read and barrier wait for all such loads in
// flight, leaves the waiting to the explicit vmcnt waits of the K loop. M0
// (the LDS base of the load) is written here; nothing else in this kernel
// reads M0 on gfx950 (its LDS instructions do not use it), hence the
// silenced warning about clobbering a reserved register.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
DEVI void lds_dma16(const uint8_t *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds)
                 : "m0");
}
#pragma clang diagnostic pop

// Byte offset of 16-byte chunk c (0..3) of LDS row r (64-byte rows). Rows
// r, r+4, r+8, r+12 start on the same bank; XOR-ing the chunk with (r / 4) % 4
// separates them, so 16 consecutive rows at one chunk use 16 distinct groups.
DEVI int swz(int r, int c) { return r * ROWB + ((c ^ ((r >> 2) & 3)) << 4); }

// Wait until at most n of this wave's vector-memory operations are pending
// (gfx9 s_waitcnt encoding: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt
// at their maximum, i.e. not waited on).
template <int n> DEVI void wait_vm()
{
    static_assert(n >= 0 && n < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

typedef floatx16_t Acc[MI][NI];

// bf16 epilogue. The K loop's LDS is free again: the tile's values go there
// as bf16 (round to nearest even, what TwELL stores), column-major, with one
// 32-bit g > 0 mask per row and 32-column block; then every thread packs one
// (row, TwELL tile) pair from LDS: count = popcounts of its four masks,
// entries = the set bits in ascending column order. Per lane this costs a
// few dozen instructions instead of a pass over every accumulator row.
constexpr int VALS_B = BN * BM * 2;              // bytes of the bf16 value tile
constexpr int NBK = BN / 32;                     // 32-column blocks per row
static_assert(VALS_B + BM * NBK * 4 <= NST * STAGE, "tile must fit the K loop's LDS");

DEVI void pack_bf16(const Acc &acc, uint8_t *lds, int m0, int n0, int T, int nt, int W, int wm,
                    int wn, int lane, int32_t *__restrict__ count, int16_t *__restrict__ col,
                    uint16_t *__restrict__ val, int32_t *__restrict__ status)
{
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const int half = lane >> 5, l32 = lane & 31;
    uint16_t *vals = (uint16_t *)lds;                 // [BN][BM]
    uint32_t *masks = (uint32_t *)(lds + VALS_B);     // [BM][NBK]
    __syncthreads(); // every wave is done reading the K loop's stages
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            const int c = wn * WN + ni * 32 + l32;
#pragma unroll
            for (int eg = 0; eg < 4; ++eg) { // rows r .. r+3, r = 8 eg + 4 half
                const int r = wm * WM + mi * 32 + 8 * eg + 4 * half;
                const bf16x2v p0 = {(__bf16)acc[mi][ni][4 * eg], (__bf16)acc[mi][ni][4 * eg + 1]};
                const bf16x2v p1 = {(__bf16)acc[mi][ni][4 * eg + 2], (__bf16)acc[mi][ni][4 * eg + 3]};
                *(uint2 *)(vals + (size_t)c * BM + r) =
                    make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
            }
        }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r = wm * WM + mi * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            const bool ok = m0 + r < T;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const uint64_t b = __ballot(ok && acc[mi][ni][e] > 0.f);
                if (l32 == 0)
                    masks[r * NBK + wn * (WN / 32) + ni] = (uint32_t)(b >> (32 * half));
            }
        }
    __syncthreads();
    for (int q = threadIdx.x; q < BM * (BN / TWELL_TILE_C); q += NT) {
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
                val[tj * W + p] = vals[(size_t)c * BM + r];
                ++p;
            }
        }
    }
}

// Generic epilogue (float32 values): per row, one ballot per 32-column block
// gives the g > 0 mask; popcounts give each wave's count in its 64 columns,
// which the two waves of a TwELL tile exchange through LDS; each positive
// lane's slot is the number of positive columns before it.
template <int DT>
DEVI void pack_rows(const Acc &acc, int (*cnt_lds)[WGN], int m0, int n0, int T, int nt, int W,
                    int wm, int wn, int half, int l32, int32_t *__restrict__ count,
                    int16_t *__restrict__ col, void *__restrict__ val,
                    int32_t *__restrict__ status)
{
    using E = elem<DT>;
    const int lane = half * 32 + l32;
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
    // the other wave of the TwELL tile counted columns 64 (wn ^ 1) .. of the
    // same rows: lane l fetches its counts for rows l and 64 + l of this
    // wave's 96, and each row's value is then broadcast from its lane
    const int pw = wn ^ 1;
    const int pc0 = cnt_lds[wm * WM + lane][pw];
    const int pc1 = cnt_lds[wm * WM + 64 + (lane & 31)][pw];
    auto partner = [&](int r) { // r: compile-time row of this wave
        return __builtin_amdgcn_readlane(r < 64 ? pc0 : pc1, r & 63);
    };
    const size_t rs = (size_t)nt * W; // slots per token row of TwELL
    const size_t rb = ((size_t)(m0 + wm * WM + 4 * half) * nt + j) * W;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r0 = mi * 32 + 8 * (e >> 2) + (e & 3); // this lane's row: r0 + 4 half
            const int t = m0 + wm * WM + r0 + 4 * half;
            const bool ok = t < T;
            const int prt = half ? partner(r0 + 4) : partner(r0);
            uint32_t m[NI];
            int before[NI];
            int run = (wn & 1) ? prt : 0;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                m[ni] = (uint32_t)(__ballot(ok && acc[mi][ni][e] > 0.f) >> (32 * half));
                before[ni] = run;
                run += __popc(m[ni]);
            }
            if (!ok)
                continue;
            const size_t rbase = rb + (size_t)r0 * rs;
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
                // run = this wave's count of the row (it starts at 0)
                const int tot = run + prt;
                count[(size_t)t * nt + j] = tot;
                if (tot > W)
                    raise_status(status, TWELL_DEV_TILE_OVERFLOW);
            }
        }
}

template <int DT>
__global__ __launch_bounds__(NT, MINB) void gate_pack_kernel(
    const uint8_t *__restrict__ x, const uint8_t *__restrict__ wg, int T, int dm, int dff, int W,
    int32_t *__restrict__ count, int16_t *__restrict__ col, void *__restrict__ val,
    int32_t *__restrict__ status)
{
    using E = elem<DT>;
    constexpr int esz = sizeof(typename E::storage);
    __shared__ __attribute__((aligned(16))) uint8_t L[NST][STAGE];
    __shared__ int cnt_lds[BM][WGN];

    // XCD-aware tile order: workgroup b runs on XCD b % 8; XCD k takes the
    // k-th contiguous run of a grouped tile order (GM token tiles x all neuron
    // tiles per group, token tile fastest), so the ~32 tiles an XCD runs at
    // once form a GM x (32 / GM) block whose x and W_g rows its L2 shares.
    const int n_nt = (dff + BN - 1) / BN, n_mt = (T + BM - 1) / BM, total = n_nt * n_mt;
    const int per = (total + NXCD - 1) / NXCD;
    const int q = (blockIdx.x % NXCD) * per + blockIdx.x / NXCD;
    if (q >= total)
        return;
    const int grp = q / (GM * n_nt), rows = min(GM, n_mt - grp * GM), r = q % (GM * n_nt);
    const int m0 = (grp * GM + r % rows) * BM, n0 = (r / rows) * BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int half = lane >> 5, l32 = lane & 31;
    const int nt = dff / TWELL_TILE_C;
    const size_t rowbytes = (size_t)dm * esz;
    const int nk = (int)(rowbytes / ROWB);

    // This wave's 1 KB blocks of a stage: block b holds tile rows
    // 16b .. 16b+15 (A rows, then B rows). Lane l writes bytes 16l .. 16l+15
    // of it, i.e. swizzled chunk l&3 of row 16b + l/4, so it loads the source
    // chunk the swizzle maps there. Rows past the operand read a clamped row:
    // they only feed outputs that are not stored.
    const int nb = wave < N_HI ? WB_HI : WB_HI - 1;
    const int b0 = wave < N_HI ? wave * WB_HI : N_HI * WB_HI + (wave - N_HI) * (WB_HI - 1);
    const uint8_t *src[WB_HI];
#pragma unroll
    for (int i = 0; i < WB_HI; ++i) {
        const int b = min(b0 + i, NBLK - 1);
        const int r = 16 * b + (lane >> 2);
        const int c = (lane & 3) ^ ((r >> 2) & 3);
        const uint8_t *row = r < BM ? x + (size_t)min(m0 + r, T - 1) * rowbytes
                                    : wg + (size_t)min(n0 + r - BM, dff - 1) * rowbytes;
        src[i] = row + c * 16;
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8 *)&L[0][0] + b0 * BLK;
    auto issue = [&](int kt) {
        const uint32_t dst = lds0 + (kt % NST) * STAGE;
#pragma unroll
        for (int i = 0; i < WB_HI; ++i)
            if (i < nb) // uniform
                lds_dma16(src[i] + (size_t)kt * ROWB, dst + i * BLK);
    };

    Acc acc;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[mi][ni][e] = 0.f;

#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < nk)
            issue(s);
    for (int kt = 0; kt < nk; ++kt) {
        // this wave's loads of step kt are done once at most the later steps' pend
        const int later = min(nk - 1, kt + NST - 2) - kt;
        if (later >= 2) {
            if (nb == WB_HI)
                wait_vm<2 * WB_HI>();
            else
                wait_vm<2 * (WB_HI - 1)>();
        } else if (later == 1) {
            if (nb == WB_HI)
                wait_vm<WB_HI>();
            else
                wait_vm<WB_HI - 1>();
        } else {
            wait_vm<0>();
        }
        __syncthreads(); // all loads of step kt are in; step kt - 1 is consumed
        if (kt + NST - 1 < nk)
            issue(kt + NST - 1);
        const uint8_t *As = L[kt % NST], *Bs = As + BM * ROWB;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            uint4 fa[MI], fb[NI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                fa[mi] = *(const uint4 *)(As + swz(wm * WM + mi * 32 + l32, 2 * g + half));
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                fb[ni] = *(const uint4 *)(Bs + swz(wn * WN + ni * 32 + l32, 2 * g + half));
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    mt::mma_group<DT>(acc[mi][ni], fa[mi], fb[ni]);
        }
    }

    // ---- epilogue. Accumulator element e of lane l in a 32x32 block holds
    // row 8*(e/4) + 4*(l/32) + e%4 and column l%32 of that block.
    if constexpr (DT == TWELL_BF16) {
        pack_bf16(acc, L[0], m0, n0, T, nt, W, wm, wn, lane, count, col, (uint16_t *)val, status);
    } else {
        pack_rows<DT>(acc, cnt_lds, m0, n0, T, nt, W, wm, wn, half, l32, count, col, val, status);
    }
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
