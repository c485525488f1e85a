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
constexpr int NT = 512;
constexpr int NST = 4; // K steps resident in LDS
constexpr int WM = 96, WN = 64, MI = 3, NI = 2; // per wave: 96 x 64 = 3 x 2 blocks of 32x32
constexpr int STAGE = (BM + BN) * ROWB;          // bytes per K step
constexpr int BLK = 256;                          // bytes one wave's 4-byte-lane load writes
constexpr int NBLK = STAGE / BLK, WBLK = NBLK / (NT / 64); // 256-byte blocks: total, per wave
static_assert(NBLK % (NT / 64) == 0, "blocks must split evenly over the waves");
static_assert(BM % 4 == 0, "a block must not straddle the two operands");

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// One 4-byte-per-lane load from global memory straight into LDS: lane l's word
// lands at LDS byte lds + 4 l. Written as assembly so that the compiler, which
// would otherwise make every LDS read and barrier wait for all such loads in
// flight, leaves the waiting to the explicit vmcnt waits of the K loop. M0
// (the LDS base of the load) is written here; nothing else in this kernel
// reads M0 on gfx950 (its LDS instructions do not use it), hence the
// silenced warning about clobbering a reserved register.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
DEVI void lds_dma4(const uint8_t *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
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

template <int DT>
__global__ __launch_bounds__(NT, 1) void gate_pack_kernel(
    const uint8_t *__restrict__ x, const uint8_t *__restrict__ wg, int T, int dm, int dff, int W,
    int32_t *__restrict__ count, int16_t *__restrict__ col, void *__restrict__ val,
    int32_t *__restrict__ status)
{
    using E = elem<DT>;
    constexpr int esz = sizeof(typename E::storage);
    __shared__ __attribute__((aligned(16))) uint8_t L[NST][STAGE];
    __shared__ int cnt_lds[BM][4];

    // XCD-aware tile order: workgroup b runs on XCD b % 8; XCD k takes the
    // k-th contiguous run of output tiles in M-major order, so its L2 holds a
    // few x row blocks and the W_g blocks they meet instead of all of both.
    const int n_nt = (dff + BN - 1) / BN, total = n_nt * ((T + BM - 1) / BM);
    const int per = (total + NXCD - 1) / NXCD;
    const int tile = (blockIdx.x % NXCD) * per + blockIdx.x / NXCD;
    if (tile >= total)
        return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int half = lane >> 5, l32 = lane & 31;
    const int m0 = (tile / n_nt) * BM, n0 = (tile % n_nt) * BN;
    const int nt = dff / TWELL_TILE_C;
    const size_t rowbytes = (size_t)dm * esz;
    const int nk = (int)(rowbytes / ROWB);

    // This wave's 256-byte blocks of a stage: block b holds tile rows
    // 4b .. 4b+3 (A rows, then B rows). Lane l writes bytes 4l .. 4l+3 of it,
    // i.e. word l&3 of swizzled chunk (l&15)>>2 of row 4b + l/16, so it loads
    // that word of the source chunk the swizzle maps there. Rows past the
    // operand read a clamped row: they only feed outputs that are not stored.
    const uint8_t *src[WBLK];
#pragma unroll
    for (int i = 0; i < WBLK; ++i) {
        const int b = wave * WBLK + i;
        const int r = 4 * b + (lane >> 4);
        const int c = ((lane & 15) >> 2) ^ ((r >> 2) & 3);
        const uint8_t *row = r < BM ? x + (size_t)min(m0 + r, T - 1) * rowbytes
                                    : wg + (size_t)min(n0 + r - BM, dff - 1) * rowbytes;
        src[i] = row + c * 16 + (lane & 3) * 4;
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8 *)&L[0][0] + wave * WBLK * BLK;
    auto issue = [&](int kt) {
        const uint32_t dst = lds0 + (kt % NST) * STAGE;
#pragma unroll
        for (int i = 0; i < WBLK; ++i)
            lds_dma4(src[i] + (size_t)kt * ROWB, dst + i * BLK);
    };

    floatx16_t acc[MI][NI];
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
        if (later >= 2)
            wait_vm<2 * WBLK>();
        else if (later == 1)
            wait_vm<WBLK>();
        else
            wait_vm<0>();
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
