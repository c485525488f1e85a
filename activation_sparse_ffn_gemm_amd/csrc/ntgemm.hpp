// Tiled MFMA main loop for dense products C[m][n] = sum_k A[m][k] B[n][k]
// whose operands are both K-contiguous (every operand row is a memory row
// along K), shared by the gate GEMM and the dense products over the hybrid's
// backup rows.
//
// A workgroup of WGM x WGN wave64s computes a BM x BN tile; each wave owns a
// WM x WN sub-tile as (WM/32) x (WN/32) blocks of 32x32 MFMA accumulators.
// Operands stream through LDS in K steps of ROWB = 64 or 128 bytes per row
// (32 or 64 bf16), NST steps resident at once: the loads of step k + NST - 1
// are issued while step k is computed. Loads go straight from global memory
// to LDS, 16 bytes per lane (one wave instruction fills 1 KB: 16 rows of 64
// bytes or 8 of 128), so no registers are spent on staging; each wave waits
// only for its own loads of the step it is about to use, then a barrier
// covers the others'. LDS rows are XOR-swizzled in 16-byte chunks so that the
// 16 lanes a 128-bit fragment read serves per cycle hit 16 distinct groups of
// the 64 banks.
//
// Rows are given per tile row by the caller (a gather of any rows is fine);
// K steps map to byte offsets through a caller function, so a product may
// run over several segments (e.g. the hi and lo halves of a bf16 pair, or two
// operand pairs summed) and over any sub-range of them (split K).
#pragma once

#include "common.hpp"

namespace ng {

// One MFMA step over a 16-byte fragment per lane of each operand (32x32
// output block). bf16: one 32x32x16 MFMA; f32: element q of both fragments is
// the same k, so four 32x32x2 MFMAs cover the chunk.
template <int DT> DEVI void mma_group(floatx16_t &acc, const uint4 &a, const uint4 &b);
template <> DEVI void mma_group<TWELL_BF16>(floatx16_t &acc, const uint4 &a, const uint4 &b)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
template <> DEVI void mma_group<TWELL_F32>(floatx16_t &acc, const uint4 &a, const uint4 &b)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

constexpr int ROWB = 64; // default bytes of one LDS row per K step
constexpr int BLK = 1024; // bytes one wave's 16-byte-lane load writes

// NST: K steps resident in LDS (NST - 1 steps of loads in flight).
// ROWB_: bytes of K per step and operand row (64 or 128): a step runs
// ROWB_ / 32 MFMA groups between two barriers.
template <int BM_, int BN_, int WGM_, int WGN_, int NST_ = 4, int ROWB_ = ROWB> struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, NST = NST_, ROWB = ROWB_;
    static constexpr int WM = BM / WGM, WN = BN / WGN, MI = WM / 32, NI = WN / 32;
    static constexpr int NT = 64 * WGM * WGN, NWV = WGM * WGN;
    // 16-byte chunks per row, rows per 1 KB load block, rows per 256-byte
    // LDS bank line, MFMA groups per step
    static constexpr int CPR = ROWB / 16, RPB = BLK / ROWB, SW = 256 / ROWB, NG = ROWB / 32;
    static constexpr int STAGE = (BM + BN) * ROWB, NBLK = STAGE / BLK;
    static_assert(ROWB == 64 || ROWB == 128, "64- or 128-byte K steps");
    // blocks per wave: the first N_HI waves take WB_HI, the others WB_HI - 1
    static constexpr int WB_HI = (NBLK + NWV - 1) / NWV, N_HI = NBLK - (WB_HI - 1) * NWV;
    static constexpr int LDS = NST * STAGE;
    static_assert(BM % 32 == 0 && BN % 32 == 0 && WM % 32 == 0 && WN % 32 == 0, "32x32 blocks");
    static_assert(STAGE % BLK == 0 && BM % RPB == 0, "a block must not straddle the operands");
    static_assert(NST >= 2 && (NST - 2) * WB_HI < 64, "loads in flight must fit the vmcnt counter");
};

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// One 16-byte-per-lane load from global memory straight into LDS: lane l's
// 16 bytes land at LDS byte lds + 16 l. Written as assembly so that the
// compiler, which would otherwise make every LDS read and barrier wait for all
// such loads in flight, leaves the waiting to the explicit vmcnt waits of the
// K loop. M0 (the LDS base of the load) is written here; nothing else in these
// kernels reads M0 on gfx950 (their LDS instructions do not use it), hence the
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

// Byte offset of 16-byte chunk c of LDS row r. With 64-byte rows, rows r,
// r+4, r+8, r+12 start on the same bank and XOR-ing the chunk with (r / 4) % 4
// separates them; with 128-byte rows the same holds for r, r+2, ..., r+14 and
// (r / 2) % 8. Either way 16 consecutive rows at one chunk use 16 distinct
// 4-bank groups.
template <class C> DEVI int swz(int r, int c)
{
    return r * C::ROWB + ((c ^ ((r / C::SW) % C::CPR)) << 4);
}

// Wait until at most n of this wave's vector-memory operations are pending
// (gfx9 s_waitcnt encoding: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt
// at their maximum, i.e. not waited on).
template <int n> DEVI void wait_vm()
{
    static_assert(n >= 0 && n < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait_vm<later * per>() for a run-time later in [0, L] (per, L compile-time)
template <int per, int L> DEVI void wait_vm_steps(int later)
{
    if constexpr (L <= 0) {
        wait_vm<0>();
    } else {
        if (later >= L)
            wait_vm<L * per>();
        else
            wait_vm_steps<per, L - 1>(later);
    }
}

// Byte offsets of one K step in the A rows and in the B rows.
struct StepOff {
    size_t a, b;
};

// Accumulators of one wave.
template <class C> struct Acc {
    floatx16_t v[C::MI][C::NI];
};

// Tile coordinates of accumulator element e of block (mi, ni) of this lane:
// row 8(e/4) + 4(l/32) + e%4 and column l%32 of the block.
template <class C> DEVI int acc_row(int wm, int mi, int e, int lane)
{
    return wm * C::WM + mi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}
template <class C> DEVI int acc_col(int wn, int ni, int lane)
{
    return wn * C::WN + ni * 32 + (lane & 31);
}
template <class C> DEVI int wave_m()
{
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) / C::WGN;
}
template <class C> DEVI int wave_n()
{
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) % C::WGN;
}

// acc += A B^T over K steps [kt0, kt1). rowa(r) / rowb(r) give the address of
// tile row r's data at K offset 0 (every row must be readable: rows outside
// an operand should repeat a valid row and their outputs be dropped);
// off(kt) gives step kt's byte offsets. L: C::LDS bytes of shared memory.
// Ends with a barrier: L may be reused right after.
// wave0: the first of the C::NWV waves that run this product. Several groups
// of waves of one workgroup may run products of their own side by side (each
// on its own L); the barriers are the workgroup's, so every group must run
// the same number of K steps.
template <class C, int DT, class RowA, class RowB, class Off>
DEVI void mainloop(uint8_t *L, RowA rowa, RowB rowb, Off off, int kt0, int kt1, Acc<C> &acc,
                   int wave0 = 0)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) - wave0;
    const int wm = wave / C::WGN, wn = wave % C::WGN;
    const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc.v[mi][ni][e] = 0.f;
    const int nk = kt1 - kt0;
    if (nk <= 0)
        return;
    // This wave's 1 KB blocks of a stage: block b holds tile rows
    // RPB b .. RPB b + RPB - 1 (A rows, then B rows). Lane l writes bytes
    // 16l .. 16l+15 of it, i.e. swizzled chunk l % CPR of row RPB b + l / CPR,
    // so it loads the source chunk the swizzle maps there.
    const int nb = wave < C::N_HI ? C::WB_HI : C::WB_HI - 1;
    const int b0 = wave < C::N_HI ? wave * C::WB_HI
                                  : C::N_HI * C::WB_HI + (wave - C::N_HI) * (C::WB_HI - 1);
    const uint8_t *src[C::WB_HI];
    bool isa[C::WB_HI];
#pragma unroll
    for (int i = 0; i < C::WB_HI; ++i) {
        const int b = min(b0 + i, C::NBLK - 1);
        const int r = C::RPB * b + lane / C::CPR;
        const int c = (lane % C::CPR) ^ ((r / C::SW) % C::CPR);
        isa[i] = C::RPB * b < C::BM; // uniform: a block is all A or all B rows
        src[i] = (isa[i] ? rowa(r) : rowb(r - C::BM)) + c * 16;
    }
    constexpr int NST = C::NST;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8 *)L + b0 * BLK;
    auto issue = [&](int kt) {
        const uint32_t dst = lds0 + ((kt - kt0) % NST) * C::STAGE;
        const StepOff o = off(kt);
#pragma unroll
        for (int i = 0; i < C::WB_HI; ++i)
            if (i < nb) // uniform
                lds_dma16(src[i] + (isa[i] ? o.a : o.b), dst + i * BLK);
    };
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < nk)
            issue(kt0 + s);
    for (int k = 0; k < nk; ++k) {
        // this wave's loads of step k are done once at most the later steps' pend
        const int later = min(nk - 1, k + NST - 2) - k;
        if (nb == C::WB_HI)
            wait_vm_steps<C::WB_HI, NST - 2>(later);
        else
            wait_vm_steps<C::WB_HI - 1, NST - 2>(later);
        __syncthreads(); // all loads of step k are in; step k - 1 is consumed
        if (k + NST - 1 < nk)
            issue(kt0 + k + NST - 1);
        const uint8_t *As = L + (k % NST) * C::STAGE, *Bs = As + C::BM * C::ROWB;
#pragma unroll
        for (int g = 0; g < C::NG; ++g) {
            uint4 fa[C::MI], fb[C::NI];
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi)
                fa[mi] = *(const uint4 *)(As + swz<C>(wm * C::WM + mi * 32 + l32, 2 * g + half));
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
                fb[ni] = *(const uint4 *)(Bs + swz<C>(wn * C::WN + ni * 32 + l32, 2 * g + half));
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni)
                    mma_group<DT>(acc.v[mi][ni], fa[mi], fb[ni]);
        }
    }
    __syncthreads(); // every wave is done reading the stages
}


// ---------------------------------------------------------------- K-major operands
// Products whose operand is stored with the contraction index as its row
// index ("[k][mn]": consecutive elements run along M or N) read it as it is
// stored: the stage holds the operand's K step as KS k-rows of BX elements,
// and the fragment reads transpose on the way out of LDS.
//
// gfx950's transposing LDS read of 16-bit elements (ds_read_b64_tr_b16)
// gives, within each group of 16 lanes, lane 4q + e element e of the 8-byte
// chunks addressed by lanes q, 4 + q, 8 + q and 12 + q (in that order; the
// layout was measured on the part). So if lane 16G + 4j + q of a wave points
// at k-row j, columns c0 + 16 (G & 1) + 4q .. + 3, lane l receives column
// c0 + l % 32 at k-rows 0..3: one half of the 8 consecutive k a 32x32x16 MFMA
// fragment takes per lane. Two reads (k-rows 0..3 and 4..7 of the lane's
// half, k-rows 8 (l / 32) .. of the group) make the fragment.
//
// K-major rows of a stage are BX * esz bytes (at least 256); their 16-byte
// chunks are XOR-swizzled with 4 (k-row % 4), so the four k-rows one read
// touches land in four different 64-byte quarters of the 64 banks.
enum Lay { KC = 0, KM = 1 }; // rows along K (as `mainloop` takes them), or along M/N

template <int DT> DEVI uint4 frag_km(const uint8_t *X, int rb, int cb, int g, int lane);

// fragment of tile columns cb .. cb + 31 for MFMA group g, from a K-major
// region X of rows of rb bytes (bf16)
template <> DEVI uint4 frag_km<TWELL_BF16>(const uint8_t *X, int rb, int cb, int g, int lane)
{
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) bf16x4_t lds_b4;
    const int G = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
    const int col = cb + 16 * (G & 1) + 4 * q; // element column of this lane's chunk
    uint2 h[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int kr = 16 * g + 8 * (G >> 1) + 4 * r + j; // k-row; kr % 4 == j
        const int off = kr * rb + ((((col * 2) >> 4) ^ (j << 2)) << 4) + ((col * 2) & 15);
        const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_b4 *)(uintptr_t)(lds_u8 *)(X + off));
        h[r] = __builtin_bit_cast(uint2, v);
    }
    return make_uint4(h[0].x, h[0].y, h[1].x, h[1].y);
}

// float32: lane l takes column cb + l % 32 at k-rows 8g + 4 (l / 32) + 0..3
// (the k order mma_group<TWELL_F32> expects), one 4-byte read each
template <> DEVI uint4 frag_km<TWELL_F32>(const uint8_t *X, int rb, int cb, int g, int lane)
{
    const int col = cb + (lane & 31);
    uint32_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int kr = 8 * g + 4 * (lane >> 5) + q;
        v[q] = *(const uint32_t *)(X + kr * rb + ((((col * 4) >> 4) ^ ((kr & 3) << 2)) << 4) +
                                   ((col * 4) & 15));
    }
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// acc += A B^T over K steps [kt0, kt1) with either operand K-contiguous (KC)
// or K-major (KM). As in `mainloop`, rowa(r) / rowb(r) give a per-row base
// address and off(kt) the uniform byte offsets of step kt (computed once per
// step): for a KC operand row r is tile row r (at K offset 0), for a KM
// operand row r is the step's k-row r (the K index kt * KS + r, KS = ROWB /
// element size) at the tile's first M (N) element, off(kt) then moving to
// the step's first k-row. Rows outside a KC operand must repeat a valid row
// (their outputs are dropped); K-major rows past the contraction's end must
// read zeros in at least one operand. va / vb: columns of a K-major A / B
// tile that lie inside the operand (a multiple of 8 elements); chunks past
// them read the row's first chunk instead (their outputs are dropped), so no
// read leaves the operand. One group of C::NWV waves; ends with a barrier.
template <class C, int DT, int LA, int LB, class RowA, class RowB, class Off>
DEVI void mainloop_mixed(uint8_t *L, RowA rowa, RowB rowb, Off off, int kt0, int kt1,
                         Acc<C> &acc, int va = 1 << 30, int vb = 1 << 30)
{
    constexpr int esz = DT == TWELL_BF16 ? 2 : 4;
    constexpr int RBA = C::BM * esz, RBB = C::BN * esz; // K-major row bytes
    static_assert(LA == KC || (RBA >= 256 && BLK % RBA == 0), "K-major A rows");
    static_assert(LB == KC || (RBB >= 256 && BLK % RBB == 0), "K-major B rows");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WGN, wn = wave % C::WGN;
    const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc.v[mi][ni][e] = 0.f;
    const int nk = kt1 - kt0;
    if (nk <= 0)
        return;
    const int nb = wave < C::N_HI ? C::WB_HI : C::WB_HI - 1;
    const int b0 = wave < C::N_HI ? wave * C::WB_HI
                                  : C::N_HI * C::WB_HI + (wave - C::N_HI) * (C::WB_HI - 1);
    // per block of this wave: which operand, and the address of the source
    // chunk (at step offset 0) that the stage's swizzle puts at this lane's
    // 16 LDS bytes
    const uint8_t *src[C::WB_HI];
    bool isa[C::WB_HI];
#pragma unroll
    for (int i = 0; i < C::WB_HI; ++i) {
        const int b = min(b0 + i, C::NBLK - 1);
        const int pos = b * BLK + 16 * lane; // byte in the stage
        isa[i] = b * BLK < C::BM * C::ROWB;  // uniform
        const int p = isa[i] ? pos : pos - C::BM * C::ROWB;
        const bool km = isa[i] ? LA == KM : LB == KM;
        const int rb = km ? (isa[i] ? RBA : RBB) : C::ROWB;
        const int r = p / rb, c = (p % rb) >> 4;
        int chunk;
        if (km) {
            const int sc = c ^ ((r & 3) << 2); // source chunk of this LDS chunk
            chunk = sc * 16 / esz < (isa[i] ? va : vb) ? sc << 4 : 0;
        } else {
            chunk = (c ^ ((r / C::SW) % C::CPR)) << 4;
        }
        src[i] = (isa[i] ? rowa(r) : rowb(r)) + chunk;
    }
    constexpr int NST = C::NST;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8 *)L + b0 * BLK;
    auto issue = [&](int kt) {
        const uint32_t dst = lds0 + ((kt - kt0) % NST) * C::STAGE;
        const StepOff o = off(kt);
#pragma unroll
        for (int i = 0; i < C::WB_HI; ++i)
            if (i < nb) // uniform
                lds_dma16(src[i] + (isa[i] ? o.a : o.b), dst + i * BLK);
    };
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < nk)
            issue(kt0 + s);
    for (int k = 0; k < nk; ++k) {
        const int later = min(nk - 1, k + NST - 2) - k;
        if (nb == C::WB_HI)
            wait_vm_steps<C::WB_HI, NST - 2>(later);
        else
            wait_vm_steps<C::WB_HI - 1, NST - 2>(later);
        __syncthreads();
        if (k + NST - 1 < nk)
            issue(kt0 + k + NST - 1);
        const uint8_t *As = L + (k % NST) * C::STAGE, *Bs = As + C::BM * C::ROWB;
#pragma unroll
        for (int g = 0; g < C::NG; ++g) {
            uint4 fa[C::MI], fb[C::NI];
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi)
                fa[mi] = LA == KM ? frag_km<DT>(As, RBA, wm * C::WM + mi * 32, g, lane)
                                  : *(const uint4 *)(As + swz<C>(wm * C::WM + mi * 32 + l32,
                                                                 2 * g + half));
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
                fb[ni] = LB == KM ? frag_km<DT>(Bs, RBB, wn * C::WN + ni * 32, g, lane)
                                  : *(const uint4 *)(Bs + swz<C>(wn * C::WN + ni * 32 + l32,
                                                                 2 * g + half));
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni)
                    mma_group<DT>(acc.v[mi][ni], fa[mi], fb[ni]);
        }
    }
    __syncthreads();
}

} // namespace ng
