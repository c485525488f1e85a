// 128 x 128 MFMA output tiles for the dense products of this library.
//
// A workgroup of four wave64s computes a 128 x 128 fp32 tile C = A B^T, with
// A (rows m) and B (rows n) both indexed by a shared K. Each wave owns a
// 64 x 64 quarter as 2 x 2 blocks of 32x32 MFMA accumulators. K advances in
// steps of 128 bytes per row (64 bf16 or 32 f32); each step of both operands
// is staged in LDS as [row][128 bytes], XOR-swizzled in 16-byte chunks, double
// buffered, with the global loads of step k+1 in flight during step k.
//
// An operand is fetched from memory in one of two shapes:
//   K-contiguous  : the operand's row (m or n) is a memory row along K;
//   MN-contiguous : the operand's K index picks a memory row whose elements
//                   run along m or n (it is transposed on the way into LDS).
#pragma once

#include "common.hpp"

namespace mt {

constexpr int TILE = 128;
constexpr int ROWB = 128;
constexpr int NT = 256;

// Byte offset of 16-byte chunk c of LDS row r (128-byte rows). A 128-bit
// fragment read serves 16 lanes per LDS cycle across 64 banks: 16 consecutive
// rows, same chunk. Row r starts at bank 32 * (r % 2), so XOR-ing the chunk with
// (r / 2) % 8 gives those 16 rows 16 distinct bank groups (no conflicts).
DEVI int swz(int r, int c) { return r * ROWB + ((c ^ ((r >> 1) & 7)) << 4); }

template <int DT> DEVI void mma_group(floatx16_t &acc, const uint4 &a, const uint4 &b);

template <> DEVI void mma_group<TWELL_BF16>(floatx16_t &acc, const uint4 &a, const uint4 &b)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

template <> DEVI void mma_group<TWELL_F32>(floatx16_t &acc, const uint4 &a, const uint4 &b)
{
    // element q of both operands is the same k: four K=2 MFMAs cover the chunk
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

typedef floatx16_t Acc[2][2];

DEVI void zero(Acc &acc)
{
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[mi][ni][e] = 0.f;
}

// One K step from LDS.
template <int DT>
DEVI void step(Acc &acc, const uint8_t *As, const uint8_t *Bs, int wm, int wn, int lane)
{
    const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        uint4 fa[2], fb[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
            fa[mi] = *(const uint4 *)(As + swz(wm * 64 + mi * 32 + l32, 2 * g + half));
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
            fb[ni] = *(const uint4 *)(Bs + swz(wn * 64 + ni * 32 + l32, 2 * g + half));
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                mma_group<DT>(acc[mi][ni], fa[mi], fb[ni]);
    }
}

struct Stage {
    uint4 v[4];
};

// K-contiguous operand. rowp(r) gives the address of the current K step of
// tile row r (0..127), or nullptr for a row outside the operand (read as 0).
template <class RowP> DEVI void load_k(Stage &st, RowP rowp, int tid)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + NT * i, r = q >> 3, c = q & 7;
        const uint8_t *p = rowp(r);
        st.v[i] = p ? ldg16(p + c * 16) : make_uint4(0, 0, 0, 0);
    }
}

DEVI void store_k(uint8_t *S, const Stage &st, int tid)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + NT * i, r = q >> 3, c = q & 7;
        *(uint4 *)(S + swz(r, c)) = st.v[i];
    }
}

// MN-contiguous operand. krowp(kk) gives the address of element (tile row 0,
// k = kk of this step), or nullptr for a k outside the operand (read as 0);
// col_ok(r0) says whether tile rows r0.. of a 16-byte chunk exist.
template <int DT, class KRowP, class ColOk>
DEVI void load_mn(Stage &st, KRowP krowp, ColOk col_ok, int tid)
{
    constexpr int esz = sizeof(typename elem<DT>::storage);
    constexpr int CPK = TILE * esz / 16; // 16-byte chunks per k row
    constexpr int P = 16 / esz;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + NT * i, kk = q / CPK, cc = q % CPK;
        const uint8_t *p = krowp(kk);
        st.v[i] = (p && col_ok(cc * P)) ? ldg16(p + cc * 16) : make_uint4(0, 0, 0, 0);
    }
}

template <int DT> DEVI void store_mn(uint8_t *S, const Stage &st, int tid)
{
    constexpr int esz = sizeof(typename elem<DT>::storage);
    constexpr int CPK = TILE * esz / 16;
    constexpr int P = 16 / esz;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + NT * i, kk = q / CPK, cc = q % CPK;
        const int kb = kk * esz;
        const uint32_t w[4] = {st.v[i].x, st.v[i].y, st.v[i].z, st.v[i].w};
#pragma unroll
        for (int e = 0; e < P; ++e) {
            const int r = cc * P + e;
            uint8_t *dst = S + swz(r, kb >> 4) + (kb & 15);
            if (esz == 2)
                *(uint16_t *)dst = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            else
                *(uint32_t *)dst = w[e];
        }
    }
}

// The pipelined K loop. load_a/load_b(stage, kt) fetch step kt from memory,
// store_a/store_b(lds, stage) put it in LDS. Ends with a barrier, so the LDS
// buffers may be reused right after.
template <int DT, class LA, class SA, class LB, class SB>
DEVI void gemm(Acc &acc, uint8_t (*As)[TILE * ROWB], uint8_t (*Bs)[TILE * ROWB], int nk, LA load_a,
               SA store_a, LB load_b, SB store_b, int wm, int wn, int lane)
{
    if (nk <= 0)
        return;
    Stage sa, sb;
    load_a(sa, 0);
    load_b(sb, 0);
    store_a(As[0], sa);
    store_b(Bs[0], sb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int b = kt & 1;
        if (kt + 1 < nk) {
            load_a(sa, kt + 1);
            load_b(sb, kt + 1);
        }
        step<DT>(acc, As[b], Bs[b], wm, wn, lane);
        if (kt + 1 < nk) {
            store_a(As[b ^ 1], sa);
            store_b(Bs[b ^ 1], sb);
        }
        __syncthreads();
    }
}

// LDS of a 128 x 128 tile GEMM: two double-buffered 128 x 128-byte stages
typedef uint8_t (*Tiles)[TILE * ROWB];
constexpr int TILE_LDS = 4 * TILE * ROWB; // As[2] + Bs[2]: 64 KB

// Float32 intermediates of the backup rows' products, array q of [rows][cols]
// arrays `stride` elements apart. For bf16 inputs each value v is stored as
// two bf16, hi = bf16(v) and lo = bf16(v - hi) (arrays 2q and 2q + 1), so a
// bf16 MFMA product over both keeps about 16 significant bits; float32
// inputs store v as is.
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

// Tile coordinates of accumulator element e of block (mi, ni) of this lane.
DEVI int acc_row(int wm, int mi, int e, int lane) { return wm * 64 + mi * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }
DEVI int acc_col(int wn, int ni, int lane) { return wn * 64 + ni * 32 + (lane & 31); }

} // namespace mt
