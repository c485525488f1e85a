// Few-token (decode) layer: the gate + TwELL pack and the fused up/down
// ("Sparser, Faster, Lighter Transformer Language Models", summary page
// sections 2.B.1 and 2.B.2) shaped for T <= TWELL_DECODE_T tokens. There the
// many-token kernels leave most of the chip idle (their parallelism comes from
// tokens) and the layer is a matrix-vector product bound by weight reads.
//
// The work is split into three phases, each spread over the whole chip:
//
//  1. gate partials. A workgroup item is one TwELL tile (128 neurons) and one
//     of ks slices of d_model; the item's [T][128] partial goes to the
//     workspace. Up to GEMV_T tokens the product is a matrix-vector one: the
//     slice of x sits in LDS, eight lanes cover one 128-byte line of a W_g row
//     (a wave load reads eight whole lines), each lane keeps its own running
//     dot products over the slice's lines and the eight lanes of a row are
//     summed at the end. With more tokens the item is a [T][128] tile of g
//     over its slice on the shared LDS-DMA MFMA main loop (ntgemm.hpp), which
//     loads every operand line whole, and each wave stores its accumulators.
//  2. pack + up. A wave item is one (token, tile): it sums the ks partials in
//     slice order, packs the tile with two ballots into the TwELL arrays, and
//     for each stored nonzero (i, h) gathers wu_t[i] and stores
//     a = h * (x[t] . wu_t[i]) in the workspace, one float per TwELL slot.
//  3. down. A workgroup item is one token and one 1 KB slice of d_model: its
//     waves share the token's (i, a) list, each gathers the slice of wd[i] for
//     its entries, and the partial slices are summed in LDS in a fixed order.
//
// Each phase is its own launch: a kernel boundary costs a few microseconds,
// while a grid-wide barrier inside one cooperative launch was measured at
// about 15 us on MI355X (the eight XCDs' L2s must be written back and
// invalidated for every workgroup), so the single-kernel form is slower.
//   twell_gate_pack (few tokens): phase 1, then phase 2 without the up part.
//   twell_decode_fwd:             phases 1, 2 and 3.
//   twell_ffn_fwd (few tokens):   the up part of phase 2 (reading the TwELL),
//                                 then phase 3.
#include <algorithm>

#include "ntgemm.hpp"
#include "rows.hpp"

namespace {

constexpr int DW = 8;          // waves per workgroup
constexpr int DNT = 64 * DW;
constexpr int LISTD = 2048;    // entries staged per pass of the down phase
constexpr int GD = 8;          // wd slices in flight per wave in the down phase
constexpr int SPT = 4;         // TwELL slots per thread per round of the down phase's list
constexpr int GATE_ITEMS = 256; // aim: about one gate item per compute unit
constexpr int GEMV_T = 4;      // most tokens of the matrix-vector gate
constexpr int GLB = 8;         // W_g lines per row in flight per lane (matrix-vector gate)

// Host-computed geometry of one decode call.
struct DecPlan {
    int T, dm, dff, nt, W;
    int ks;      // d_model slices per tile (gate items)
    int nsl;     // 1 KB slices of a d_model row (down items per token)
    int nk;      // 64-byte K steps of a d_model row (tiled MFMA gate)
    bool gemv;   // matrix-vector gate: item k covers 128-byte lines [k lpi, (k + 1) lpi)
    int nl, lpi; // 128-byte lines of a d_model row, lines per gate item
    size_t a_off, bytes; // workspace: partials [ks][T][dff] at 0, a [T][nt][W] at a_off
};

DecPlan dec_plan(int dt, int T, int dm, int dff, int W, bool with_gate)
{
    const int esz = dt == TWELL_BF16 ? 2 : 4;
    DecPlan P{};
    P.T = T;
    P.dm = dm;
    P.dff = dff;
    P.nt = dff / TWELL_TILE_C;
    P.W = W;
    P.gemv = T <= GEMV_T;
    P.nl = dm * esz / 128; // d_model % 64 == 0: whole lines
    P.nk = dm * esz / 64;
    if (P.gemv) { // about one item per compute unit
        const int ks0 = std::max(1, std::min(GATE_ITEMS / P.nt, P.nl));
        P.lpi = (P.nl + ks0 - 1) / ks0;
        P.ks = (P.nl + P.lpi - 1) / P.lpi;
    } else {
        // tiled MFMA gate: about two items per compute unit, at least 12 K
        // steps per item, the partials at most half of W_g's bytes
        int ks = std::max(1, 2 * GATE_ITEMS / P.nt);
        ks = std::min(ks, std::max(1, P.nk / 12));
        P.ks = std::min(ks, std::max(1, dm * esz / (8 * std::max(T, 1))));
    }
    P.nsl = (dm * esz + 1023) / 1024;
    const size_t part = with_gate ? (size_t)P.ks * T * dff * 4 : 0;
    P.a_off = (part + 255) / 256 * 256;
    P.bytes = P.a_off + (size_t)T * P.nt * W * 4;
    return P;
}

template <int DT> DEVI float as_stored(float v)
{
    if constexpr (DT == TWELL_BF16)
        return bf16_to_f32(f32_to_bf16(v));
    else
        return v;
}

// Tile j of one token: lane l holds g for columns l (g0) and 64 + l (g1).
// Writes count, col and val of the tile; returns the two ballots.
template <int DT>
DEVI void pack_tile(float g0, float g1, size_t tj, int n0, int W, int lane, int32_t *count,
                    int16_t *col, void *val, int32_t *status, uint64_t &m0, uint64_t &m1)
{
    using E = elem<DT>;
    m0 = __ballot(g0 > 0.f);
    m1 = __ballot(g1 > 0.f);
    const uint64_t below = (1ull << lane) - 1ull;
    const int c0 = __popcll(m0), n = c0 + __popcll(m1);
    if (g0 > 0.f) {
        const int p = __popcll(m0 & below);
        if (p < W) {
            col[tj * W + p] = (int16_t)(n0 + lane);
            E::store1(val, tj * W + p, g0);
        }
    }
    if (g1 > 0.f) {
        const int p = c0 + __popcll(m1 & below);
        if (p < W) {
            col[tj * W + p] = (int16_t)(n0 + 64 + lane);
            E::store1(val, tj * W + p, g1);
        }
    }
    if (lane == 0) {
        count[tj] = n;
        if (n > W)
            raise_status(status, TWELL_DEV_TILE_OVERFLOW);
    }
}

// Matrix-vector form of phase 1 (T <= GEMV_T, TT = T rounded up to a power of
// two): item = (tile, slice of lpi lines). Lane 8q + c of wave w covers
// 16-byte chunk c of one line of rows 16w + q and 16w + 8 + q; xs holds the
// slice of x, [T][lpi * 8] chunks.
template <int DT, int TT>
DEVI void gate_gemv_item(const DecPlan &P, const uint8_t *__restrict__ x,
                         const uint8_t *__restrict__ wg, int item, float *__restrict__ part,
                         uint4 *xs)
{
    using E = elem<DT>;
    constexpr int EPL = E::per16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, q = lane >> 3, c = lane & 7;
    const int j = item / P.ks, k = item % P.ks, n0 = j * TWELL_TILE_C;
    const int l0 = k * P.lpi, nli = min(P.nl, l0 + P.lpi) - l0;
    const size_t rowbytes = (size_t)P.nl * 128;
    for (int i = threadIdx.x; i < P.T * nli * 8; i += DNT) {
        const int t = i / (nli * 8), r = i % (nli * 8);
        xs[t * P.lpi * 8 + r] = ldg16(x + (size_t)t * rowbytes + (size_t)l0 * 128 + r * 16);
    }
    __syncthreads();
    const uint8_t *w0 = wg + (size_t)(n0 + 16 * wave + q) * rowbytes + (size_t)l0 * 128 + c * 16;
    const uint8_t *w1 = w0 + 8 * rowbytes;
    float acc[2][TT];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int t = 0; t < TT; ++t)
            acc[g][t] = 0.f;
    for (int lb = 0; lb < nli; lb += GLB) {
        uint4 v[2][GLB];
#pragma unroll
        for (int u = 0; u < GLB; ++u) {
            const int l = min(lb + u, nli - 1); // lines past the slice re-read its last, unused
            v[0][u] = ldg16(w0 + (size_t)l * 128);
            v[1][u] = ldg16(w1 + (size_t)l * 128);
        }
#pragma unroll
        for (int u = 0; u < GLB; ++u)
            if (lb + u < nli) { // uniform
                float f0[EPL], f1[EPL];
                E::widen(v[0][u], f0);
                E::widen(v[1][u], f1);
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    float xf[EPL];
                    E::widen(xs[min(t, P.T - 1) * P.lpi * 8 + (lb + u) * 8 + c], xf);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        acc[0][t] += f0[e] * xf[e];
                        acc[1][t] += f1[e] * xf[e];
                    }
                }
            }
    }
    // the eight lanes of a row: a fixed butterfly, then lane c == 0 stores
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float s = acc[g][t];
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            s += __shfl_xor(s, 4, 64);
            if (c == 0 && t < P.T)
                part[((size_t)k * P.T + t) * P.dff + n0 + 16 * wave + 8 * g + q] = s;
        }
}

// ---------------------------------------------------------------- phase 2
// a = h * (x[t] . wu_t[c]) for the ns stored entries of one (token, tile),
// with G rows of wu_t in flight. next() yields the entries' global columns in
// slot order, hval(c) the stored value of the entry just handed out for
// column c (both wave-uniform).
template <int DT, int NW, int G, class Next, class HVal>
DEVI void up_entries(const Row<DT, NW> &geo, const uint32_t (&xw)[NW], const uint8_t *wu, int ns,
                     float *arow, int lane, Next next, HVal hval)
{
    int cq[G];
    float hq[G];
    uint32_t vu[G][NW];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (g < ns) { // uniform
            cq[g] = next();
            hq[g] = hval(cq[g]);
        } else {
            cq[g] = cq[0];
            hq[g] = 0.f;
        }
        geo.load_w(wu, cq[g], vu[g]);
    }
    for (int s0 = 0; s0 < ns; s0 += G) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int s = s0 + g;
            const float u = wave_sum(geo.dotw(xw, vu[g]));
            if (s < ns && lane == 0)
                arow[s] = hq[g] * u;
            if (s + G < ns) { // uniform: the next entry for this buffer
                cq[g] = next();
                hq[g] = hval(cq[g]);
                geo.load_w(wu, cq[g], vu[g]);
            }
        }
    }
}

// UP = false: pack only (twell_gate_pack).
template <int DT, int NW, int G, bool UP>
DEVI void pack_up_item(const DecPlan &P, const uint8_t *__restrict__ x,
                       const uint8_t *__restrict__ wu, const float *__restrict__ part, int p,
                       int32_t *count, int16_t *col, void *val, float *aw, int32_t *status)
{
    const int lane = threadIdx.x & 63;
    const int t = p / P.nt, j = p % P.nt, n0 = j * TWELL_TILE_C;
    // sum of the ks partials in slice order
    const float *pp = part + (size_t)t * P.dff + n0 + lane;
    const size_t ksd = (size_t)P.T * P.dff;
    float g0 = 0.f, g1 = 0.f;
    for (int k0 = 0; k0 < P.ks; k0 += 8) {
        float a[8], b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const size_t o = (size_t)min(k0 + u, P.ks - 1) * ksd;
            a[u] = pp[o];
            b[u] = pp[o + 64];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (k0 + u < P.ks) {
                g0 += a[u];
                g1 += b[u];
            }
    }
    uint64_t m0, m1;
    pack_tile<DT>(g0, g1, (size_t)p, n0, P.W, lane, count, col, val, status, m0, m1);
    const int ns = min(__popcll(m0) + __popcll(m1), P.W);
    if (!UP || ns == 0)
        return;
    const Row<DT, NW> geo(P.dm, lane, 0);
    uint32_t xw[NW];
    geo.load_w(x, t, xw);
    const float h0 = as_stored<DT>(g0), h1 = as_stored<DT>(g1);
    uint64_t r0 = m0, r1 = m1; // columns not yet handed out
    up_entries<DT, NW, G>(
        geo, xw, wu, ns, aw + (size_t)p * P.W, lane,
        [&]() {
            int c;
            if (r0) {
                c = __builtin_ctzll(r0);
                r0 &= r0 - 1;
            } else {
                c = 64 + __builtin_ctzll(r1);
                r1 &= r1 - 1;
            }
            return n0 + c;
        },
        [&](int c) { return bcast(c - n0 < 64 ? h0 : h1, (c - n0) & 63); });
}

// Up only, from a TwELL (few-token twell_ffn_fwd): wave item p = (token, tile).
template <int DT, int NW, int G>
DEVI void up_item(const DecPlan &P, const uint8_t *__restrict__ x, const uint8_t *__restrict__ wu,
                  const int32_t *__restrict__ count, const int16_t *__restrict__ col,
                  const void *__restrict__ val, int p, float *aw, int32_t *status)
{
    using E = elem<DT>;
    const int lane = threadIdx.x & 63;
    const int t = p / P.nt;
    const int ns = min(count[p], P.W);
    if (ns <= 0)
        return;
    // slots lane and 64 + lane (W <= 128); a corrupt column is reported and
    // its entry contributes nothing
    const size_t src = (size_t)p * P.W;
    int cA = 0, cB = 0;
    float vA = 0.f, vB = 0.f;
    if (lane < ns) {
        cA = col[src + lane];
        vA = E::load1(val, src + lane);
    }
    if (64 + lane < ns) {
        cB = col[src + 64 + lane];
        vB = E::load1(val, src + 64 + lane);
    }
    if (cA < 0 || cA >= P.dff) {
        raise_status(status, TWELL_DEV_BAD_INDEX);
        cA = 0;
        vA = 0.f;
    }
    if (cB < 0 || cB >= P.dff) {
        raise_status(status, TWELL_DEV_BAD_INDEX);
        cB = 0;
        vB = 0.f;
    }
    const Row<DT, NW> geo(P.dm, lane, 0);
    uint32_t xw[NW];
    geo.load_w(x, t, xw);
    int s = 0; // slot handed out next
    int sv = 0; // slot whose value is asked for next
    up_entries<DT, NW, G>(
        geo, xw, wu, ns, aw + src, lane,
        [&]() {
            const int c = bcast(s < 64 ? cA : cB, s & 63);
            ++s;
            return c;
        },
        [&](int) {
            const float v = bcast(sv < 64 ? vA : vB, sv & 63);
            ++sv;
            return v;
        });
}

// ---------------------------------------------------------------- phase 3
// y[t][slice] = sum over token t's stored entries of a * wd[c][slice].
template <int DT>
DEVI void down_item(const DecPlan &P, const int32_t *__restrict__ count,
                    const int16_t *__restrict__ col, const float *__restrict__ aw,
                    const uint8_t *__restrict__ wd, int q, float *__restrict__ y, int32_t *status,
                    float *smem)
{
    using E = elem<DT>;
    constexpr int esz = sizeof(typename E::storage);
    constexpr int EPL = E::per16;     // elements per lane (16 bytes)
    constexpr int SLE = 64 * EPL;     // elements per slice (1 KB)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int *lcol = (int *)smem;
    float *la = smem + LISTD;
    int *tstart = (int *)(smem + 2 * LISTD); // [nt] tile starts, [nt] total (nt <= 256)
    float *red = smem + 2 * LISTD + 260;     // [DW][SLE]
    const int t = q / P.nsl, e0 = (q % P.nsl) * SLE;
    const bool in = e0 + lane * EPL < P.dm;
    const size_t rowbytes = (size_t)P.dm * esz;
    const uint8_t *wdl = wd + (size_t)(e0 + lane * EPL) * esz;
    // The token's slots (tile j, slot s) are q = j W + s. When there are few
    // enough, every thread requests the column and a of its SPT slots before
    // the count scan, so both wait on one trip to memory; entries are kept
    // only where s < the tile's count.
    const int nslots = P.nt * P.W;
    const bool ahead = nslots <= SPT * DNT;
    const size_t tsl = (size_t)t * nslots;
    int cpre[SPT];
    float apre[SPT];
    if (ahead)
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int qs = min((int)threadIdx.x + u * DNT, nslots - 1); // past the end: unused
            cpre[u] = col[tsl + qs];
            apre[u] = aw[tsl + qs];
        }
    if (wave == 0) {
        int run = 0;
        for (int jb = 0; jb < P.nt; jb += 64) {
            const int jj = jb + lane;
            const int n = jj < P.nt ? min(max(count[(size_t)t * P.nt + jj], 0), P.W) : 0;
            const int incl = wave_incl_scan(n, lane);
            if (jj < P.nt)
                tstart[jj] = run + incl - n;
            run += __shfl(incl, 63, 64);
        }
        if (lane == 0)
            tstart[P.nt] = run;
    }
    __syncthreads();
    const int total = tstart[P.nt];
    float acc[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        acc[i] = 0.f;
    for (int p0 = 0; p0 < total; p0 += LISTD) {
        // list entries [p0, p0 + LISTD): SPT slots per thread per round, the
        // round's loads in flight together
        for (int q0 = threadIdx.x; q0 < nslots; q0 += SPT * DNT) {
            int pos[SPT], c[SPT];
            float a[SPT];
#pragma unroll
            for (int u = 0; u < SPT; ++u) {
                const int qs = q0 + u * DNT;
                pos[u] = -1;
                if (qs < nslots) {
                    const int j = qs / P.W, sl = qs % P.W, st = tstart[j];
                    const int e = st + sl - p0;
                    if (sl < tstart[j + 1] - st && e >= 0 && e < LISTD) {
                        pos[u] = e;
                        c[u] = ahead ? cpre[u] : col[tsl + qs];
                        a[u] = ahead ? apre[u] : aw[tsl + qs];
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < SPT; ++u)
                if (pos[u] >= 0) {
                    if (c[u] < 0 || c[u] >= P.dff) { // corrupt entry: skipped and reported
                        raise_status(status, TWELL_DEV_BAD_INDEX);
                        c[u] = 0;
                        a[u] = 0.f;
                    }
                    lcol[pos[u]] = c[u];
                    la[pos[u]] = a[u];
                }
        }
        __syncthreads();
        const int ne = min(LISTD, total - p0);
        for (int e = wave; e < ne; e += DW * GD) {
            uint4 v[GD];
#pragma unroll
            for (int g = 0; g < GD; ++g) {
                const int c = lcol[min(e + DW * g, ne - 1)];
                v[g] = in ? ldg16(wdl + (size_t)c * rowbytes) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int g = 0; g < GD; ++g)
                if (e + DW * g < ne) { // uniform
                    const float a = la[e + DW * g];
                    float f[EPL];
                    E::widen(v[g], f);
#pragma unroll
                    for (int i = 0; i < EPL; ++i)
                        acc[i] += a * f[i];
                }
        }
        __syncthreads(); // the list is rewritten by the next pass
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        red[wave * SLE + lane * EPL + i] = acc[i];
    __syncthreads();
    for (int i = threadIdx.x; i < SLE; i += DNT)
        if (e0 + i < P.dm) {
            float s = red[i];
#pragma unroll
            for (int w = 1; w < DW; ++w)
                s += red[w * SLE + i];
            y[(size_t)t * P.dm + e0 + i] = s;
        }
    __syncthreads(); // smem is reused by the next item
}

size_t down_lds() { return (2 * LISTD + 260 + DW * 512) * 4; }

// ---------------------------------------------------------------- kernels
template <int DT, int TT>
__global__ __launch_bounds__(DNT) void dec_gate_gemv_kernel(
    DecPlan P, const uint8_t *__restrict__ x, const uint8_t *__restrict__ wg, float *part)
{
    extern __shared__ __attribute__((aligned(16))) uint4 xs[];
    gate_gemv_item<DT, TT>(P, x, wg, blockIdx.x, part, xs);
}

// Phase 1 for more than GEMV_T tokens: item (tile j, slice k) is a [T][128]
// tile of g over K steps [k nk / ks, (k + 1) nk / ks) on the shared LDS-DMA
// MFMA main loop (C::BM = 32 or 64 token rows; rows past T repeat the last
// token and are not stored); each wave stores its accumulators as the item's
// partial. Every operand line is loaded whole, straight into LDS.
using GC32 = ng::Cfg<32, 128, 1, 4, 4, 64>; // up to 32 tokens: four waves of 32 x 32
using GC64 = ng::Cfg<64, 128, 2, 4, 4, 64>; // up to 64 tokens: eight waves of 32 x 32
template <int DT, class C>
__global__ __launch_bounds__(C::NT) void dec_gate_mm_kernel(DecPlan P, const uint8_t *__restrict__ x,
                                                            const uint8_t *__restrict__ wg,
                                                            float *__restrict__ part)
{
    __shared__ __attribute__((aligned(16))) uint8_t L[C::LDS];
    const int j = blockIdx.x / P.ks, k = blockIdx.x % P.ks, n0 = j * TWELL_TILE_C;
    const size_t rowbytes = (size_t)P.nk * 64;
    const int kt0 = (int)((long)P.nk * k / P.ks), kt1 = (int)((long)P.nk * (k + 1) / P.ks);
    auto rowa = [&](int r) { return x + (size_t)min(r, P.T - 1) * rowbytes; };
    auto rowb = [&](int r) { return wg + (size_t)(n0 + r) * rowbytes; };
    auto off = [](int kt) { return ng::StepOff{(size_t)kt * C::ROWB, (size_t)kt * C::ROWB}; };
    ng::Acc<C> acc;
    ng::mainloop<C, DT>(L, rowa, rowb, off, kt0, kt1, acc);
    const int lane = threadIdx.x & 63, wm = ng::wave_m<C>(), wn = ng::wave_n<C>();
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = ng::acc_row<C>(wm, mi, e, lane);
                if (r < P.T)
                    part[((size_t)k * P.T + r) * P.dff + n0 + ng::acc_col<C>(wn, ni, lane)] =
                        acc.v[mi][ni][e];
            }
}

template <int DT, int NW, int G, bool UP>
__global__ __launch_bounds__(DNT) void dec_pack_kernel(
    DecPlan P, const uint8_t *__restrict__ x, const uint8_t *__restrict__ wu,
    const float *__restrict__ part, int32_t *count, int16_t *col, void *val, float *aw,
    int32_t *status)
{
    const int p = blockIdx.x * DW + wave_id();
    if (p < P.T * P.nt)
        pack_up_item<DT, NW, G, UP>(P, x, wu, part, p, count, col, val, aw, status);
}

template <int DT, int NW, int G>
__global__ __launch_bounds__(DNT) void dec_up_kernel(
    DecPlan P, const uint8_t *__restrict__ x, const uint8_t *__restrict__ wu,
    const int32_t *__restrict__ count, const int16_t *__restrict__ col,
    const void *__restrict__ val, float *aw, int32_t *status)
{
    const int p = blockIdx.x * DW + wave_id();
    if (p < P.T * P.nt)
        up_item<DT, NW, G>(P, x, wu, count, col, val, p, aw, status);
}

template <int DT>
__global__ __launch_bounds__(DNT) void dec_down_kernel(
    DecPlan P, const int32_t *__restrict__ count, const int16_t *__restrict__ col,
    const float *__restrict__ aw, const uint8_t *__restrict__ wd, float *__restrict__ y,
    int32_t *status)
{
    extern __shared__ __attribute__((aligned(16))) float smem[];
    down_item<DT>(P, count, col, aw, wd, blockIdx.x, y, status, smem);
}

// words per lane for a row of ndw words: the smallest supported count
int dec_nw(int ndw)
{
    const int need = (ndw + 63) / 64;
    for (int v : {1, 2, 4, 8, 12, 16, 18, 24})
        if (v >= need)
            return v;
    return 32;
}

template <int NW> constexpr int up_g() { return NW <= 8 ? 4 : 2; } // wu rows in flight per wave

int pack_grid(const DecPlan &P) { return (P.T * P.nt + DW - 1) / DW; }

template <int DT>
void launch_gate_part(const DecPlan &P, const void *x, const void *wg, float *part, Timer &tm,
                      hipStream_t s)
{
    if (P.gemv) {
        const size_t lds = (size_t)P.T * P.lpi * 128;
        const uint8_t *xb = (const uint8_t *)x, *wb = (const uint8_t *)wg;
        const dim3 g(P.nt * P.ks), b(DNT);
        if (P.T == 1)
            hipLaunchKernelGGL((dec_gate_gemv_kernel<DT, 1>), g, b, lds, s, P, xb, wb, part);
        else if (P.T == 2)
            hipLaunchKernelGGL((dec_gate_gemv_kernel<DT, 2>), g, b, lds, s, P, xb, wb, part);
        else
            hipLaunchKernelGGL((dec_gate_gemv_kernel<DT, 4>), g, b, lds, s, P, xb, wb, part);
        tm.mark("dec_gate_gemv_kernel");
        return;
    }
    if (P.T > 32)
        hipLaunchKernelGGL((dec_gate_mm_kernel<DT, GC64>), dim3(P.nt * P.ks), dim3(GC64::NT), 0,
                           s, P, (const uint8_t *)x, (const uint8_t *)wg, part);
    else
        hipLaunchKernelGGL((dec_gate_mm_kernel<DT, GC32>), dim3(P.nt * P.ks), dim3(GC32::NT), 0,
                           s, P, (const uint8_t *)x, (const uint8_t *)wg, part);
    tm.mark("dec_gate_mm_kernel");
}

template <int DT>
void launch_down(const DecPlan &P, const twell_t *h, const void *wd, const float *aw, float *y,
                 int32_t *status, Timer &tm, hipStream_t s)
{
    hipLaunchKernelGGL(dec_down_kernel<DT>, dim3(P.T * P.nsl), dim3(DNT), down_lds(), s, P,
                       h->count, h->col, aw, (const uint8_t *)wd, y, status);
    tm.mark("dec_down_kernel");
}

template <int DT, int NW>
void launch_layer_nw(const DecPlan &P, const void *x, const void *wg, const void *wu,
                     const void *wd, const twell_t *o, float *y, float *ws, int32_t *status,
                     Timer &tm, hipStream_t s)
{
    float *aw = ws + P.a_off / 4;
    launch_gate_part<DT>(P, x, wg, ws, tm, s);
    hipLaunchKernelGGL((dec_pack_kernel<DT, NW, up_g<NW>(), true>), dim3(pack_grid(P)),
                       dim3(DNT), 0, s, P, (const uint8_t *)x, (const uint8_t *)wu, ws, o->count,
                       o->col, o->val, aw, status);
    tm.mark("dec_pack_up_kernel");
    launch_down<DT>(P, o, wd, aw, y, status, tm, s);
}

template <int DT, int NW>
void launch_ffn_nw(const DecPlan &P, const void *x, const twell_t *h, const void *wu,
                   const void *wd, float *y, float *aw, int32_t *status, Timer &tm,
                   hipStream_t s)
{
    hipLaunchKernelGGL((dec_up_kernel<DT, NW, up_g<NW>()>), dim3(pack_grid(P)), dim3(DNT), 0, s,
                       P, (const uint8_t *)x, (const uint8_t *)wu, h->count, h->col, h->val, aw,
                       status);
    tm.mark("dec_up_kernel");
    launch_down<DT>(P, h, wd, aw, y, status, tm, s);
}

#define DEC_NW_SWITCH(ndw, CALL)                                                         \
    switch (dec_nw(ndw)) {                                                               \
    case 1: CALL(1); break;                                                              \
    case 2: CALL(2); break;                                                              \
    case 4: CALL(4); break;                                                              \
    case 8: CALL(8); break;                                                              \
    case 12: CALL(12); break;                                                            \
    case 16: CALL(16); break;                                                            \
    case 18: CALL(18); break;                                                            \
    case 24: CALL(24); break;                                                            \
    default: CALL(32); break;                                                            \
    }

template <int DT>
void launch_layer_dt(const DecPlan &P, const void *x, const void *wg, const void *wu,
                     const void *wd, const twell_t *o, float *y, float *ws, int32_t *status,
                     Timer &tm, hipStream_t s)
{
    const int ndw = DT == TWELL_BF16 ? P.dm / 2 : P.dm;
#define DEC_LAYER(N) launch_layer_nw<DT, N>(P, x, wg, wu, wd, o, y, ws, status, tm, s)
    DEC_NW_SWITCH(ndw, DEC_LAYER)
#undef DEC_LAYER
}

template <int DT>
void launch_ffn_dt(const DecPlan &P, const void *x, const twell_t *h, const void *wu,
                   const void *wd, float *y, float *aw, int32_t *status, Timer &tm,
                   hipStream_t s)
{
    const int ndw = DT == TWELL_BF16 ? P.dm / 2 : P.dm;
#define DEC_FFN(N) launch_ffn_nw<DT, N>(P, x, h, wu, wd, y, aw, status, tm, s)
    DEC_NW_SWITCH(ndw, DEC_FFN)
#undef DEC_FFN
}

template <int DT>
void launch_gate_dt(const DecPlan &P, const void *x, const void *wg, const twell_t *o, float *ws,
                    int32_t *status, Timer &tm, hipStream_t s)
{
    launch_gate_part<DT>(P, x, wg, ws, tm, s);
    hipLaunchKernelGGL((dec_pack_kernel<DT, 1, 1, false>), dim3(pack_grid(P)), dim3(DNT), 0, s, P,
                       (const uint8_t *)x, (const uint8_t *)nullptr, ws, o->count, o->col, o->val,
                       (float *)nullptr, status);
    tm.mark("dec_pack_kernel");
}

} // namespace

size_t dec_gate_workspace(int dt, int T, int dm, int dff)
{
    const DecPlan P = dec_plan(dt, T, dm, dff, 1, true);
    return P.a_off;
}

size_t dec_ffn_workspace(int dt, int T, int dm, int dff, int W)
{
    return dec_plan(dt, T, dm, dff, W, false).bytes;
}

size_t dec_layer_workspace(int dt, int T, int dm, int dff, int W)
{
    return dec_plan(dt, T, dm, dff, W, true).bytes;
}

hipError_t launch_dec_gate(twell_dtype dt, const void *x, const void *wg_t, int T, int dm,
                           const twell_t *o, void *ws, int32_t *status, Timer &tm, hipStream_t s)
{
    const DecPlan P = dec_plan(dt, T, dm, o->d_ff, o->width, true);
    if (dt == TWELL_BF16)
        launch_gate_dt<TWELL_BF16>(P, x, wg_t, o, (float *)ws, status, tm, s);
    else
        launch_gate_dt<TWELL_F32>(P, x, wg_t, o, (float *)ws, status, tm, s);
    return hipGetLastError();
}

hipError_t launch_dec_ffn(twell_dtype dt, const void *x, const twell_t *h, const void *wu_t,
                          const void *wd, int dm, float *y, void *ws, int32_t *status, Timer &tm,
                          hipStream_t s)
{
    const DecPlan P = dec_plan(dt, h->T, dm, h->d_ff, h->width, false);
    float *aw = (float *)((uint8_t *)ws + P.a_off);
    if (dt == TWELL_BF16)
        launch_ffn_dt<TWELL_BF16>(P, x, h, wu_t, wd, y, aw, status, tm, s);
    else
        launch_ffn_dt<TWELL_F32>(P, x, h, wu_t, wd, y, aw, status, tm, s);
    return hipGetLastError();
}

hipError_t launch_dec_layer(twell_dtype dt, const void *x, const void *wg_t, const void *wu_t,
                            const void *wd, int dm, const twell_t *o, float *y, void *ws,
                            int32_t *status, twell_timing_t *timing, hipStream_t s)
{
    Timer tm(timing, s);
    const DecPlan P = dec_plan(dt, o->T, dm, o->d_ff, o->width, true);
    if (dt == TWELL_BF16)
        launch_layer_dt<TWELL_BF16>(P, x, wg_t, wu_t, wd, o, y, (float *)ws, status, tm, s);
    else
        launch_layer_dt<TWELL_F32>(P, x, wg_t, wu_t, wd, o, y, (float *)ws, status, tm, s);
    return hipGetLastError();
}
