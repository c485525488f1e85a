// TwELL -> hybrid ELL + dense backup ("Sparser, Faster, Lighter Transformer
// Language Models", summary page section 2.B.3: training sparsity is uneven,
// so rows with few nonzeros go to a compact ELL matrix and overflow rows are
// redirected to a dense backup, through a dedicated conversion kernel).
//
// Three launches, all integer / copy work:
//   1. rows:  one wave per row sums the tile counts (row_nnz) and, for a row
//             with row_nnz <= K, concatenates its tiles into ELL row t; the
//             tiles are in column order, so the ELL row is ascending.
//   2. slots: one thread per row; a workgroup counts the overflow rows of
//             the blocks before its own (a reduction over row_nnz) and scans
//             its block's flags, so backup slots follow ascending row order;
//             writes row_slot and ovf_rows, and the last block n_ovf.
//   3. dense: one workgroup per backup slot builds that row (zeros, then its
//             entries) in LDS and stores it with 16-byte lanes, all backup
//             rows at once.
#include "common.hpp"

namespace {

template <int DT>
__global__ __launch_bounds__(256) void hyb_rows_kernel(
    const int32_t *__restrict__ count, const int16_t *__restrict__ col,
    const void *__restrict__ val, int T, int nt, int W, int K, int32_t *__restrict__ row_nnz,
    int16_t *__restrict__ ell_col, void *__restrict__ ell_val)
{
    using S = typename elem<DT>::storage;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave_id();
    if (t >= T)
        return;
    // tile j's n stored entries to ELL slots [excl, excl + n) of row t, 8 at a
    // time with all loads of a lane in flight together; only stored slots are
    // read: each lane reads its own tile, so every load is a request of its
    // own, and most tiles hold one or two entries
    auto copy = [&](int j, int n, int excl) {
        const size_t src = ((size_t)t * nt + j) * W;
        const size_t dst = (size_t)t * K + excl;
        for (int s0 = 0; s0 < n; s0 += 8) {
            int16_t c[8];
            S v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < n) {
                    c[u] = col[src + s0 + u];
                    v[u] = ((const S *)val)[src + s0 + u];
                }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < n) {
                    ell_col[dst + s0 + u] = c[u];
                    ((S *)ell_val)[dst + s0 + u] = v[u];
                }
        }
    };
    if (nt <= 64) { // one tile per lane: the counts are read once
        const int n = lane < nt ? min(count[(size_t)t * nt + lane], W) : 0;
        const int incl = wave_incl_scan(n, lane);
        const int total = __shfl(incl, 63, 64);
        if (lane == 0)
            row_nnz[t] = total;
        if (total <= K) // otherwise an overflow row: it goes to the dense backup
            copy(lane, n, incl - n);
        return;
    }
    int total = 0;
    for (int j0 = 0; j0 < nt; j0 += 64) {
        const int j = j0 + lane;
        const int n = j < nt ? min(count[(size_t)t * nt + j], W) : 0;
        total += __shfl(wave_incl_scan(n, lane), 63, 64);
    }
    if (lane == 0)
        row_nnz[t] = total;
    if (total > K)
        return; // overflow row: goes to the dense backup
    int base = 0;
    for (int j0 = 0; j0 < nt; j0 += 64) {
        const int j = j0 + lane;
        const int n = j < nt ? min(count[(size_t)t * nt + j], W) : 0;
        const int incl = wave_incl_scan(n, lane);
        copy(j, n, base + incl - n);
        base += __shfl(incl, 63, 64);
    }
}

constexpr int SNT = 256;       // threads (and rows) per workgroup of the slot launch
constexpr int DNT = 256;       // threads per workgroup of the dense launch
constexpr int ROW_LDS = 32768; // bytes of one dense row built in LDS (d_ff 16384 bf16 / 8192 f32)

__global__ __launch_bounds__(SNT) void hyb_slots_kernel(
    const int32_t *__restrict__ row_nnz, int T, int K, int max_ovf,
    int32_t *__restrict__ row_slot, int32_t *__restrict__ ovf_rows, int32_t *__restrict__ n_ovf,
    int32_t *__restrict__ status)
{
    __shared__ int wsum[SNT / 64];
    __shared__ int n_before;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r0 = blockIdx.x * SNT;
    if (tid == 0)
        n_before = 0;
    __syncthreads();
    // overflow rows of the blocks before this one: 8 loads per thread in
    // flight (rows clamped, flags masked), per-thread counts summed in LDS
    int mine = 0;
    for (int t0 = 0; t0 < r0; t0 += 8 * SNT) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = row_nnz[min(t0 + u * SNT + tid, r0 - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            mine += (t0 + u * SNT + tid < r0 && v[u] > K) ? 1 : 0;
    }
    if (mine)
        atomicAdd(&n_before, mine);
    // this block: one flag per thread, slots by a block scan (ballots per
    // wave, wave totals in LDS)
    const int t = r0 + tid;
    const bool f = t < T && row_nnz[t] > K;
    const unsigned long long m = __ballot(f);
    if (lane == 0)
        wsum[wv] = __popcll(m);
    __syncthreads();
    int before = n_before;
    for (int w = 0; w < wv; ++w)
        before += wsum[w];
    const int slot = before + __popcll(m & ((1ull << lane) - 1ull));
    if (t < T) {
        row_slot[t] = f ? slot : -1;
        if (f && slot < max_ovf)
            ovf_rows[slot] = t;
    }
    if (tid == SNT - 1 && r0 + SNT >= T) { // last block: the true total
        int total = n_before;
        for (int w = 0; w < SNT / 64; ++w)
            total += wsum[w];
        *n_ovf = total;
        if (total > max_ovf)
            raise_status(status, TWELL_DEV_OVF_CAPACITY);
    }
}

template <int DT>
__global__ __launch_bounds__(DNT) void hyb_dense_kernel(
    const int32_t *__restrict__ count, const int16_t *__restrict__ col,
    const void *__restrict__ val, int nt, int W, int dff, int max_ovf,
    const int32_t *__restrict__ ovf_rows, const int32_t *__restrict__ n_ovf,
    void *__restrict__ dense, int32_t *__restrict__ status)
{
    using S = typename elem<DT>::storage;
    __shared__ __attribute__((aligned(16))) uint8_t rowbuf[ROW_LDS];
    const int slot = blockIdx.x, tid = threadIdx.x;
    if (slot >= min(*n_ovf, max_ovf))
        return;
    const int t = ovf_rows[slot];
    S *drow = (S *)dense + (size_t)slot * dff;
    // rows wider than the LDS buffer are built straight in memory
    const bool in_lds = (size_t)dff * sizeof(S) <= ROW_LDS;
    S *brow = in_lds ? (S *)rowbuf : drow;
    if (in_lds)
        for (int i = tid; i < dff * (int)sizeof(S) / 16; i += DNT)
            ((uint4 *)rowbuf)[i] = make_uint4(0, 0, 0, 0);
    else
        for (int i = tid; i < dff; i += DNT)
            drow[i] = S(0);
    __syncthreads();
    // every slot of the row's TwELL tiles, 8 per thread at a time (loads
    // unconditional, stores of the stored slots only)
    const size_t src = (size_t)t * nt * W;
    const int nslot = nt * W;
    for (int q0 = 0; q0 < nslot; q0 += 8 * DNT) {
        int c[8], n[8];
        S v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int q = min(q0 + u * DNT + tid, nslot - 1);
            n[u] = count[(size_t)t * nt + q / W];
            c[u] = col[src + q];
            v[u] = ((const S *)val)[src + q];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int q = q0 + u * DNT + tid;
            if (q < nslot && q % W < min(n[u], W)) {
                if (c[u] >= 0 && c[u] < dff)
                    brow[c[u]] = v[u];
                else
                    raise_status(status, TWELL_DEV_BAD_INDEX);
            }
        }
    }
    if (in_lds) {
        __syncthreads();
        for (int i = tid; i < dff * (int)sizeof(S) / 16; i += DNT)
            ((uint4 *)drow)[i] = ((const uint4 *)rowbuf)[i];
    }
}

template <int DT>
hipError_t launch(const twell_t *h, const hybrid_t *o, int32_t *status, Timer &tm, hipStream_t s)
{
    const int nt = h->d_ff / TWELL_TILE_C;
    if (h->T > 0) {
        hipLaunchKernelGGL(hyb_rows_kernel<DT>, dim3((h->T + 3) / 4), dim3(256), 0, s, h->count,
                           h->col, h->val, h->T, nt, h->width, o->K, o->row_nnz, o->ell_col,
                           o->ell_val);
        tm.mark("hyb_rows_kernel");
    }
    hipLaunchKernelGGL(hyb_slots_kernel, dim3(h->T > 0 ? (h->T + SNT - 1) / SNT : 1), dim3(SNT),
                       0, s, o->row_nnz, h->T, o->K, o->max_ovf, o->row_slot, o->ovf_rows,
                       o->n_ovf, status);
    tm.mark("hyb_slots_kernel");
    if (o->max_ovf > 0 && h->T > 0) {
        hipLaunchKernelGGL(hyb_dense_kernel<DT>, dim3(o->max_ovf), dim3(DNT), 0, s, h->count,
                           h->col, h->val, nt, h->width, h->d_ff, o->max_ovf, o->ovf_rows,
                           o->n_ovf, o->dense, status);
        tm.mark("hyb_dense_kernel");
    }
    return hipGetLastError();
}

} // namespace

hipError_t launch_to_hybrid(const twell_t *h, const hybrid_t *o, int32_t *status,
                            twell_timing_t *timing, hipStream_t s)
{
    Timer tm(timing, s);
    return h->dtype == TWELL_BF16 ? launch<TWELL_BF16>(h, o, status, tm, s)
                                  : launch<TWELL_F32>(h, o, status, tm, s);
}
