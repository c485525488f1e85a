// TwELL -> hybrid ELL + dense backup ("Sparser, Faster, Lighter Transformer
// Language Models", summary page section 2.B.3: training sparsity is uneven,
// so rows with few nonzeros go to a compact ELL matrix and overflow rows are
// redirected to a dense backup, through a dedicated conversion kernel).
//
// Two launches, all integer / copy work:
//   1. rows:   one wave per row sums the tile counts (row_nnz) and, for a row
//              with row_nnz <= K, concatenates its tiles into ELL row t; the
//              tiles are in column order, so the ELL row is ascending.
//   2. backup: R workgroups per block of 256 rows. Each scans its block's
//              flags; the first of the R, and those with a backup row to
//              build, then count the overflow rows of the blocks before their
//              own (a reduction over row_nnz), so backup slots follow
//              ascending row order. The first writes row_slot and ovf_rows
//              (and, in the last block, n_ovf), and workgroup j builds the
//              block's backup rows j, j + R, ... (zeros, then the row's
//              entries) in LDS and stores them with 16-byte lanes. Slots and dense rows
//              share the launch, so backup rows cost no launch of their own.
#include <algorithm>

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

constexpr int SNT = 256;       // threads (and rows) per workgroup of the backup launch
constexpr int ROW_LDS = 32768; // bytes of one dense row built in LDS (d_ff 16384 bf16 / 8192 f32)
constexpr int RMAX = 32;       // workgroups per block of rows (backup rows built in parallel)

// Backup row `slot` from TwELL row t, by the whole workgroup: zeros, then
// every stored entry of the row's tiles (loads unconditional, 8 per thread at
// a time; stores of stored slots only), in LDS and then to memory with
// 16-byte lanes (rows wider than the LDS buffer are built in memory).
template <int DT>
DEVI void build_dense_row(const int32_t *__restrict__ count, const int16_t *__restrict__ col,
                          const void *__restrict__ val, int nt, int W, int dff, int t, int slot,
                          void *__restrict__ dense, int32_t *__restrict__ status,
                          uint8_t *rowbuf)
{
    using S = typename elem<DT>::storage;
    const int tid = threadIdx.x;
    S *drow = (S *)dense + (size_t)slot * dff;
    const bool in_lds = (size_t)dff * sizeof(S) <= ROW_LDS;
    S *brow = in_lds ? (S *)rowbuf : drow;
    if (in_lds)
        for (int i = tid; i < dff * (int)sizeof(S) / 16; i += SNT)
            ((uint4 *)rowbuf)[i] = make_uint4(0, 0, 0, 0);
    else
        for (int i = tid; i < dff; i += SNT)
            drow[i] = S(0);
    __syncthreads();
    const size_t src = (size_t)t * nt * W;
    const int nslot = nt * W;
    for (int q0 = 0; q0 < nslot; q0 += 8 * SNT) {
        int c[8], n[8];
        S v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int q = min(q0 + u * SNT + tid, nslot - 1);
            n[u] = count[(size_t)t * nt + q / W];
            c[u] = col[src + q];
            v[u] = ((const S *)val)[src + q];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int q = q0 + u * SNT + tid;
            if (q < nslot && q % W < min(n[u], W)) {
                if (c[u] >= 0 && c[u] < dff)
                    brow[c[u]] = v[u];
                else
                    raise_status(status, TWELL_DEV_BAD_INDEX);
            }
        }
    }
    __syncthreads();
    if (in_lds)
        for (int i = tid; i < dff * (int)sizeof(S) / 16; i += SNT)
            ((uint4 *)drow)[i] = ((const uint4 *)rowbuf)[i];
    __syncthreads(); // the buffer is rebuilt by the workgroup's next row
}

template <int DT>
__global__ __launch_bounds__(SNT) void hyb_backup_kernel(
    const int32_t *__restrict__ row_nnz, int T, int K, int max_ovf, int R,
    int32_t *__restrict__ row_slot, int32_t *__restrict__ ovf_rows, int32_t *__restrict__ n_ovf,
    const int32_t *__restrict__ count, const int16_t *__restrict__ col,
    const void *__restrict__ val, int nt, int W, int dff, void *__restrict__ dense,
    int32_t *__restrict__ status)
{
    __shared__ __attribute__((aligned(16))) uint8_t rowbuf[ROW_LDS];
    __shared__ int wsum[SNT / 64];
    __shared__ int n_before;
    __shared__ int brows[SNT]; // the block's backup rows, by slot - first slot of the block
    const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
    const int blk = blockIdx.x / R, j = blockIdx.x % R;
    const int r0 = blk * SNT;
    // this block: one flag per thread, ranks by a block scan (ballots per
    // wave, wave totals in LDS)
    const int t = r0 + tid;
    const bool f = t < T && row_nnz[t] > K;
    const unsigned long long m = __ballot(f);
    if (lane == 0)
        wsum[wv] = __popcll(m);
    if (tid == 0)
        n_before = 0;
    __syncthreads();
    int nb = 0, in_blk = 0; // backup rows of this block; of the waves before this one
    for (int w = 0; w < SNT / 64; ++w) {
        in_blk += w < wv ? wsum[w] : 0;
        nb += wsum[w];
    }
    if (j != 0 && j >= nb) // uniform: no row to build and not the block's first workgroup
        return;
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
    const int rank = in_blk + __popcll(m & ((1ull << lane) - 1ull)); // within the block
    if (f)
        brows[rank] = t;
    __syncthreads(); // n_before and brows complete
    const int first = n_before;
    const int slot = first + rank;
    if (j == 0) {
        if (t < T) {
            row_slot[t] = f ? slot : -1;
            if (f && slot < max_ovf)
                ovf_rows[slot] = t;
        }
        if (tid == SNT - 1 && r0 + SNT >= T) { // last block: the true total
            const int total = first + nb;
            *n_ovf = total;
            if (total > max_ovf)
                raise_status(status, TWELL_DEV_OVF_CAPACITY);
        }
    }
    for (int k = j; k < nb && first + k < max_ovf; k += R)
        build_dense_row<DT>(count, col, val, nt, W, dff, brows[k], first + k, dense, status,
                            rowbuf);
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
    // R workgroups per block of rows, for about one backup row each at the
    // capacity: the capacity's rows spread over the blocks, at most RMAX
    const int nblk = h->T > 0 ? (h->T + SNT - 1) / SNT : 1;
    const int R = std::max(1, std::min(RMAX, (o->max_ovf + nblk - 1) / nblk));
    hipLaunchKernelGGL((hyb_backup_kernel<DT>), dim3(nblk * R), dim3(SNT), 0, s, o->row_nnz,
                       h->T, o->K, o->max_ovf, R, o->row_slot, o->ovf_rows, o->n_ovf, h->count,
                       h->col, h->val, nt, h->width, h->d_ff, o->dense, status);
    tm.mark("hyb_backup_kernel");
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
