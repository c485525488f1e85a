// TwELL -> hybrid ELL + dense backup ("Sparser, Faster, Lighter Transformer
// Language Models", summary page section 2.B.3: training sparsity is uneven,
// so rows with few nonzeros go to a compact ELL matrix and overflow rows are
// redirected to a dense backup, through a dedicated conversion kernel).
//
// Three launches, all integer / copy work:
//   1. rows:  one wave per row sums the tile counts (row_nnz) and, for a row
//             with row_nnz <= K, concatenates its tiles into ELL row t; the
//             tiles are in column order, so the ELL row is ascending.
//   2. slots: one workgroup scans the overflow flags in row order, giving
//             backup slots in ascending row order, ovf_rows and n_ovf.
//   3. dense: one workgroup per used backup slot zero-fills the dense row
//             and scatters the row's values into it.
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
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T)
        return;
    int total = 0;
    for (int j0 = 0; j0 < nt; j0 += 64) {
        const int j = j0 + lane;
        const int n = j < nt ? min(count[(size_t)t * nt + j], W) : 0;
        total += __shfl(wave_incl_scan(n, lane), 63, 64);
    }
    if (lane == 0)
        row_nnz[t] = total;
    if (total > K)
        return; // overflow row: handled by the dense launch
    int base = 0;
    for (int j0 = 0; j0 < nt; j0 += 64) {
        const int j = j0 + lane;
        const int n = j < nt ? min(count[(size_t)t * nt + j], W) : 0;
        const int incl = wave_incl_scan(n, lane);
        const int excl = base + incl - n;
        const size_t src = ((size_t)t * nt + j) * W;
        const size_t dst = (size_t)t * K + excl;
        for (int s = 0; s < n; ++s) {
            ell_col[dst + s] = col[src + s];
            ((S *)ell_val)[dst + s] = ((const S *)val)[src + s];
        }
        base += __shfl(incl, 63, 64);
    }
}

constexpr int SCAN_NT = 1024;

__global__ __launch_bounds__(SCAN_NT) void hyb_slots_kernel(
    const int32_t *__restrict__ row_nnz, int T, int K, int max_ovf, int32_t *__restrict__ row_slot,
    int32_t *__restrict__ ovf_rows, int32_t *__restrict__ n_ovf, int32_t *__restrict__ status)
{
    __shared__ int wsum[SCAN_NT / 64];
    __shared__ int carry;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (tid == 0)
        carry = 0;
    __syncthreads();
    for (int t0 = 0; t0 < T; t0 += SCAN_NT) {
        const int t = t0 + tid;
        const int f = (t < T && row_nnz[t] > K) ? 1 : 0;
        const int incl = wave_incl_scan(f, lane);
        if (lane == 63)
            wsum[wv] = incl;
        __syncthreads();
        int before = carry;
        for (int w = 0; w < wv; ++w)
            before += wsum[w];
        const int slot = before + incl - f;
        if (t < T) {
            row_slot[t] = f ? slot : -1;
            if (f && slot < max_ovf)
                ovf_rows[slot] = t;
        }
        __syncthreads();
        if (tid == SCAN_NT - 1)
            carry = slot + f;
        __syncthreads();
    }
    if (tid == 0) {
        *n_ovf = carry;
        if (carry > max_ovf)
            raise_status(status, TWELL_DEV_OVF_CAPACITY);
    }
}

template <int DT>
__global__ __launch_bounds__(256) void hyb_dense_kernel(
    const int32_t *__restrict__ count, const int16_t *__restrict__ col,
    const void *__restrict__ val, int nt, int W, int dff, int max_ovf,
    const int32_t *__restrict__ ovf_rows, const int32_t *__restrict__ n_ovf,
    void *__restrict__ dense, int32_t *__restrict__ status)
{
    using S = typename elem<DT>::storage;
    const int slot = blockIdx.x;
    if (slot >= min(*n_ovf, max_ovf))
        return;
    const int t = ovf_rows[slot];
    S *drow = (S *)dense + (size_t)slot * dff;
    for (int i = threadIdx.x; i < dff; i += blockDim.x)
        drow[i] = S(0);
    __syncthreads();
    for (int j = threadIdx.x; j < nt; j += blockDim.x) {
        const int n = min(count[(size_t)t * nt + j], W);
        const size_t src = ((size_t)t * nt + j) * W;
        for (int s = 0; s < n; ++s) {
            const int c = col[src + s];
            if (c >= 0 && c < dff)
                drow[c] = ((const S *)val)[src + s];
            else
                raise_status(status, TWELL_DEV_BAD_INDEX);
        }
    }
}

template <int DT>
hipError_t launch(const twell_t *h, const hybrid_t *o, int32_t *status, Timer &tm, hipStream_t s)
{
    const int nt = h->d_ff / TWELL_TILE_C;
    if (h->T > 0)
        hipLaunchKernelGGL(hyb_rows_kernel<DT>, dim3((h->T + 3) / 4), dim3(256), 0, s, h->count,
                           h->col, h->val, h->T, nt, h->width, o->K, o->row_nnz, o->ell_col,
                           o->ell_val);
    tm.mark("hyb_rows_kernel");
    hipLaunchKernelGGL(hyb_slots_kernel, dim3(1), dim3(SCAN_NT), 0, s, o->row_nnz, h->T, o->K,
                       o->max_ovf, o->row_slot, o->ovf_rows, o->n_ovf, status);
    tm.mark("hyb_slots_kernel");
    const int nslots = min(o->max_ovf, h->T);
    if (nslots > 0)
        hipLaunchKernelGGL(hyb_dense_kernel<DT>, dim3(nslots), dim3(256), 0, s, h->count, h->col,
                           h->val, nt, h->width, h->d_ff, o->max_ovf, o->ovf_rows, o->n_ovf,
                           o->dense, status);
    tm.mark("hyb_dense_kernel");
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
