// Dense products over the hybrid's backup rows ("Sparser, Faster, Lighter
// Transformer Language Models", summary page section 2.B.3: rows with many
// nonzeros go to a dense backup, whose products run densely).
//
// O = the backup rows (n_ovf of them, ovf_rows[m] their token rows), h_O
// their stored h (the backup's dense array), x_O / dy_O their x / dy rows.
// Forward:
//   A = h_O (.) (x_O W_u)                        [n_ovf x d_ff]
//   y_O = A W_d                                  [n_ovf x d_model]
// Backward, with u = x_O W_u and da = dy_O W_d^T:
//   a = h_O u,  du = da h_O,  dg = da u + l1 where h_O != 0, else 0
//   dx_O = du W_u^T + dg W_g^T
//   dW_d = a^T dy_O,  dW_u = du^T x_O,  dW_g = dg^T x_O  (the ELL rows' share
//   is added by the neuron pass that runs after them)
//
// Every operand is read as it is stored. Products over K-contiguous rows
// (u = x_O W_u and da = dy_O W_d^T: x, dy, wu_t and wd rows all run along
// d_model) take the shared main loop; the others take its mixed-layout form
// (ntgemm.hpp), which reads an operand stored with the contraction index as
// its row index straight from that layout through gfx950's transposing LDS
// reads: W_d in y_O = A W_d, W_u and W_g in dx_O, and both operands of the
// dW products (a, du, dg as [rows][d_ff], and x_O, dy_O as [rows][d_model],
// the latter gathered once by extra workgroups of the ELL masks launch). No
// transposed copy of any weight or activation is made. For bf16 inputs a
// float32 intermediate v is stored as two bf16, hi = bf16(v) and
// lo = bf16(v - hi), and a product over it runs over both halves (about 16
// significant bits); float32 inputs keep one float32 array.
//
// y_O and dx_O have few rows and a long K (d_ff, or 2-4 segments of it): K is
// split over S workgroups per tile, each writing a float32 partial. A backup
// row's S partials are added in split order, starting from zero, by the ELL
// row kernels that run next (they skip backup rows otherwise; see BkPart), or
// for the large layers' y_O by a third forward launch (bk_out).
// Row counts are device values: workgroups whose rows all lie past n_ovf
// return at once, and the grids are sized for the capacity max_ovf. The
// backward's products run as extra workgroups of the ELL passes' launches
// (the u/da tiles with the block scans, the dx_O and dW tiles with the CSC
// fill; bwd.hip), so that a layer without backup rows pays no launch for them;
// the forward's have launches of their own (this file), on a second stream
// beside the ELL passes for the large layers (hyb_fwd.hip).
#include "backup_tiles.hpp"

using namespace bk;

namespace {

constexpr int WT = 256; // backup rows are padded to whole 256-row blocks

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }
int pad_rows(int max_ovf) { return (max_ovf + WT - 1) / WT * WT; }

// K split of the y_O / dx_O products: few row tiles give one workgroup per
// CU far too little to overlap; aim at `target` workgroups over the
// capacity's tiles (tiles wholly past n_ovf return at once), at most 16
// splits, at least 16 K steps each. The callers aim at 1024: at the 1.5B
// skewed layer (1024 rows of capacity, 410 used) that is 8 splits, which ran
// faster than 16 (and 4) and halves the float32 partials.
int split_k(int R, int dm, int nk, int tile = WT, int target = 512)
{
    const int tiles = (R / tile) * ((dm + tile - 1) / tile);
    int S = std::max(1, target / std::max(tiles, 1));
    S = std::min(S, 16);
    S = std::min(S, std::max(1, nk / 16));
    return S;
}

// ---------------------------------------------------------------- kernels
template <int DT>
__global__ __launch_bounds__(UD_NT, 1) void bk_a_kernel(
    const uint8_t *__restrict__ x, const int32_t *__restrict__ ovf_rows,
    const int32_t *__restrict__ n_ovf_p, int max_ovf, const uint8_t *__restrict__ wu, int dm,
    int dff, int R, const void *__restrict__ dense, void *__restrict__ inter)
{
    __shared__ __attribute__((aligned(16))) uint8_t L[ud_lds<DT>()];
    const int n = n_rows(n_ovf_p, max_ovf);
    if (n <= 0)
        return;
    const int b = blockIdx.x, nx = dff / TILE;
    ud_tile<DT, false>(x, nullptr, ovf_rows, n, wu, nullptr, dm, dff, R, dense, 0.f, inter,
                       b % nx, b / nx, L);
}

template <int DT, int NH>
__global__ __launch_bounds__(CY::NT, 2) void bk_y_kernel(
    const uint8_t *__restrict__ a, const uint8_t *__restrict__ wd,
    const int32_t *__restrict__ n_ovf_p, int max_ovf, int dm, int dff, int R, int S,
    float *__restrict__ part)
{
    __shared__ __attribute__((aligned(16))) uint8_t L[CY::LDS];
    rowsw_tile<CY, DT, NH, 4>(a, wd, wd, n_rows(n_ovf_p, max_ovf), dm, dff, R, S, part,
                              blockIdx.x, blockIdx.y, blockIdx.z, L);
}

// y rows of the backup rows: y[ovf_rows[m]] = sum over s = 0 .. S-1, in that
// order from zero, of part[s][m] (float32 [S][R][d_model]). One wave per row,
// four floats per lane (d_model is a multiple of 64), eight splits in flight.
constexpr int OUT_NT = 256;
__global__ __launch_bounds__(OUT_NT) void bk_out_kernel(
    const float *__restrict__ part, const int32_t *__restrict__ ovf_rows,
    const int32_t *__restrict__ n_ovf_p, int max_ovf, int R, int S, int dm,
    float *__restrict__ y)
{
    const int m = blockIdx.x * (OUT_NT / 64) + wave_id();
    if (m >= n_rows(n_ovf_p, max_ovf))
        return;
    const int lane = threadIdx.x & 63;
    const size_t stride = (size_t)R * dm;
    const float *src = part + (size_t)m * dm;
    float *dst = y + (size_t)ovf_rows[m] * dm;
    for (int c = lane * 4; c < dm; c += 256) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s0 = 0; s0 < S; s0 += 8) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = *(const float4 *)(src + (size_t)min(s0 + u, S - 1) * stride + c);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < S) {
                    acc.x += v[u].x;
                    acc.y += v[u].y;
                    acc.z += v[u].z;
                    acc.w += v[u].w;
                }
        }
        *(float4 *)(dst + c) = acc;
    }
}

} // namespace

// ---------------------------------------------------------------- host side
struct BkLayout {
    size_t inter, xo, part, total;
    int R, S;
};

// Workspace of the backup products, bytes from `base`:
//   inter   fwd: A (hi, lo) [NH][R][dff]; bwd: a, du, dg (hi, lo each) [3][NH][R][dff]
//   xo      bwd only: x_O, dy_O gathered, [2][R][dm]
//   part    [S][R][dm] float32 partials of y_O / dx_O
BkLayout bk_layout(int dt, int dm, int dff, int max_ovf, bool bwd)
{
    BkLayout L{};
    const size_t esz = dt == TWELL_BF16 ? 2 : 4, nh = dt == TWELL_BF16 ? 2 : 1;
    L.R = pad_rows(max_ovf);
    const int nseg = (int)(bwd ? 2 * nh : nh);
    L.S = bwd ? split_k(L.R, dm, nseg * (int)(dff * esz / DX::ROWB), DX::BM, 1024)
              : split_k(L.R, dm, nseg * (int)(dff * esz / CY::ROWB), CY::BM, 1024);
    size_t o = 0;
    L.inter = o; o += up256((bwd ? 3 : 1) * nh * L.R * dff * esz);
    L.xo = o;    o += bwd ? up256(2 * (size_t)L.R * dm * esz) : 0;
    L.part = o;  o += up256((size_t)L.S * L.R * dm * 4);
    L.total = max_ovf > 0 ? o : 0;
    return L;
}

template <int DT>
void bk_fwd_dt(const void *x, const hybrid_t *h, const void *wu, const void *wd, int dm, float *y,
               uint8_t *ws, bool out_rows, Timer &tm, hipStream_t s)
{
    const int dff = h->d_ff;
    const BkLayout L = bk_layout(DT, dm, dff, h->max_ovf, false);
    const int n_a = (dff / TILE) * (L.R / TILE);
    hipLaunchKernelGGL((bk_a_kernel<DT>), dim3(n_a), dim3(UD_NT), 0, s, (const uint8_t *)x,
                       h->ovf_rows, h->n_ovf, h->max_ovf, (const uint8_t *)wu, dm, dff, L.R,
                       h->dense, (void *)(ws + L.inter));
    tm.mark("bk_a_kernel");
    constexpr int NH = DT == TWELL_BF16 ? 2 : 1;
    hipLaunchKernelGGL((bk_y_kernel<DT, NH>), dim3((dm + CY::BN - 1) / CY::BN, L.R / CY::BM, L.S),
                       dim3(CY::NT), 0, s, (const uint8_t *)(ws + L.inter),
                       (const uint8_t *)wd, h->n_ovf, h->max_ovf, dm, dff, L.R, L.S,
                       (float *)(ws + L.part));
    tm.mark("bk_y_kernel");
    if (!out_rows)
        return;
    hipLaunchKernelGGL(bk_out_kernel, dim3(L.R / (OUT_NT / 64)), dim3(OUT_NT), 0, s,
                       (const float *)(ws + L.part), h->ovf_rows, h->n_ovf, h->max_ovf, L.R, L.S,
                       dm, y);
    tm.mark("bk_out_kernel");
}

BkPart bk_part(int dt, int dm, int dff, int max_ovf, bool bwd, const void *ws)
{
    const BkLayout L = bk_layout(dt, dm, dff, max_ovf, bwd);
    if (max_ovf <= 0)
        return BkPart{nullptr, 0, 0};
    return BkPart{(const float *)((const uint8_t *)ws + L.part), L.S, L.R};
}

size_t bk_workspace(int dt, int dm, int dff, int max_ovf, bool bwd)
{
    return bk_layout(dt, dm, dff, max_ovf, bwd).total;
}

BkBwd bk_bwd(int dt, int dm, int dff, int max_ovf, void *ws)
{
    if (max_ovf <= 0)
        return BkBwd{};
    const BkLayout L = bk_layout(dt, dm, dff, max_ovf, true);
    uint8_t *w = (uint8_t *)ws;
    const int nd = (dm + DX::BN - 1) / DX::BN;
    return BkBwd{w + L.inter, w + L.xo, (float *)(w + L.part), L.R, L.S,
                 (dff / TILE) * (L.R / TILE), nd * (L.R / DX::BM) * L.S,
                 nd * ((dff + DX::BM - 1) / DX::BM) * 3};
}

BkGather bk_gather(int dt, int dm, int dff, int max_ovf, void *ws)
{
    if (max_ovf <= 0)
        return BkGather{nullptr, 0, 0};
    const BkLayout L = bk_layout(dt, dm, dff, max_ovf, true);
    return BkGather{(uint8_t *)ws + L.xo, L.R, bk_gather_blocks(L.R)};
}

void launch_bk_fwd(twell_dtype dt, const void *x, const hybrid_t *h, const void *wu,
                   const void *wd, int dm, float *y, void *ws, bool out_rows, Timer &tm,
                   hipStream_t s)
{
    if (h->max_ovf <= 0 || h->T <= 0)
        return;
    if (dt == TWELL_BF16)
        bk_fwd_dt<TWELL_BF16>(x, h, wu, wd, dm, y, (uint8_t *)ws, out_rows, tm, s);
    else
        bk_fwd_dt<TWELL_F32>(x, h, wu, wd, dm, y, (uint8_t *)ws, out_rows, tm, s);
}
