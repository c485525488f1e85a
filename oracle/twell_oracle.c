/*
 * twell_oracle.c -- plain CPU oracle for the activation-sparse ReLU-gated FFN.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library. The HIP product path
 * never calls it, and the two share no code.
 *
 * What it computes follows "Sparser, Faster, Lighter Transformer Language
 * Models" (Cetin, Peluchetti, Castillo, Naruse, Murakami, Jones; summary page
 * gist.science/it/paper/2603.23198):
 *   - section 1 and 2.B.2: the gated FFN y = (h_g (.) x W_u) W_d;
 *   - section 2.A and 2.B.1: h_g = ReLU(x W_g), whose exact zeros are skipped;
 *   - section 2.B.1: TwELL, the column dimension cut into tiles, each tile of
 *     each row holding a nonzero count, the column indices and the values;
 *   - section 2.B.3: the hybrid layout (rows with few nonzeros in a compact
 *     ELL matrix, overflow rows in a dense backup) and the backward pass made
 *     of dense-to-sparse (sampled) and sparse-to-dense products.
 * The dothoosh.com article (MarkTechPost report) adds that the tiles match the
 * matmul kernel's tile and that ReLU replaces SiLU to give exact zeros.
 *
 * Readings where the pages are silent (each one is also stated where used):
 *   - an entry is stored iff g > 0 strictly (g == 0, -0 and NaN are not);
 *   - tile j covers columns [j*tile_c, (j+1)*tile_c); entries inside a tile are
 *     in ascending column order; at most W slots per (row, tile), the true
 *     count is kept and the first W entries are stored;
 *   - a row with at most K entries is an ELL row, otherwise the whole row goes
 *     to the dense backup; backup slots are given in ascending row order;
 *   - the backward runs on the stored pattern: an entry whose stored value is
 *     zero is inactive (ReLU'(0) = 0).
 *
 * Arithmetic: everything in float64; every sum runs in ascending index order;
 * OpenMP only splits independent output axes (tokens, neurons or model
 * columns), never a reduction, so results do not depend on the thread count.
 *
 * Storage layouts (row-major): x, dy [T][dm]; wg_t, wu_t, wd [dff][dm], where
 * row i of wg_t / wu_t is column i of W_g / W_u and row i of wd is row i of
 * W_d. TwELL: count [T][nt], col [T][nt][W], val [T][nt][W] with nt = dff /
 * tile_c. Hybrid: row_nnz [T], row_slot [T] (-1 = ELL row), ell_col/ell_val
 * [T][K], ovf_rows [max_ovf], dense [max_ovf][dff].
 */
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef int64_t i64;

static double dot(const double *a, const double *b, int n)
{
    double s = 0.0;
    for (int k = 0; k < n; ++k)
        s += a[k] * b[k];
    return s;
}

/* Gate pre-activations g = x W_g (section 2.B.1 of the summary page). */
void orc_gate(const double *x, const double *wg_t, int T, int dm, int dff, double *g)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int i = 0; i < dff; ++i)
            g[(i64)t * dff + i] = dot(x + (i64)t * dm, wg_t + (i64)i * dm, dm);
}

/*
 * TwELL encoding of h = ReLU(g) (section 2.B.1): for each row t and column
 * tile j, the ascending list of columns with g > 0, their count and values.
 * Returns 1 if some (row, tile) held more than W entries, else 0.
 */
int orc_twell_pack(const double *g, int T, int dff, int tile_c, int W,
                   int32_t *count, int32_t *col, double *val)
{
    int nt = dff / tile_c, over = 0;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < nt; ++j) {
            i64 base = ((i64)t * nt + j) * W;
            int n = 0;
            for (int c = j * tile_c; c < (j + 1) * tile_c; ++c) {
                double v = g[(i64)t * dff + c];
                if (v > 0.0) {
                    if (n < W) {
                        col[base + n] = c;
                        val[base + n] = v;
                    }
                    ++n;
                }
            }
            count[(i64)t * nt + j] = n;
            if (n > W)
                over = 1;
        }
    return over;
}

/* Dense gated FFN y = (ReLU(x W_g) (.) x W_u) W_d over every neuron (section 1). */
void orc_ffn_dense(const double *x, const double *wg_t, const double *wu_t, const double *wd,
                   int T, int dm, int dff, double *y)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const double *xt = x + (i64)t * dm;
        double *yt = y + (i64)t * dm;
        for (int k = 0; k < dm; ++k)
            yt[k] = 0.0;
        for (int i = 0; i < dff; ++i) {
            double g = dot(xt, wg_t + (i64)i * dm, dm);
            double h = g > 0.0 ? g : 0.0;
            double u = dot(xt, wu_t + (i64)i * dm, dm);
            double a = h * u;
            const double *wdi = wd + (i64)i * dm;
            for (int k = 0; k < dm; ++k)
                yt[k] += a * wdi[k];
        }
    }
}

/*
 * The same FFN restricted to the entries a TwELL holds (section 2.B.2: up and
 * down projections computed only for the nonzeros). Tiles and slots are
 * visited in ascending column order, the order of the dense sum.
 */
void orc_ffn_twell(const double *x, const int32_t *count, const int32_t *col, const double *val,
                   int T, int nt, int W, const double *wu_t, const double *wd, int dm, double *y)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const double *xt = x + (i64)t * dm;
        double *yt = y + (i64)t * dm;
        for (int k = 0; k < dm; ++k)
            yt[k] = 0.0;
        for (int j = 0; j < nt; ++j) {
            int n = count[(i64)t * nt + j];
            if (n > W)
                n = W;
            for (int s = 0; s < n; ++s) {
                i64 e = ((i64)t * nt + j) * W + s;
                int i = col[e];
                double u = dot(xt, wu_t + (i64)i * dm, dm);
                double a = val[e] * u;
                const double *wdi = wd + (i64)i * dm;
                for (int k = 0; k < dm; ++k)
                    yt[k] += a * wdi[k];
            }
        }
    }
}

/*
 * TwELL -> hybrid (section 2.B.3). row_nnz[t] = number of stored entries of
 * row t. Rows with row_nnz <= K keep their entries, concatenated in ascending
 * column order, in ELL row t. Other rows are overflow rows: they take the next
 * backup slot (ascending t); the slot's dense row holds the values at their
 * columns and zeros elsewhere. *n_ovf is the true number of overflow rows.
 * Returns 1 if that exceeds max_ovf (rows past the capacity are not stored).
 * ELL slots past row_nnz, and ELL rows of overflow rows, are left untouched.
 */
int orc_to_hybrid(const int32_t *count, const int32_t *col, const double *val,
                  int T, int nt, int W, int dff, int K, int max_ovf,
                  int32_t *row_nnz, int32_t *row_slot, int32_t *ell_col, double *ell_val,
                  int32_t *ovf_rows, double *dense, int32_t *n_ovf)
{
    int n = 0;
    for (int t = 0; t < T; ++t) {
        int nnz = 0;
        for (int j = 0; j < nt; ++j) {
            int c = count[(i64)t * nt + j];
            nnz += c > W ? W : c;
        }
        row_nnz[t] = nnz;
        if (nnz <= K) {
            row_slot[t] = -1;
            int e = 0;
            for (int j = 0; j < nt; ++j) {
                int c = count[(i64)t * nt + j];
                if (c > W)
                    c = W;
                for (int s = 0; s < c; ++s, ++e) {
                    ell_col[(i64)t * K + e] = col[((i64)t * nt + j) * W + s];
                    ell_val[(i64)t * K + e] = val[((i64)t * nt + j) * W + s];
                }
            }
        } else {
            row_slot[t] = n;
            if (n < max_ovf) {
                ovf_rows[n] = t;
                double *dr = dense + (i64)n * dff;
                for (int i = 0; i < dff; ++i)
                    dr[i] = 0.0;
                for (int j = 0; j < nt; ++j) {
                    int c = count[(i64)t * nt + j];
                    if (c > W)
                        c = W;
                    for (int s = 0; s < c; ++s) {
                        i64 e = ((i64)t * nt + j) * W + s;
                        dr[col[e]] = val[e];
                    }
                }
            }
            ++n;
        }
    }
    *n_ovf = n;
    return n > max_ovf;
}

/* Per-row entry lists (column, value) of a hybrid, ascending columns. */
typedef struct {
    i64 *off;   /* [T+1] */
    int *col;   /* [nnz] */
    double *h;  /* [nnz] */
} rows_t;

static int hybrid_rows(int T, int dff, const int32_t *row_nnz, const int32_t *row_slot,
                       const int32_t *ell_col, const double *ell_val, int K,
                       const double *dense, rows_t *r)
{
    r->off = (i64 *)malloc(sizeof(i64) * (T + 1));
    if (!r->off)
        return -1;
    r->off[0] = 0;
    for (int t = 0; t < T; ++t) {
        i64 n = 0;
        if (row_slot[t] < 0) {
            for (int s = 0; s < row_nnz[t]; ++s)
                n += ell_val[(i64)t * K + s] != 0.0;
        } else {
            const double *dr = dense + (i64)row_slot[t] * dff;
            for (int i = 0; i < dff; ++i)
                n += dr[i] != 0.0;
        }
        r->off[t + 1] = r->off[t] + n;
    }
    i64 nnz = r->off[T];
    r->col = (int *)malloc(sizeof(int) * (nnz + 1));
    r->h = (double *)malloc(sizeof(double) * (nnz + 1));
    if (!r->col || !r->h)
        return -1;
    for (int t = 0; t < T; ++t) {
        i64 e = r->off[t];
        if (row_slot[t] < 0) {
            for (int s = 0; s < row_nnz[t]; ++s) {
                double v = ell_val[(i64)t * K + s];
                if (v != 0.0) {
                    r->col[e] = ell_col[(i64)t * K + s];
                    r->h[e++] = v;
                }
            }
        } else {
            const double *dr = dense + (i64)row_slot[t] * dff;
            for (int i = 0; i < dff; ++i)
                if (dr[i] != 0.0) {
                    r->col[e] = i;
                    r->h[e++] = dr[i];
                }
        }
    }
    return 0;
}

/*
 * Forward over a hybrid (section 2.B.3: the hybrid layout serves the training
 * forward as well as the backward): y[t] = sum over the row's entries, in
 * ascending column order, of h * (x[t] . wu_t[i]) * wd[i], the row's entries
 * being its ELL entries or the nonzeros of its dense backup row. On a
 * lossless hybrid this is orc_ffn_twell's sum term for term (zero values
 * contribute exact zeros). Returns 0, or -1 if memory ran out.
 */
int orc_ffn_hybrid(const double *x, int T, int dm, int dff, const int32_t *row_nnz,
                   const int32_t *row_slot, const int32_t *ell_col, const double *ell_val, int K,
                   const double *dense, const double *wu_t, const double *wd, double *y)
{
    rows_t r;
    if (hybrid_rows(T, dff, row_nnz, row_slot, ell_col, ell_val, K, dense, &r))
        return -1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const double *xt = x + (i64)t * dm;
        double *yt = y + (i64)t * dm;
        for (int k = 0; k < dm; ++k)
            yt[k] = 0.0;
        for (i64 e = r.off[t]; e < r.off[t + 1]; ++e) {
            int i = r.col[e];
            double a = r.h[e] * dot(xt, wu_t + (i64)i * dm, dm);
            const double *wdi = wd + (i64)i * dm;
            for (int k = 0; k < dm; ++k)
                yt[k] += a * wdi[k];
        }
    }
    free(r.off);
    free(r.col);
    free(r.h);
    return 0;
}

/*
 * Backward of y = (h (.) u) W_d, u = x W_u, h = ReLU(x W_g), on the pattern
 * P of a hybrid (section 2.B.3), with ReLU' = 1 on P and 0 off it:
 *   u = x W_u and da = dy W_d^T sampled at P          (dense-to-sparse)
 *   a = h u,  du = da h,  dg = da u                    (at P)
 *   dx = du W_u^T + dg W_g^T                          (sparse-to-dense)
 *   dW_d = a^T dy,  dW_u = x^T du,  dW_g = x^T dg      (sparse^T-to-dense)
 * With an L1 activation penalty l1 * sum(h) added to the loss (the dothoosh
 * article's training recipe: an L1 term on the FFN activations to induce
 * sparsity), its gradient l1 * ReLU'(g) adds l1 to dg at every entry of P.
 * Outputs are overwritten; weight gradients are in the storage layouts
 * (dwg_t = dW_g^T, dwu_t = dW_u^T, dwd = dW_d). Overflow rows whose slot is
 * past max_ovf must not occur (the caller checks the capacity flag).
 * Returns 0, or -1 if memory ran out.
 */
int orc_bwd_hybrid(const double *x, const double *dy, int T, int dm, int dff,
                   const int32_t *row_nnz, const int32_t *row_slot,
                   const int32_t *ell_col, const double *ell_val, int K, const double *dense,
                   const double *wg_t, const double *wu_t, const double *wd, double l1,
                   double *dx, double *dwg_t, double *dwu_t, double *dwd)
{
    rows_t r;
    if (hybrid_rows(T, dff, row_nnz, row_slot, ell_col, ell_val, K, dense, &r))
        return -1;
    i64 nnz = r.off[T];
    double *ca = (double *)malloc(sizeof(double) * (nnz + 1));
    double *cdu = (double *)malloc(sizeof(double) * (nnz + 1));
    double *cdg = (double *)malloc(sizeof(double) * (nnz + 1));
    if (!ca || !cdu || !cdg)
        return -1;

    /* sampled products and the per-entry coefficients, then dx (per token);
     * su[k] and sg[k] are the two sums of dx[t][k], each over ascending i */
#pragma omp parallel
    {
        double *su = (double *)malloc(sizeof(double) * dm);
        double *sg = (double *)malloc(sizeof(double) * dm);
#pragma omp for schedule(dynamic, 16)
        for (int t = 0; t < T; ++t) {
            const double *xt = x + (i64)t * dm, *dyt = dy + (i64)t * dm;
            double *dxt = dx + (i64)t * dm;
            for (int k = 0; k < dm; ++k)
                su[k] = sg[k] = 0.0;
            for (i64 e = r.off[t]; e < r.off[t + 1]; ++e) {
                int i = r.col[e];
                double u = dot(xt, wu_t + (i64)i * dm, dm);
                double da = dot(dyt, wd + (i64)i * dm, dm);
                ca[e] = r.h[e] * u;
                cdu[e] = da * r.h[e];
                cdg[e] = da * u + l1;
                const double *wui = wu_t + (i64)i * dm, *wgi = wg_t + (i64)i * dm;
                for (int k = 0; k < dm; ++k) {
                    su[k] += cdu[e] * wui[k];
                    sg[k] += cdg[e] * wgi[k];
                }
            }
            for (int k = 0; k < dm; ++k)
                dxt[k] = su[k] + sg[k];
        }
        free(su);
        free(sg);
    }

    /* weight gradients: every dW[i][k] sums its terms in ascending t; threads
     * split the model columns k into independent blocks of 64 */
    int nkb = (dm + 63) / 64;
#pragma omp parallel for schedule(dynamic, 1)
    for (int kb = 0; kb < nkb; ++kb) {
        int k0 = kb * 64, k1 = k0 + 64 < dm ? k0 + 64 : dm;
        for (int i = 0; i < dff; ++i)
            for (int k = k0; k < k1; ++k) {
                dwd[(i64)i * dm + k] = 0.0;
                dwu_t[(i64)i * dm + k] = 0.0;
                dwg_t[(i64)i * dm + k] = 0.0;
            }
        for (int t = 0; t < T; ++t) {
            const double *xt = x + (i64)t * dm, *dyt = dy + (i64)t * dm;
            for (i64 e = r.off[t]; e < r.off[t + 1]; ++e) {
                i64 o = (i64)r.col[e] * dm;
                for (int k = k0; k < k1; ++k) {
                    dwd[o + k] += ca[e] * dyt[k];
                    dwu_t[o + k] += cdu[e] * xt[k];
                    dwg_t[o + k] += cdg[e] * xt[k];
                }
            }
        }
    }
    free(ca);
    free(cdu);
    free(cdg);
    free(r.off);
    free(r.col);
    free(r.h);
    return 0;
}

/*
 * Dense backward of the same layer over every (t, i), with ReLU'(g) = [g > 0]:
 * the plain gradient formulas of the dense layer, written without any
 * sparsity, used to check orc_bwd_hybrid on a lossless pattern. l1 is the
 * weight of the activation penalty l1 * sum(ReLU(g)) in the loss.
 */
int orc_bwd_dense(const double *x, const double *dy, int T, int dm, int dff,
                  const double *wg_t, const double *wu_t, const double *wd, double l1,
                  double *dx, double *dwg_t, double *dwu_t, double *dwd)
{
    i64 n = (i64)T * dff;
    double *a = (double *)malloc(sizeof(double) * n);
    double *du = (double *)malloc(sizeof(double) * n);
    double *dg = (double *)malloc(sizeof(double) * n);
    if (!a || !du || !dg)
        return -1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const double *xt = x + (i64)t * dm, *dyt = dy + (i64)t * dm;
        for (int i = 0; i < dff; ++i) {
            double g = dot(xt, wg_t + (i64)i * dm, dm);
            double h = g > 0.0 ? g : 0.0;
            double u = dot(xt, wu_t + (i64)i * dm, dm);
            double da = dot(dyt, wd + (i64)i * dm, dm);
            a[(i64)t * dff + i] = h * u;
            du[(i64)t * dff + i] = da * h;
            dg[(i64)t * dff + i] = g > 0.0 ? da * u + l1 : 0.0;
        }
        double *su = dx + (i64)t * dm; /* first sum, in place */
        double *sg = (double *)malloc(sizeof(double) * dm);
        for (int k = 0; k < dm; ++k)
            su[k] = sg[k] = 0.0;
        for (int i = 0; i < dff; ++i) {
            double cu = du[(i64)t * dff + i], cg = dg[(i64)t * dff + i];
            for (int k = 0; k < dm; ++k) {
                su[k] += cu * wu_t[(i64)i * dm + k];
                sg[k] += cg * wg_t[(i64)i * dm + k];
            }
        }
        for (int k = 0; k < dm; ++k)
            su[k] = su[k] + sg[k];
        free(sg);
    }
#pragma omp parallel for schedule(static)
    for (int i = 0; i < dff; ++i)
        for (int k = 0; k < dm; ++k) {
            double sd = 0.0, su = 0.0, sg = 0.0;
            for (int t = 0; t < T; ++t) {
                sd += a[(i64)t * dff + i] * dy[(i64)t * dm + k];
                su += du[(i64)t * dff + i] * x[(i64)t * dm + k];
                sg += dg[(i64)t * dff + i] * x[(i64)t * dm + k];
            }
            dwd[(i64)i * dm + k] = sd;
            dwu_t[(i64)i * dm + k] = su;
            dwg_t[(i64)i * dm + k] = sg;
        }
    free(a);
    free(du);
    free(dg);
    return 0;
}

/* Number of OpenMP threads the oracle's parallel loops run with. */
int orc_num_threads(void)
{
    return omp_get_max_threads();
}

/* Threads the parallel loops use from now on (n >= 1). Results do not depend
 * on it (no reduction is split), only the time does. */
void orc_set_num_threads(int n)
{
    omp_set_num_threads(n > 0 ? n : 1);
}
