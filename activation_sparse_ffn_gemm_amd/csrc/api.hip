// C-ABI entry points: argument validation, then launches on the caller's
// stream. Nothing here allocates, synchronises or keeps state.
#include "common.hpp"

hipError_t launch_gate_pack(twell_dtype dt, const void *x, const void *wg_t, int T, int dm,
                            const twell_t *o, void *ws, int32_t *status, twell_timing_t *timing,
                            hipStream_t s);
size_t dec_gate_workspace(int dt, int T, int dm, int dff);
hipError_t launch_ffn_fwd(twell_dtype dt, const void *x, const twell_t *h, const void *wu_t,
                          const void *wd, int dm, float *y, void *ws, int32_t *status,
                          twell_timing_t *timing, hipStream_t s);
size_t fwd_workspace(int dt, int T, int dm, int dff, int W);
hipError_t launch_to_hybrid(const twell_t *h, const hybrid_t *o, int32_t *status,
                            twell_timing_t *timing, hipStream_t s);
hipError_t launch_bwd(twell_dtype dt, const void *x, const void *dy, const hybrid_t *h,
                      const void *wg_t, const void *wu_t, const void *wd, int dm, float l1,
                      float *dx,
                      float *dwg_t, float *dwu_t, float *dwd, void *ws, int32_t *status,
                      twell_timing_t *timing, hipStream_t s);
size_t bwd_workspace_layout(int dt, int T, int dm, int dff, int K, int max_ovf);
hipError_t launch_hyb_fwd(twell_dtype dt, const void *x, const hybrid_t *h, const void *wu_t,
                          const void *wd, int dm, float *y, void *ws, int32_t *status,
                          twell_timing_t *timing, hipStream_t s);
size_t hyb_fwd_workspace(int dt, int T, int dm, int max_ovf, int dff, int K);
size_t dec_layer_workspace(int dt, int T, int dm, int dff, int W);
hipError_t launch_dec_layer(twell_dtype dt, const void *x, const void *wg_t, const void *wu_t,
                            const void *wd, int dm, const twell_t *o, float *y, void *ws,
                            int32_t *status, twell_timing_t *timing, hipStream_t s);

namespace {

bool a16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool dtype_ok(int dt) { return dt == TWELL_BF16 || dt == TWELL_F32; }

int check_dm(twell_dtype dt, int32_t dm)
{
    const int max_dm = dt == TWELL_BF16 ? 4096 : 2048;
    return (dm >= 64 && dm <= max_dm && dm % 64 == 0) ? TWELL_OK : TWELL_E_SHAPE;
}

int check_dff(int32_t dff)
{
    return (dff >= TWELL_TILE_C && dff <= 32768 && dff % TWELL_TILE_C == 0) ? TWELL_OK
                                                                              : TWELL_E_SHAPE;
}

// dtype, token count, d_model and d_ff within the documented limits
bool sizes_ok(int dt, int32_t T, int32_t dm, int32_t dff)
{
    return dtype_ok(dt) && T >= 0 && T <= TWELL_MAX_ROWS && !check_dm((twell_dtype)dt, dm) &&
           !check_dff(dff);
}

// a hybrid's K and backup capacity for T rows of d_ff columns; ELL slots are
// numbered t * K + s in 32-bit integers (the backward's transpose)
bool hybrid_sizes_ok(int32_t T, int32_t dff, int32_t K, int32_t max_ovf)
{
    return K >= 1 && K <= dff && K <= 32767 && max_ovf >= 0 && max_ovf <= TWELL_MAX_ROWS &&
           (int64_t)T * K <= INT32_MAX;
}

int check_twell(const twell_t *h, twell_dtype dt)
{
    if (!h)
        return TWELL_E_NULL;
    if (!dtype_ok(h->dtype) || h->dtype != dt)
        return TWELL_E_DTYPE;
    if (h->T < 0 || h->T > TWELL_MAX_ROWS || h->width < 1 || h->width > TWELL_TILE_C)
        return TWELL_E_SHAPE;
    if (int rc = check_dff(h->d_ff))
        return rc;
    if (h->T > 0 && (!h->count || !h->col || !h->val))
        return TWELL_E_NULL;
    return TWELL_OK;
}

int check_hybrid(const hybrid_t *h, twell_dtype dt)
{
    if (!h)
        return TWELL_E_NULL;
    if (!dtype_ok(h->dtype) || h->dtype != dt)
        return TWELL_E_DTYPE;
    if (h->T < 0 || h->T > TWELL_MAX_ROWS || !hybrid_sizes_ok(h->T, h->d_ff, h->K, h->max_ovf))
        return TWELL_E_SHAPE;
    if (int rc = check_dff(h->d_ff))
        return rc;
    if (!h->n_ovf)
        return TWELL_E_NULL;
    if (h->T > 0 && (!h->row_nnz || !h->row_slot || !h->ell_col || !h->ell_val))
        return TWELL_E_NULL;
    if (h->max_ovf > 0 && (!h->ovf_rows || !h->dense))
        return TWELL_E_NULL;
    return TWELL_OK;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? TWELL_OK : TWELL_E_HIP; }

} // namespace

// Every argument check of twell_decode_fwd except the workspace's (shared
// with twell_decode_fwd_noalloc, whose scratch is the library's own).
int check_decode_args(twell_dtype dt, const void *x, const void *wg_t, const void *wu_t,
                      const void *wd, int32_t d_model, const twell_t *out, const float *y)
{
    if (!dtype_ok(dt))
        return TWELL_E_DTYPE;
    if (!wg_t || !wu_t || !wd || !out)
        return TWELL_E_NULL;
    if (int rc = check_twell(out, dt))
        return rc;
    if (out->T > 0 && (!x || !y))
        return TWELL_E_NULL;
    if (int rc = check_dm(dt, d_model))
        return rc;
    if (out->T > TWELL_DECODE_T)
        return TWELL_E_SHAPE;
    if (!a16(x) || !a16(wg_t) || !a16(wu_t) || !a16(wd) || !a16(y))
        return TWELL_E_ALIGN;
    return TWELL_OK;
}

extern "C" {

const char *twell_status_str(int code)
{
    switch (code) {
    case TWELL_OK: return "ok";
    case TWELL_E_NULL: return "a required pointer is NULL";
    case TWELL_E_SHAPE: return "a size is out of range or inconsistent";
    case TWELL_E_DTYPE: return "unsupported or mismatched element type";
    case TWELL_E_ALIGN: return "a pointer is not 16-byte aligned";
    case TWELL_E_WORKSPACE: return "workspace too small";
    case TWELL_E_HIP: return "HIP launch failed";
    case TWELL_E_SCRATCH: return "the call needs more scratch than the static buffer holds";
    default: return "unknown status";
    }
}

size_t twell_gate_workspace_bytes(twell_dtype dt, int32_t T, int32_t d_model, int32_t d_ff)
{
    if (!sizes_ok(dt, T, d_model, d_ff))
        return 0;
    return T <= TWELL_DECODE_T ? dec_gate_workspace(dt, T, d_model, d_ff) : 0;
}

int twell_gate_pack(twell_dtype dt, const void *x, const void *wg_t, int32_t T, int32_t d_model,
                    const twell_t *out, void *workspace, size_t workspace_bytes,
                    int32_t *dev_status, twell_timing_t *timing, void *stream)
{
    if (!dtype_ok(dt))
        return TWELL_E_DTYPE;
    if ((!x && T != 0) || !wg_t || !out)
        return TWELL_E_NULL;
    if (int rc = check_twell(out, dt))
        return rc;
    if (int rc = check_dm(dt, d_model))
        return rc;
    if (T < 0 || T > TWELL_MAX_ROWS || out->T != T)
        return TWELL_E_SHAPE;
    if (!a16(x) || !a16(wg_t))
        return TWELL_E_ALIGN;
    const size_t need = twell_gate_workspace_bytes(dt, T, d_model, out->d_ff);
    if (workspace_bytes < need || (need && !workspace))
        return TWELL_E_WORKSPACE;
    if (!a16(workspace))
        return TWELL_E_ALIGN;
    if (T == 0)
        return TWELL_OK;
    return hip_rc(launch_gate_pack(dt, x, wg_t, T, d_model, out, workspace, dev_status, timing,
                                   (hipStream_t)stream));
}

size_t twell_fwd_workspace_bytes(twell_dtype dt, int32_t T, int32_t d_model, int32_t d_ff,
                                 int32_t width)
{
    if (!sizes_ok(dt, T, d_model, d_ff) || width < 1 || width > TWELL_TILE_C)
        return 0;
    return fwd_workspace(dt, T, d_model, d_ff, width);
}

int twell_ffn_fwd(twell_dtype dt, const void *x, const twell_t *h, const void *wu_t,
                  const void *wd, int32_t d_model, float *y, void *workspace,
                  size_t workspace_bytes, int32_t *dev_status, twell_timing_t *timing,
                  void *stream)
{
    if (!dtype_ok(dt))
        return TWELL_E_DTYPE;
    if (!h || !wu_t || !wd)
        return TWELL_E_NULL;
    if (int rc = check_twell(h, dt))
        return rc;
    if (h->T > 0 && (!x || !y))
        return TWELL_E_NULL;
    if (int rc = check_dm(dt, d_model))
        return rc;
    if (!a16(x) || !a16(wu_t) || !a16(wd) || !a16(y))
        return TWELL_E_ALIGN;
    const size_t need = twell_fwd_workspace_bytes(dt, h->T, d_model, h->d_ff, h->width);
    if (workspace_bytes < need || (need && !workspace))
        return TWELL_E_WORKSPACE;
    if (!a16(workspace))
        return TWELL_E_ALIGN;
    if (h->T == 0)
        return TWELL_OK;
    return hip_rc(launch_ffn_fwd(dt, x, h, wu_t, wd, d_model, y, workspace, dev_status, timing,
                                 (hipStream_t)stream));
}

size_t twell_decode_workspace_bytes(twell_dtype dt, int32_t T, int32_t d_model, int32_t d_ff,
                                    int32_t width)
{
    if (!sizes_ok(dt, T, d_model, d_ff) || T > TWELL_DECODE_T || width < 1 ||
        width > TWELL_TILE_C)
        return 0;
    return dec_layer_workspace(dt, T, d_model, d_ff, width);
}

int twell_decode_fwd(twell_dtype dt, const void *x, const void *wg_t, const void *wu_t,
                     const void *wd, int32_t d_model, const twell_t *out, float *y,
                     void *workspace, size_t workspace_bytes, int32_t *dev_status,
                     twell_timing_t *timing, void *stream)
{
    if (int rc = check_decode_args(dt, x, wg_t, wu_t, wd, d_model, out, y))
        return rc;
    const size_t need =
        twell_decode_workspace_bytes(dt, out->T, d_model, out->d_ff, out->width);
    if (workspace_bytes < need || (need && !workspace))
        return TWELL_E_WORKSPACE;
    if (!a16(workspace))
        return TWELL_E_ALIGN;
    if (out->T == 0)
        return TWELL_OK;
    return hip_rc(launch_dec_layer(dt, x, wg_t, wu_t, wd, d_model, out, y, workspace,
                                   dev_status, timing, (hipStream_t)stream));
}

int twell_to_hybrid(const twell_t *h, const hybrid_t *out, int32_t *dev_status,
                    twell_timing_t *timing, void *stream)
{
    if (!h || !out)
        return TWELL_E_NULL;
    if (!dtype_ok(h->dtype))
        return TWELL_E_DTYPE;
    if (int rc = check_twell(h, h->dtype))
        return rc;
    if (int rc = check_hybrid(out, h->dtype))
        return rc;
    if (out->T != h->T || out->d_ff != h->d_ff)
        return TWELL_E_SHAPE;
    return hip_rc(launch_to_hybrid(h, out, dev_status, timing, (hipStream_t)stream));
}

size_t hybrid_fwd_workspace_bytes(twell_dtype dt, int32_t T, int32_t d_model, int32_t d_ff,
                                  int32_t K, int32_t max_ovf)
{
    if (!sizes_ok(dt, T, d_model, d_ff) || !hybrid_sizes_ok(T, d_ff, K, max_ovf))
        return 0;
    return hyb_fwd_workspace(dt, T, d_model, max_ovf, d_ff, K);
}

int hybrid_ffn_fwd(twell_dtype dt, const void *x, const hybrid_t *h, const void *wu_t,
                   const void *wd, int32_t d_model, float *y, void *workspace,
                   size_t workspace_bytes, int32_t *dev_status, twell_timing_t *timing,
                   void *stream)
{
    if (!dtype_ok(dt))
        return TWELL_E_DTYPE;
    if (!h || !wu_t || !wd)
        return TWELL_E_NULL;
    if (int rc = check_hybrid(h, dt))
        return rc;
    if (h->T > 0 && (!x || !y))
        return TWELL_E_NULL;
    if (int rc = check_dm(dt, d_model))
        return rc;
    if (!a16(x) || !a16(wu_t) || !a16(wd) || !a16(y) || !a16(workspace))
        return TWELL_E_ALIGN;
    const size_t need = hybrid_fwd_workspace_bytes(dt, h->T, d_model, h->d_ff, h->K, h->max_ovf);
    if (workspace_bytes < need || (need && !workspace))
        return TWELL_E_WORKSPACE;
    if (h->T == 0)
        return TWELL_OK;
    return hip_rc(launch_hyb_fwd(dt, x, h, wu_t, wd, d_model, y, workspace, dev_status, timing,
                                 (hipStream_t)stream));
}

size_t hybrid_bwd_workspace_bytes(twell_dtype dt, int32_t T, int32_t d_model, int32_t d_ff,
                                  int32_t K, int32_t max_ovf)
{
    if (!sizes_ok(dt, T, d_model, d_ff) || !hybrid_sizes_ok(T, d_ff, K, max_ovf))
        return 0;
    return bwd_workspace_layout(dt, T, d_model, d_ff, K, max_ovf);
}

int hybrid_ffn_bwd(twell_dtype dt, const void *x, const void *dy, const hybrid_t *h,
                   const void *wg_t, const void *wu_t, const void *wd, int32_t d_model,
                   float l1, float *dx, float *dwg_t, float *dwu_t, float *dwd, void *workspace,
                   size_t workspace_bytes, int32_t *dev_status, twell_timing_t *timing,
                   void *stream)
{
    if (!dtype_ok(dt))
        return TWELL_E_DTYPE;
    if (!h || !wg_t || !wu_t || !wd || !dwg_t || !dwu_t || !dwd)
        return TWELL_E_NULL;
    if (int rc = check_hybrid(h, dt))
        return rc;
    if (h->T > 0 && (!x || !dy || !dx))
        return TWELL_E_NULL;
    if (int rc = check_dm(dt, d_model))
        return rc;
    if (!a16(x) || !a16(dy) || !a16(wg_t) || !a16(wu_t) || !a16(wd) || !a16(dx) || !a16(dwg_t) ||
        !a16(dwu_t) || !a16(dwd) || !a16(workspace))
        return TWELL_E_ALIGN;
    const size_t need = hybrid_bwd_workspace_bytes(dt, h->T, d_model, h->d_ff, h->K, h->max_ovf);
    if (workspace_bytes < need || (need && !workspace))
        return TWELL_E_WORKSPACE;
    if (!(l1 == l1) || l1 > 3.4e38f || l1 < -3.4e38f) // NaN or infinite
        return TWELL_E_SHAPE;
    return hip_rc(launch_bwd(dt, x, dy, h, wg_t, wu_t, wd, d_model, l1, dx, dwg_t, dwu_t, dwd,
                             workspace, dev_status, timing, (hipStream_t)stream));
}

} // extern "C"
