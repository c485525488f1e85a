/*
 * twell.h -- C-ABI of the activation-sparse ReLU-gated FFN on MI355X (gfx950).
 *
 * The layer is y = (h_g (.) x W_u) W_d with h_g = ReLU(x W_g), whose gate
 * activations are almost all exact zeros. The method is the one of "Sparser,
 * Faster, Lighter Transformer Language Models" (Cetin, Peluchetti, Castillo,
 * Naruse, Murakami, Jones), summarised on gist.science/it/paper/2603.23198:
 *   section 2.B.1  TwELL (Tile-wise ELLPACK), written by the gate matmul's
 *                  epilogue                                -> twell_gate_pack
 *   section 2.B.2  one fused stage applying the up and down projections to
 *                  the TwELL nonzeros only                  -> twell_ffn_fwd
 *   section 2.B.3  TwELL -> hybrid (ELL rows + dense backup) conversion, the
 *                  training forward over the hybrid and the sparse<->dense
 *                  products of the backward          -> twell_to_hybrid,
 *                                                      hybrid_ffn_fwd,
 *                                                      hybrid_ffn_bwd
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer unless marked (host). The caller owns
 *     all memory, including workspaces; the library allocates nothing, frees
 *     nothing and keeps no pointer after a call returns.
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL = the null
 *     stream) and return without synchronising.
 *   - No global state: concurrent calls on different streams are safe as long
 *     as their output buffers do not overlap.
 *   - The return value is a host-side status: TWELL_OK, or a negative
 *     TWELL_E_* code when an argument is rejected before anything is launched
 *     (or TWELL_E_HIP if a launch failed). No exception crosses the ABI.
 *   - Data-dependent conditions found on the device are OR-ed as
 *     TWELL_DEV_* bits into the int32 at `dev_status` (may be NULL); the call
 *     does not fail for them. The caller zeroes the word and reads it when it
 *     likes.
 *   - Row-major storage. x, dy: [T][d_model]. Weights, one contiguous d_model
 *     vector per neuron: wg_t, wu_t, wd: [d_ff][d_model], where row i of wg_t
 *     (wu_t) is column i of W_g (W_u) and row i of wd is row i of W_d.
 *   - Element types: TWELL_BF16 (bfloat16 storage, float32 accumulation) or
 *     TWELL_F32. y, dx and every weight gradient are float32.
 *   - Limits: d_model % 64 == 0 and 64 <= d_model <= 4096 (2048 for F32);
 *     d_ff % 128 == 0 and d_ff <= 32768; 0 <= T <= TWELL_MAX_ROWS; a
 *     hybrid's max_ovf <= TWELL_MAX_ROWS. With T == 0 the token
 *     arrays (x, dy, y, dx) may be NULL; the forward calls do nothing and the
 *     backward writes zero weight gradients.
 *     x, dy, weights, y, dx and gradients must be 16-byte aligned.
 */
#ifndef TWELL_H
#define TWELL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type. In C++ the enumeration has a fixed 32-bit underlying type, so
 * any int32 a caller passes is a value of the type: the calls check it and
 * return TWELL_E_DTYPE for anything but the two below. */
#ifdef __cplusplus
typedef enum : int32_t { TWELL_F32 = 0, TWELL_BF16 = 1 } twell_dtype;
#else
typedef enum { TWELL_F32 = 0, TWELL_BF16 = 1 } twell_dtype;
#endif

enum {
    TWELL_OK = 0,
    TWELL_E_NULL = -1,      /* a required pointer is NULL */
    TWELL_E_SHAPE = -2,     /* a size is out of range or inconsistent */
    TWELL_E_DTYPE = -3,     /* unsupported element type */
    TWELL_E_ALIGN = -4,     /* a pointer is not 16-byte aligned */
    TWELL_E_WORKSPACE = -5, /* workspace smaller than the *_workspace_bytes figure */
    TWELL_E_HIP = -6,       /* the HIP runtime rejected a launch */
    TWELL_E_SCRATCH = -7    /* more scratch needed than TWELL_STATIC_SCRATCH_BYTES */
};

/* device status bits */
enum {
    TWELL_DEV_TILE_OVERFLOW = 1, /* a (row, tile) held more than `width` nonzeros */
    TWELL_DEV_OVF_CAPACITY = 2,  /* more overflow rows than the backup's max_ovf */
    TWELL_DEV_BAD_INDEX = 4      /* a stored column was outside [0, d_ff); entry skipped */
};

#define TWELL_TILE_C 128 /* columns per TwELL tile: the gate kernel's N tile */
#define TWELL_MAX_ROWS (1 << 28) /* most tokens, and most backup rows, a call takes */
#define TWELL_DECODE_T 64 /* calls with at most this many tokens take the
                             few-token (decode) kernels; twell_decode_fwd's limit */

/*
 * Optional per-call kernel timing (host struct, caller-owned; pass NULL for
 * none). The caller creates up to TWELL_TIMING_MAX + 1 hipEvent_t handles and
 * puts them in events[0 .. n_events). A call records events[0] on its stream
 * before its first kernel and events[k] right after its k-th kernel, sets
 * n_used to the number of events it recorded and names[k - 1] to the name of
 * the k-th kernel. Recording stops when the events run out.
 */
#define TWELL_TIMING_MAX 24
typedef struct {
    void *events[TWELL_TIMING_MAX + 1];
    int32_t n_events;
    int32_t n_used;
    const char *names[TWELL_TIMING_MAX];
} twell_timing_t;

/*
 * TwELL of h = ReLU(x W_g) (section 2.B.1 of the summary page: the columns
 * are cut into tiles and each tile of each row keeps a count, the column
 * indices and the values of its nonzeros).
 *   count [T][d_ff/128] int32: number of g > 0 in the tile (the TRUE count,
 *                              which may exceed width; then the first `width`
 *                              entries are kept and TILE_OVERFLOW is raised)
 *   col   [T][d_ff/128][width] int16: global column in [0, d_ff), ascending
 *                              within the tile; slots >= count are untouched
 *   val   [T][d_ff/128][width] dtype: h = g rounded to nearest even
 * width in [1, 128]; 128 is lossless.
 */
typedef struct {
    int32_t T, d_ff, width;
    twell_dtype dtype;
    int32_t *count;
    int16_t *col;
    void *val;
} twell_t;

/*
 * Hybrid ELL + dense backup (section 2.B.3 of the summary page: rows with few
 * nonzeros in a compact ELL matrix, overflow rows redirected to a dense
 * backup). A row with row_nnz <= K is an ELL row; any other row is an
 * overflow row and goes whole to the backup. 1 <= K <= min(d_ff, 32767) and
 * T * K <= 2^31 - 1 (ELL slots are numbered in 32-bit integers); calls given
 * a larger hybrid return TWELL_E_SHAPE.
 *   row_nnz  [T] int32: stored entries of the row (sum over tiles of
 *                       min(count, width))
 *   row_slot [T] int32: -1 for an ELL row, else the row's backup slot; slots
 *                       are given in ascending row order
 *   ell_col  [T][K] int16, ell_val [T][K] dtype: the row's entries in
 *                       ascending column order (ELL rows only; other slots
 *                       are untouched)
 *   ovf_rows [max_ovf] int32: row of each backup slot, ascending
 *   dense    [max_ovf][d_ff] dtype: h at the row's columns, 0 elsewhere
 *   n_ovf    int32 (device scalar): TRUE number of overflow rows; if it
 *            exceeds max_ovf, OVF_CAPACITY is raised and rows past the
 *            capacity are not stored (the backward is then undefined)
 */
typedef struct {
    int32_t T, d_ff, K, max_ovf;
    twell_dtype dtype;
    int32_t *row_nnz;
    int32_t *row_slot;
    int16_t *ell_col;
    void *ell_val;
    int32_t *ovf_rows;
    void *dense;
    int32_t *n_ovf;
} hybrid_t;

/*
 * Gate matmul g = x W_g with the TwELL packing of h = ReLU(g) done in the
 * matmul's epilogue (section 2.B.1 of the summary page; the dothoosh.com
 * article: the conversion moved into the kernel's epilogue, tiles matched to
 * the matmul tile). g is never written to memory.
 *   x [T][d_model], wg_t [d_ff][d_model] (dtype dt); out (host struct with
 *   device arrays) sized as documented at twell_t, out->T == T,
 *   out->dtype == dt. Every count of every row < T is written.
 *   workspace: at least twell_gate_workspace_bytes(...) bytes; that is 0
 *   (workspace may be NULL) unless T <= TWELL_DECODE_T, where d_model is
 *   split across workgroups and the partial products of g (float32) pass
 *   through the workspace before the pack.
 * Errors: NULL / SHAPE / DTYPE / ALIGN / WORKSPACE / HIP.
 */
int twell_gate_pack(twell_dtype dt, const void *x, const void *wg_t, int32_t T, int32_t d_model,
                    const twell_t *out, void *workspace, size_t workspace_bytes,
                    int32_t *dev_status, twell_timing_t *timing, void *stream);

/* Workspace bytes twell_gate_pack needs (0 on invalid arguments). */
size_t twell_gate_workspace_bytes(twell_dtype dt, int32_t T, int32_t d_model, int32_t d_ff);

/*
 * Fused up and down projections over the TwELL nonzeros (section 2.B.2 of the
 * summary page): y[t] = sum over stored (i, h) of row t of
 * h * (x[t] . wu_t[i]) * wd[i], float32 accumulation. y [T][d_model] float32
 * is overwritten. workspace: at least twell_fwd_workspace_bytes(...) bytes
 * (it holds one float32 per TwELL slot).
 * Errors: NULL / SHAPE / DTYPE / ALIGN / WORKSPACE / HIP.
 */
int twell_ffn_fwd(twell_dtype dt, const void *x, const twell_t *h, const void *wu_t,
                  const void *wd, int32_t d_model, float *y, void *workspace,
                  size_t workspace_bytes, int32_t *dev_status, twell_timing_t *timing,
                  void *stream);

/* Workspace bytes twell_ffn_fwd needs (0 when it needs none, and on invalid
 * arguments). */
size_t twell_fwd_workspace_bytes(twell_dtype dt, int32_t T, int32_t d_model, int32_t d_ff,
                                 int32_t width);

/*
 * The whole layer for few tokens in one call: the matrix-vector regime of
 * decoding (the summary page, section 2.B.1, speaks of the gate product as a
 * dense matrix-vector kernel whose epilogue packs TwELL; the dothoosh.com
 * article notes that unstructured sparsity was long thought to pay off only
 * there). Three launches: gate partials over slices of d_model; per (token,
 * tile) the partials summed, the tile packed and a = h (x . wu_t[i]) formed
 * for its nonzeros; y by gathering slices of the wd rows. Nothing is
 * allocated or synchronised, so a caller may capture the call in a graph.
 *   out->T = T with 0 <= T <= TWELL_DECODE_T (T == 0: nothing is done);
 *   x [T][d_model], wg_t, wu_t, wd [d_ff][d_model] (dtype dt).
 *   out receives the TwELL of h as twell_gate_pack writes it (same counts,
 *   columns and values); y [T][d_model] float32 is overwritten with
 *   sum over stored (i, h) of h (x[t] . wu_t[i]) wd[i], float32 accumulation.
 *   workspace: at least twell_decode_workspace_bytes(...) bytes.
 * Errors: NULL / SHAPE / DTYPE / ALIGN / WORKSPACE / HIP.
 */
int twell_decode_fwd(twell_dtype dt, const void *x, const void *wg_t, const void *wu_t,
                     const void *wd, int32_t d_model, const twell_t *out, float *y,
                     void *workspace, size_t workspace_bytes, int32_t *dev_status,
                     twell_timing_t *timing, void *stream);

/* Workspace bytes twell_decode_fwd needs (0 on invalid arguments). */
size_t twell_decode_workspace_bytes(twell_dtype dt, int32_t T, int32_t d_model, int32_t d_ff,
                                    int32_t width);

/*
 * twell_decode_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels, arguments and results, with the scratch taken from a
 * static device array of TWELL_STATIC_SCRATCH_BYTES bytes that the library
 * holds on each GPU it runs on until the process ends. Nothing is allocated,
 * freed or synchronised. A call whose twell_decode_workspace_bytes(...)
 * exceeds the array returns TWELL_E_SCRATCH and launches nothing: the 2B
 * decode layer (d_model 2304, d_ff 6144) needs at most 9.4 MB for T <= 64,
 * the largest shapes (d_model 4096, d_ff 32768, width 128) need 16 MiB.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (on different streams, or from different threads) race and must be
 * ordered by the caller.
 * Errors: those of twell_decode_fwd except WORKSPACE, plus SCRATCH.
 */
#define TWELL_STATIC_SCRATCH_BYTES ((size_t)12 << 20)
int twell_decode_fwd_noalloc(twell_dtype dt, const void *x, const void *wg_t, const void *wu_t,
                             const void *wd, int32_t d_model, const twell_t *out, float *y,
                             int32_t *dev_status, twell_timing_t *timing, void *stream);

/*
 * TwELL -> hybrid conversion (section 2.B.3 of the summary page: a dedicated
 * conversion kernel). h and out must agree on T, d_ff and dtype;
 * 1 <= K <= d_ff; max_ovf >= 0. Writes every row_nnz, row_slot and n_ovf,
 * the ELL rows of ELL rows and the backup rows of the first max_ovf overflow
 * rows (whole rows, zeros included).
 * Errors: NULL / SHAPE / DTYPE / HIP.
 */
int twell_to_hybrid(const twell_t *h, const hybrid_t *out, int32_t *dev_status,
                    twell_timing_t *timing, void *stream);

/*
 * Training forward over a hybrid (section 2.B.3 of the summary page: the
 * hybrid layout carries the training forward as well as the backward):
 * y[t] = sum over row t's stored nonzeros (i, h) of h * (x[t] . wu_t[i]) * wd[i],
 * float32 accumulation. ELL rows use gathers; backup rows use two dense MFMA
 * products, A = h (.) (x_O W_u) then y_O = A W_d (A kept as a float32
 * intermediate in the workspace, for bf16 inputs as a hi/lo bf16 pair).
 *   x [T][d_model] dtype dt; y [T][d_model] float32, every row written.
 *   workspace: at least hybrid_fwd_workspace_bytes(...) bytes.
 * Streams: for large layers (at least 1024 tokens and 16 MB per weight
 * matrix) the backup rows' products run on a second stream that the library
 * keeps per device (non-blocking, default priority), ordered after the work
 * already on `stream` and joined back into it before the call returns: work
 * queued on `stream` afterwards sees every row of y, as with one stream.
 * While `stream` is being captured into a graph, and when timing is given,
 * every kernel runs on `stream`. Calls from several host threads at once
 * share the second stream (their backup products run one after another).
 * Undefined if the hybrid's OVF_CAPACITY bit was raised.
 * Errors: NULL / SHAPE / DTYPE / ALIGN / WORKSPACE / HIP.
 */
int hybrid_ffn_fwd(twell_dtype dt, const void *x, const hybrid_t *h, const void *wu_t,
                   const void *wd, int32_t d_model, float *y, void *workspace,
                   size_t workspace_bytes, int32_t *dev_status, twell_timing_t *timing,
                   void *stream);

/* Workspace bytes hybrid_ffn_fwd needs (0 on invalid arguments). */
size_t hybrid_fwd_workspace_bytes(twell_dtype dt, int32_t T, int32_t d_model, int32_t d_ff,
                                  int32_t K, int32_t max_ovf);

/*
 * Backward of y = (h (.) x W_u) W_d on the pattern P held by a hybrid
 * (section 2.B.3 of the summary page: sparse-to-dense and dense-to-sparse
 * products, no dense work on zeros). An entry is in P iff it is stored with a
 * nonzero value; ReLU' = 1 on P. With u = x W_u and da = dy W_d^T sampled on
 * P, a = h u, du = da h and dg = da u + l1:
 *   dx = du W_u^T + dg W_g^T,  dW_d = a^T dy,  dW_u = x^T du,  dW_g = x^T dg.
 * l1 is the weight of an L1 activation penalty l1 * sum(h) in the loss (the
 * training recipe of the dothoosh.com article: an L1 term on the FFN
 * activations); its gradient adds l1 to dg on P. Pass 0 for none; any scaling
 * (e.g. by the token count) is the caller's.
 * ELL rows use gathers; backup rows use dense MFMA products.
 *   dy [T][d_model] dtype dt; dx [T][d_model] float32; dwg_t, dwu_t, dwd
 *   [d_ff][d_model] float32 (storage layouts: dwg_t = dW_g^T, dwu_t = dW_u^T,
 *   dwd = dW_d); all overwritten. workspace: at least
 *   hybrid_bwd_workspace_bytes(...) bytes.
 * Undefined if the hybrid's OVF_CAPACITY bit was raised.
 * Errors: NULL / SHAPE / DTYPE / ALIGN / WORKSPACE / HIP.
 */
int hybrid_ffn_bwd(twell_dtype dt, const void *x, const void *dy, const hybrid_t *h,
                   const void *wg_t, const void *wu_t, const void *wd, int32_t d_model, float l1,
                   float *dx, float *dwg_t, float *dwu_t, float *dwd, void *workspace,
                   size_t workspace_bytes, int32_t *dev_status, twell_timing_t *timing,
                   void *stream);

/* Workspace bytes hybrid_ffn_bwd needs (0 on invalid arguments). */
size_t hybrid_bwd_workspace_bytes(twell_dtype dt, int32_t T, int32_t d_model, int32_t d_ff,
                                  int32_t K, int32_t max_ovf);

/* Static text for a TWELL_* status code (host). */
const char *twell_status_str(int code);

#ifdef __cplusplus
}
#endif

#endif /* TWELL_H */
