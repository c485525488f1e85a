// twell_decode_fwd without a caller workspace: for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). The decode layer's scratch (the gate's
// partial sums, then one float per TwELL slot) lives in a file-scope device
// array instead, one copy per GPU, held until the process ends. The kernels
// overwrite every byte of it they later read, so nothing is cleared between
// calls; calls that overlap on one GPU share the array and race.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is handed to the kernels.
#include <mutex>

#include "common.hpp"

int check_decode_args(twell_dtype dt, const void *x, const void *wg_t, const void *wu_t,
                      const void *wd, int32_t d_model, const twell_t *out, const float *y);
hipError_t launch_dec_layer(twell_dtype dt, const void *x, const void *wg_t, const void *wu_t,
                            const void *wd, int dm, const twell_t *o, float *y, void *ws,
                            int32_t *status, twell_timing_t *timing, hipStream_t s);

static __device__ __align__(256) uint8_t scratch[TWELL_STATIC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_scratch[MAX_DEVICES]; // device address of `scratch` on each device, or null

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device; null if the lookup fails.
void *scratch_ptr()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
        return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

} // namespace

extern "C" int twell_decode_fwd_noalloc(twell_dtype dt, const void *x, const void *wg_t,
                                        const void *wu_t, const void *wd, int32_t d_model,
                                        const twell_t *out, float *y, int32_t *dev_status,
                                        twell_timing_t *timing, void *stream)
{
    if (int rc = check_decode_args(dt, x, wg_t, wu_t, wd, d_model, out, y))
        return rc;
    const size_t need = twell_decode_workspace_bytes(dt, out->T, d_model, out->d_ff, out->width);
    if (need > TWELL_STATIC_SCRATCH_BYTES)
        return TWELL_E_SCRATCH;
    if (out->T == 0)
        return TWELL_OK;
    void *ws = scratch_ptr();
    if (!ws)
        return TWELL_E_HIP;
    return launch_dec_layer(dt, x, wg_t, wu_t, wd, d_model, out, y, ws, dev_status, timing,
                            (hipStream_t)stream) == hipSuccess
               ? TWELL_OK
               : TWELL_E_HIP;
}
