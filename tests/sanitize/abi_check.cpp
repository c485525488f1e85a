// Host-side checks of the C-ABI, built without device code and run under
// AddressSanitizer and UndefinedBehaviorSanitizer (no GPU is touched):
//   - every entry point refuses bad arguments with the documented code before
//     it reaches the HIP runtime;
//   - every workspace sizer, fed sizes up to INT32_MAX, returns without
//     undefined behaviour (signed overflow, bad shifts) and either refuses the
//     shape (0) or returns a size that covers at least its float32 outputs;
//   - the allocation-free decode call refuses, on the host, a call larger
//     than its static scratch.
// Prints "abi_check ok" and exits 0; any failed expectation exits 1, and any
// sanitizer report aborts the program.
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "twell.h"

static int failures = 0;

#define EXPECT(cond)                                                                       \
    do {                                                                                   \
        if (!(cond)) {                                                                     \
            std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__,    \
                         #cond);                                                           \
            ++failures;                                                                    \
        }                                                                                  \
    } while (0)

// 16-byte aligned addresses that are never dereferenced: every call below is
// refused before any pointer is used.
static void *const FAKE = (void *)(uintptr_t)0x100000;
static void *const MISALIGNED = (void *)(uintptr_t)0x100004;

static twell_t twell(int32_t T = 4, int32_t d_ff = 256, int32_t width = 128,
                     twell_dtype dt = TWELL_BF16, void *p = FAKE)
{
    twell_t t;
    t.T = T;
    t.d_ff = d_ff;
    t.width = width;
    t.dtype = dt;
    t.count = (int32_t *)p;
    t.col = (int16_t *)p;
    t.val = p;
    return t;
}

static hybrid_t hybrid(int32_t T = 4, int32_t d_ff = 256, int32_t K = 16, int32_t max_ovf = 4,
                       twell_dtype dt = TWELL_BF16, void *p = FAKE)
{
    hybrid_t h;
    h.T = T;
    h.d_ff = d_ff;
    h.K = K;
    h.max_ovf = max_ovf;
    h.dtype = dt;
    h.row_nnz = (int32_t *)p;
    h.row_slot = (int32_t *)p;
    h.ell_col = (int16_t *)p;
    h.ell_val = p;
    h.ovf_rows = (int32_t *)p;
    h.dense = p;
    h.n_ovf = (int32_t *)p;
    return h;
}

static void check_status_strings()
{
    for (int c = -7; c <= 0; ++c)
        EXPECT(twell_status_str(c) && std::strlen(twell_status_str(c)) > 0);
    EXPECT(std::strcmp(twell_status_str(99), "unknown status") == 0);
    EXPECT(std::strcmp(twell_status_str(INT_MIN), "unknown status") == 0);
}

static void check_gate_pack()
{
    const size_t big = (size_t)1 << 30;
    twell_t t = twell();
    EXPECT(twell_gate_pack((twell_dtype)7, FAKE, FAKE, 4, 64, &t, FAKE, big, 0, 0, 0) ==
           TWELL_E_DTYPE);
    EXPECT(twell_gate_pack(TWELL_BF16, 0, FAKE, 4, 64, &t, FAKE, big, 0, 0, 0) == TWELL_E_NULL);
    EXPECT(twell_gate_pack(TWELL_BF16, FAKE, FAKE, 4, 64, 0, FAKE, big, 0, 0, 0) ==
           TWELL_E_NULL);
    EXPECT(twell_gate_pack(TWELL_BF16, FAKE, FAKE, 4, 96, &t, FAKE, big, 0, 0, 0) ==
           TWELL_E_SHAPE);
    EXPECT(twell_gate_pack(TWELL_BF16, FAKE, FAKE, 4, INT_MAX, &t, FAKE, big, 0, 0, 0) ==
           TWELL_E_SHAPE);
    EXPECT(twell_gate_pack(TWELL_BF16, FAKE, FAKE, -1, 64, &t, FAKE, big, 0, 0, 0) ==
           TWELL_E_SHAPE);
    EXPECT(twell_gate_pack(TWELL_BF16, FAKE, FAKE, 5, 64, &t, FAKE, big, 0, 0, 0) ==
           TWELL_E_SHAPE);
    t = twell(4, 200);
    EXPECT(twell_gate_pack(TWELL_BF16, FAKE, FAKE, 4, 64, &t, FAKE, big, 0, 0, 0) ==
           TWELL_E_SHAPE);
    t = twell(4, 65536);
    EXPECT(twell_gate_pack(TWELL_BF16, FAKE, FAKE, 4, 64, &t, FAKE, big, 0, 0, 0) ==
           TWELL_E_SHAPE);
    t = twell(4, 256, 0);
    EXPECT(twell_gate_pack(TWELL_BF16, FAKE, FAKE, 4, 64, &t, FAKE, big, 0, 0, 0) ==
           TWELL_E_SHAPE);
    t = twell(4, 256, 129);
    EXPECT(twell_gate_pack(TWELL_BF16, FAKE, FAKE, 4, 64, &t, FAKE, big, 0, 0, 0) ==
           TWELL_E_SHAPE);
    t = twell();
    EXPECT(twell_gate_pack(TWELL_BF16, MISALIGNED, FAKE, 4, 64, &t, FAKE, big, 0, 0, 0) ==
           TWELL_E_ALIGN);
    const size_t need = twell_gate_workspace_bytes(TWELL_BF16, 4, 64, 256);
    EXPECT(need >= (size_t)4 * 256 * 4);
    EXPECT(twell_gate_pack(TWELL_BF16, FAKE, FAKE, 4, 64, &t, FAKE, need - 1, 0, 0, 0) ==
           TWELL_E_WORKSPACE);
    EXPECT(twell_gate_pack(TWELL_BF16, FAKE, FAKE, 4, 64, &t, 0, 0, 0, 0, 0) ==
           TWELL_E_WORKSPACE);
    t = twell(0, 256, 128, TWELL_BF16, 0);
    EXPECT(twell_gate_pack(TWELL_BF16, 0, FAKE, 0, 64, &t, 0, 0, 0, 0, 0) == TWELL_OK);
}

static void check_ffn_fwd()
{
    twell_t t = twell();
    const size_t big = (size_t)1 << 30;
    EXPECT(twell_ffn_fwd((twell_dtype)9, FAKE, &t, FAKE, FAKE, 64, (float *)FAKE, FAKE, big, 0,
                         0, 0) == TWELL_E_DTYPE);
    EXPECT(twell_ffn_fwd(TWELL_BF16, FAKE, &t, FAKE, FAKE, 64, 0, FAKE, big, 0, 0, 0) ==
           TWELL_E_NULL);
    EXPECT(twell_ffn_fwd(TWELL_BF16, FAKE, 0, FAKE, FAKE, 64, (float *)FAKE, FAKE, big, 0, 0,
                         0) == TWELL_E_NULL);
    EXPECT(twell_ffn_fwd(TWELL_BF16, FAKE, &t, FAKE, FAKE, 100, (float *)FAKE, FAKE, big, 0, 0,
                         0) == TWELL_E_SHAPE);
    EXPECT(twell_ffn_fwd(TWELL_BF16, FAKE, &t, FAKE, FAKE, 64, (float *)MISALIGNED, FAKE, big,
                         0, 0, 0) == TWELL_E_ALIGN);
    twell_t f = twell(4, 256, 128, TWELL_F32);
    EXPECT(twell_ffn_fwd(TWELL_BF16, FAKE, &f, FAKE, FAKE, 64, (float *)FAKE, FAKE, big, 0, 0,
                         0) == TWELL_E_DTYPE);
    twell_t z = twell(0, 256, 128, TWELL_BF16, 0);
    EXPECT(twell_ffn_fwd(TWELL_BF16, FAKE, &z, FAKE, FAKE, 64, (float *)FAKE, FAKE, big, 0, 0,
                         0) == TWELL_OK);
    const size_t need = twell_fwd_workspace_bytes(TWELL_BF16, 4, 64, 256, 128);
    if (need)
        EXPECT(twell_ffn_fwd(TWELL_BF16, FAKE, &t, FAKE, FAKE, 64, (float *)FAKE, FAKE,
                             need - 1, 0, 0, 0) == TWELL_E_WORKSPACE);
}

static void check_decode()
{
    twell_t t = twell();
    const size_t need = twell_decode_workspace_bytes(TWELL_BF16, 4, 64, 256, 128);
    EXPECT(need >= (size_t)4 * 256 * 4 + (size_t)4 * 2 * 128 * 4);
    EXPECT(twell_decode_workspace_bytes(TWELL_BF16, 65, 64, 256, 128) == 0);
    EXPECT(twell_decode_fwd((twell_dtype)9, FAKE, FAKE, FAKE, FAKE, 64, &t, (float *)FAKE, FAKE,
                            need, 0, 0, 0) == TWELL_E_DTYPE);
    EXPECT(twell_decode_fwd(TWELL_BF16, FAKE, 0, FAKE, FAKE, 64, &t, (float *)FAKE, FAKE, need,
                            0, 0, 0) == TWELL_E_NULL);
    EXPECT(twell_decode_fwd(TWELL_BF16, FAKE, FAKE, FAKE, FAKE, 100, &t, (float *)FAKE, FAKE,
                            need, 0, 0, 0) == TWELL_E_SHAPE);
    twell_t t65 = twell(65);
    EXPECT(twell_decode_fwd(TWELL_BF16, FAKE, FAKE, FAKE, FAKE, 64, &t65, (float *)FAKE, FAKE,
                            need, 0, 0, 0) == TWELL_E_SHAPE);
    EXPECT(twell_decode_fwd(TWELL_BF16, FAKE, FAKE, FAKE, FAKE, 64, &t, (float *)FAKE, FAKE,
                            need - 1, 0, 0, 0) == TWELL_E_WORKSPACE);
    EXPECT(twell_decode_fwd(TWELL_BF16, FAKE, FAKE, FAKE, FAKE, 64, &t, (float *)FAKE,
                            MISALIGNED, need, 0, 0, 0) == TWELL_E_ALIGN);
    // allocation-free variant: same checks, and the static-scratch limit
    EXPECT(twell_decode_fwd_noalloc(TWELL_BF16, FAKE, FAKE, FAKE, FAKE, 64, &t, 0, 0, 0, 0) ==
           TWELL_E_NULL);
    EXPECT(twell_decode_fwd_noalloc(TWELL_BF16, FAKE, FAKE, FAKE, FAKE, 100, &t, (float *)FAKE,
                                    0, 0, 0) == TWELL_E_SHAPE);
    twell_t big = twell(64, 32768, 128);
    EXPECT(twell_decode_workspace_bytes(TWELL_BF16, 64, 4096, 32768, 128) >
           TWELL_STATIC_SCRATCH_BYTES);
    EXPECT(twell_decode_fwd_noalloc(TWELL_BF16, FAKE, FAKE, FAKE, FAKE, 4096, &big,
                                    (float *)FAKE, 0, 0, 0) == TWELL_E_SCRATCH);
    twell_t z = twell(0, 256, 128, TWELL_BF16, 0);
    EXPECT(twell_decode_fwd_noalloc(TWELL_BF16, 0, FAKE, FAKE, FAKE, 64, &z, 0, 0, 0, 0) ==
           TWELL_OK);
}

static void check_hybrid_calls()
{
    twell_t t = twell();
    hybrid_t h = hybrid();
    hybrid_t bad = hybrid(5);
    EXPECT(twell_to_hybrid(&t, &bad, 0, 0, 0) == TWELL_E_SHAPE);
    bad = hybrid(4, 256, 0);
    EXPECT(twell_to_hybrid(&t, &bad, 0, 0, 0) == TWELL_E_SHAPE);
    bad = hybrid(4, 256, 300);
    EXPECT(twell_to_hybrid(&t, &bad, 0, 0, 0) == TWELL_E_SHAPE);
    bad = hybrid(4, 256, 16, -1);
    EXPECT(twell_to_hybrid(&t, &bad, 0, 0, 0) == TWELL_E_SHAPE);
    bad = hybrid(4, 256, 16, 4, TWELL_F32);
    EXPECT(twell_to_hybrid(&t, &bad, 0, 0, 0) == TWELL_E_DTYPE);
    bad = hybrid(4, 256, 16, 4, TWELL_BF16, 0);
    EXPECT(twell_to_hybrid(&t, &bad, 0, 0, 0) == TWELL_E_NULL);
    EXPECT(twell_to_hybrid(0, &h, 0, 0, 0) == TWELL_E_NULL);
    // T * K past 2^31 - 1: ELL slot numbers would overflow
    twell_t tb = twell(1 << 20, 4096);
    hybrid_t hb = hybrid(1 << 20, 4096, 4096);
    EXPECT(twell_to_hybrid(&tb, &hb, 0, 0, 0) == TWELL_E_SHAPE);
    EXPECT(hybrid_bwd_workspace_bytes(TWELL_BF16, 1 << 20, 64, 4096, 4096, 4) == 0);
    EXPECT(hybrid_ffn_bwd(TWELL_BF16, FAKE, FAKE, &hb, FAKE, FAKE, FAKE, 64, 0.f, (float *)FAKE,
                          (float *)FAKE, (float *)FAKE, (float *)FAKE, FAKE, (size_t)1 << 40, 0,
                          0, 0) == TWELL_E_SHAPE);

    const size_t nf = hybrid_fwd_workspace_bytes(TWELL_BF16, 4, 64, 256, 16, 4);
    EXPECT(nf > 0);
    EXPECT(hybrid_fwd_workspace_bytes(TWELL_BF16, 4, 64, 256, 16, 0) == 0);
    EXPECT(hybrid_ffn_fwd(TWELL_BF16, FAKE, &h, FAKE, FAKE, 64, (float *)FAKE, FAKE, nf - 1, 0,
                          0, 0) == TWELL_E_WORKSPACE);
    EXPECT(hybrid_ffn_fwd(TWELL_BF16, 0, &h, FAKE, FAKE, 64, (float *)FAKE, FAKE, nf, 0, 0, 0) ==
           TWELL_E_NULL);
    EXPECT(hybrid_ffn_fwd(TWELL_BF16, FAKE, &h, FAKE, FAKE, 32, (float *)FAKE, FAKE, nf, 0, 0,
                          0) == TWELL_E_SHAPE);
    EXPECT(hybrid_ffn_fwd(TWELL_F32, FAKE, &h, FAKE, FAKE, 64, (float *)FAKE, FAKE, nf, 0, 0,
                          0) == TWELL_E_DTYPE);

    const size_t nb = hybrid_bwd_workspace_bytes(TWELL_BF16, 4, 64, 256, 16, 4);
    EXPECT(nb > 0);
    float *F = (float *)FAKE;
    EXPECT(hybrid_ffn_bwd(TWELL_BF16, FAKE, FAKE, &h, FAKE, FAKE, FAKE, 64, NAN, F, F, F, F,
                          FAKE, nb, 0, 0, 0) == TWELL_E_SHAPE);
    EXPECT(hybrid_ffn_bwd(TWELL_BF16, FAKE, FAKE, &h, FAKE, FAKE, FAKE, 64, INFINITY, F, F, F,
                          F, FAKE, nb, 0, 0, 0) == TWELL_E_SHAPE);
    EXPECT(hybrid_ffn_bwd(TWELL_BF16, FAKE, FAKE, &h, FAKE, FAKE, FAKE, 64, 0.f, F, F, F, F,
                          FAKE, nb - 1, 0, 0, 0) == TWELL_E_WORKSPACE);
    EXPECT(hybrid_ffn_bwd(TWELL_BF16, FAKE, FAKE, &h, FAKE, FAKE, FAKE, 64, 0.f, 0, F, F, F,
                          FAKE, nb, 0, 0, 0) == TWELL_E_NULL);
    EXPECT(hybrid_ffn_bwd(TWELL_BF16, FAKE, FAKE, &h, FAKE, FAKE, FAKE, 32, 0.f, F, F, F, F,
                          FAKE, nb, 0, 0, 0) == TWELL_E_SHAPE);
    EXPECT(hybrid_ffn_bwd(TWELL_BF16, FAKE, FAKE, &h, FAKE, FAKE, FAKE, 64, 0.f,
                          (float *)MISALIGNED, F, F, F, FAKE, nb, 0, 0, 0) == TWELL_E_ALIGN);
}

// Sizes from the edges of every argument's range: no undefined behaviour, and
// a size, when one is returned, at least as large as the float32 data it must
// hold at minimum.
static void check_sizers()
{
    const int32_t Ts[] = {0, 1, 64, 65, 4096, 1 << 20, INT_MAX};
    const int32_t dms[] = {64, 2048, 4096, 8192, INT_MAX - 63};
    const int32_t dffs[] = {128, 5632, 32768, 65536, INT_MAX - 127};
    const int32_t Ks[] = {1, 128, 32767, INT_MAX};
    const int32_t ovfs[] = {0, 1, 1024, 1 << 20, INT_MAX};
    const int32_t Ws[] = {1, 32, 128, 129, INT_MAX};
    const twell_dtype dts[] = {TWELL_F32, TWELL_BF16, (twell_dtype)5};
    volatile size_t sink = 0;
    for (twell_dtype dt : dts)
        for (int32_t T : Ts)
            for (int32_t dm : dms)
                for (int32_t dff : dffs) {
                    sink += twell_gate_workspace_bytes(dt, T, dm, dff);
                    for (int32_t W : Ws) {
                        sink += twell_fwd_workspace_bytes(dt, T, dm, dff, W);
                        const size_t d = twell_decode_workspace_bytes(dt, T, dm, dff, W);
                        if (d)
                            EXPECT(d >= (size_t)T * (size_t)dff * 4);
                    }
                    for (int32_t K : Ks)
                        for (int32_t o : ovfs) {
                            sink += hybrid_fwd_workspace_bytes(dt, T, dm, dff, K, o);
                            const size_t b = hybrid_bwd_workspace_bytes(dt, T, dm, dff, K, o);
                            if (b && T > 0)
                                EXPECT(b >= (size_t)T * (size_t)(K < dff ? K : dff) * 4 * 2);
                        }
                }
    (void)sink;
}

int main()
{
    check_status_strings();
    check_gate_pack();
    check_ffn_fwd();
    check_decode();
    check_hybrid_calls();
    check_sizers();
    if (failures) {
        std::fprintf(stderr, "abi_check: %d expectation(s) failed\n", failures);
        return 1;
    }
    std::printf("abi_check ok\n");
    return 0;
}
