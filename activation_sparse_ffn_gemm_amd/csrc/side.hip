// Per-device side streams (side.hpp).
#include "side.hpp"

namespace {
constexpr int MAX_DEVICES = 64;
SideStream g_side[MAX_DEVICES];
std::once_flag g_once[MAX_DEVICES];
} // namespace

SideStream *side_stream(hipStream_t s)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
        (void)hipGetLastError();
        return nullptr;
    }
    int d = -1;
    if (hipStreamGetDevice(s, &d) != hipSuccess || d < 0 || d >= MAX_DEVICES) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::call_once(g_once[d], [d] {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess || hipSetDevice(d) != hipSuccess) {
            (void)hipGetLastError();
            return;
        }
        SideStream &ss = g_side[d];
        bool ok = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) == hipSuccess;
        for (int k = 0; ok && k < SideStream::NEV; ++k)
            ok = hipEventCreateWithFlags(&ss.ev[k], hipEventDisableTiming |
                                                        hipEventReleaseToDevice) == hipSuccess;
        ss.ok = ok;
        (void)hipSetDevice(cur);
        (void)hipGetLastError();
    });
    return g_side[d].ok ? &g_side[d] : nullptr;
}

bool side_fork(SideStream *ss, hipStream_t s, std::unique_lock<std::mutex> &lk)
{
    lk = std::unique_lock<std::mutex>(ss->m);
    if (hipEventRecord(ss->ev[0], s) == hipSuccess &&
        hipStreamWaitEvent(ss->s, ss->ev[0], 0) == hipSuccess)
        return true;
    (void)hipGetLastError();
    lk.unlock();
    return false;
}

bool side_mark(SideStream *ss, int k)
{
    if (hipEventRecord(ss->ev[k], ss->s) == hipSuccess)
        return true;
    (void)hipGetLastError();
    return false;
}

void side_wait(SideStream *ss, int k, bool marked, hipStream_t s)
{
    if (marked && hipStreamWaitEvent(s, ss->ev[k], 0) == hipSuccess)
        return;
    (void)hipGetLastError();
    (void)hipStreamSynchronize(ss->s);
}
