// A second stream per device, for products that can run beside the work of
// the stream a call was given (host side only).
//
// Per device: a non-blocking stream of default priority and NEV events
// (timing off, device-scope release: both streams are on one device, and the
// default system-scope release would write back and invalidate the caches),
// made on first use and kept until the process ends. A call records ev[0] on
// its stream and makes the side stream wait on it (fork), queues work on the
// side stream, records further events there (marks) and makes its stream
// wait on them where it needs that work (joins). The mutex holds one call's fork ... join sequence together
// when several host threads call at once; their side work then also queues
// one piece after another on the one side stream.
#pragma once

#include <mutex>

#include "common.hpp"

struct SideStream {
    static constexpr int NEV = 2;
    hipStream_t s = nullptr;
    hipEvent_t ev[NEV] = {};
    std::mutex m;
    bool ok = false;
};

// The side stream of stream s's device, or nullptr when s is being captured
// into a graph, its device is unknown or the stream could not be made: the
// caller then queues everything on s, in order.
SideStream *side_stream(hipStream_t s);

// Fork: lock ss, then make its stream wait for everything already queued on
// s. Returns false (and leaves ss unlocked) when the fork could not be made.
bool side_fork(SideStream *ss, hipStream_t s, std::unique_lock<std::mutex> &lk);

// Mark k (1 <= k < NEV): record ev[k] on the side stream after the work
// queued there so far. Returns whether it was recorded.
bool side_mark(SideStream *ss, int k);

// Make s wait for mark k (marked: what side_mark returned). Where that cannot
// be queued, the host waits for the side stream instead, so that whatever is
// queued on s afterwards still runs after the side work.
void side_wait(SideStream *ss, int k, bool marked, hipStream_t s);
