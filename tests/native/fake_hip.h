// The log and knobs of the host-only HIP stand-in (fake_hip.cpp).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <vector>

namespace fake {

struct Call {
    const char *what;     // "record", "wait", "sync", "copy", "launch"
    hipStream_t stream;   // the stream the call targets (none for "sync")
    hipEvent_t event;     // record, wait, sync
    int64_t a, b;         // launch: first tile, tiles; copy: bytes
    unsigned lds;         // launch: LDS reserved per workgroup
    bool pair;            // launch: two tiles per workgroup
};

extern std::vector<Call> g_log;
extern long g_live_events;       // events created and not destroyed
extern long g_max_live_events;   // the most ever alive at once
extern hipError_t g_stream_query;   // what hipStreamQuery returns (default: hipErrorNotReady)
extern hipError_t g_event_query;    // what hipEventQuery returns for a recorded event (default: hipSuccess)
extern bool g_logging;              // append calls to g_log
extern bool g_capturing;            // what hipStreamIsCapturing reports for every non-null stream
extern long g_stream_queries;       // hipStreamQuery calls so far

long stamp_of(hipEvent_t e);
void reset_log();

}  // namespace fake
