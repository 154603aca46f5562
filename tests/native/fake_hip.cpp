// A host-only stand-in for the HIP runtime calls and kernel launchers that
// libddp's host half (reducer.cpp) uses, so that the device path's host logic
// (table upload, stream ordering, the timing ring, failure handling) runs on
// a machine without a GPU, under AddressSanitizer and
// UndefinedBehaviorSanitizer. Nothing here computes a reduction.
//
// Streams are opaque pointers chosen by the test. Events are small host
// objects; recording one stamps it with a global sequence number, and the
// elapsed time between two events is the start event's stamp (so a test can
// tell which launch a duration was read from). Work completes at once:
// queries and waits succeed. Every call is appended to a log the test reads.
// The static table area is host memory here.
#include "fake_hip.h"

#include "ddp.h"
#include "internal.h"
#include "static_area.h"

#include <cstdlib>
#include <cstring>

namespace fake {

std::vector<Call> g_log;
long g_live_events = 0;
long g_max_live_events = 0;
long g_stamp = 0;
hipError_t g_stream_query = hipErrorNotReady;
hipError_t g_event_query = hipSuccess;
bool g_logging = true;
bool g_capturing = false;
long g_stream_queries = 0;

namespace {

struct Event {
    long stamp = -1;   // sequence number of the last record; -1: never recorded
};

void log_call(Call c)
{
    if (g_logging) g_log.push_back(c);
}

hipError_t launch(const char *what, hipStream_t s, int32_t tile0, int32_t tiles, unsigned lds, bool pair)
{
    Call c{};
    c.what = what;
    c.stream = s;
    c.a = tile0;
    c.b = tiles;
    c.lds = lds;
    c.pair = pair;
    log_call(c);
    return hipSuccess;
}

}  // namespace

long stamp_of(hipEvent_t e)
{
    return reinterpret_cast<Event *>(e)->stamp;
}

void reset_log()
{
    g_log.clear();
}

}  // namespace fake

using fake::Call;

extern "C" {

hipError_t hipEventCreateWithFlags(hipEvent_t *event, unsigned)
{
    // malloc, not new: tests that make operator new fail must not fail here
    void *mem = std::malloc(sizeof(fake::Event));
    if (!mem) return hipErrorOutOfMemory;
    *event = reinterpret_cast<hipEvent_t>(new (mem) fake::Event());
    ++fake::g_live_events;
    if (fake::g_live_events > fake::g_max_live_events) fake::g_max_live_events = fake::g_live_events;
    return hipSuccess;
}

hipError_t hipEventDestroy(hipEvent_t event)
{
    if (!event) return hipErrorInvalidHandle;
    std::free(reinterpret_cast<void *>(event));
    --fake::g_live_events;
    return hipSuccess;
}

hipError_t hipEventRecord(hipEvent_t event, hipStream_t stream)
{
    if (!event) return hipErrorInvalidHandle;
    reinterpret_cast<fake::Event *>(event)->stamp = fake::g_stamp++;
    Call c{};
    c.what = "record";
    c.stream = stream;
    c.event = event;
    fake::log_call(c);
    return hipSuccess;
}

hipError_t hipStreamWaitEvent(hipStream_t stream, hipEvent_t event, unsigned int)
{
    if (!event) return hipErrorInvalidHandle;
    Call c{};
    c.what = "wait";
    c.stream = stream;
    c.event = event;
    fake::log_call(c);
    return hipSuccess;
}

hipError_t hipStreamQuery(hipStream_t)
{
    ++fake::g_stream_queries;
    return fake::g_stream_query;
}

hipError_t hipStreamIsCapturing(hipStream_t stream, hipStreamCaptureStatus *status)
{
    if (!status) return hipErrorInvalidValue;
    *status = stream && fake::g_capturing ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
    return hipSuccess;
}

hipError_t hipEventQuery(hipEvent_t event)
{
    if (!event) return hipErrorInvalidHandle;
    return fake::stamp_of(event) < 0 ? hipSuccess : fake::g_event_query;
}

hipError_t hipEventSynchronize(hipEvent_t event)
{
    if (!event) return hipErrorInvalidHandle;
    Call c{};
    c.what = "sync";
    c.event = event;
    fake::log_call(c);
    return hipSuccess;
}

hipError_t hipEventElapsedTime(float *ms, hipEvent_t start, hipEvent_t stop)
{
    if (!start || !stop || !ms) return hipErrorInvalidHandle;
    const long a = fake::stamp_of(start), b = fake::stamp_of(stop);
    if (a < 0 || b < a) return hipErrorNotReady;
    *ms = float(a);
    return hipSuccess;
}

hipError_t hipMemcpy(void *dst, const void *src, size_t n, hipMemcpyKind)
{
    std::memcpy(dst, src, n);
    return hipSuccess;
}

hipError_t hipMemcpyAsync(void *dst, const void *src, size_t n, hipMemcpyKind, hipStream_t stream)
{
    std::memcpy(dst, src, n);
    Call c{};
    c.what = "copy";
    c.stream = stream;
    c.a = int64_t(n);
    fake::log_call(c);
    return hipSuccess;
}

hipError_t hipHostMalloc(void **ptr, size_t size, unsigned int)
{
    *ptr = std::malloc(size ? size : 1);
    return *ptr ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t hipHostFree(void *ptr)
{
    std::free(ptr);
    return hipSuccess;
}

hipError_t hipGetDevice(int *device)
{
    *device = 0;
    return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t attr, int)
{
    (void)attr;   // gfx950: 160 KiB of LDS per CU, all of it available to one workgroup
    *value = 160 * 1024;
    return hipSuccess;
}

const char *hipGetErrorString(hipError_t)
{
    return "fake HIP error";
}

hipError_t hipDeviceSynchronize(void)
{
    Call c{};
    c.what = "device_sync";
    fake::log_call(c);
    return hipSuccess;
}

}  // extern "C"

namespace ddp {

// The static table area, as host memory: one area, device 0 only.
namespace {
alignas(256) unsigned char g_area[DDP_STATIC_TABLE_BYTES];
uint64_t g_area_generation = 0;
}  // namespace

hipError_t static_table_area(int device, void **ptr, size_t *bytes)
{
    if (device != 0) return hipErrorInvalidDevice;
    *ptr = g_area;
    *bytes = sizeof(g_area);
    return hipSuccess;
}

uint64_t claim_static_table_area(int)
{
    return ++g_area_generation;
}

uint64_t static_table_generation(int)
{
    return g_area_generation;
}

hipError_t launch_mean(int, int, bool, const Scale &, const KernelTables &, int32_t tile0, int32_t tiles,
                       unsigned lds, bool pair, hipStream_t s)
{
    return fake::launch("launch", s, tile0, tiles, lds, pair);
}

hipError_t launch_bf16_hook(int, int, bool, const Scale &, const KernelTables &, int32_t tile0, int32_t tiles,
                            unsigned lds, bool pair, hipStream_t s)
{
    return fake::launch("launch", s, tile0, tiles, lds, pair);
}

hipError_t launch_fp16_hook(int, int, bool, const Scale &, const KernelTables &, int32_t tile0, int32_t tiles,
                            unsigned lds, bool pair, hipStream_t s)
{
    return fake::launch("launch", s, tile0, tiles, lds, pair);
}

}  // namespace ddp
