// The static table area: device memory that the library owns for callers
// that cannot allocate (ddp_reducer_create_static). It holds a reducer's
// device tables (gradient and flat pointer tables, segment records, the
// tile -> segment map) in place of a caller-allocated workspace.
//
// The array below is a device variable: in host code its name is only a
// host-side stand-in, never a device address. Its device address is looked
// up once per device, with that device current, through
// hipGetSymbolAddress, and only that address is ever handed to a copy or a
// kernel. Each device holds its own copy of the array for the life of the
// process. Every static reducer created on a device claims the whole area
// (a new generation); the reducer remembers its generation and refuses to
// launch once a later claim has replaced its tables.
#include "../../include/ddp.h"
#include "internal.h"
#include "static_area.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

namespace {

static __device__ __align__(256) unsigned char scratch[DDP_STATIC_TABLE_BYTES];

constexpr int kMaxDevices = 64;

std::mutex g_lock;
void *g_addr[kMaxDevices] = {};                    // device address of scratch, per device
std::atomic<uint64_t> g_generation[kMaxDevices];   // last claim per device (0: none)

}  // namespace

namespace ddp {

hipError_t static_table_area(int device, void **ptr, size_t *bytes)
{
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    int current = -1;
    hipError_t e = hipGetDevice(&current);
    if (e != hipSuccess) return e;
    if (current != device) return hipErrorInvalidDevice;   // looked up with its device current only
    std::lock_guard<std::mutex> hold(g_lock);
    if (!g_addr[device]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_addr[device] = p;
    }
    *ptr = g_addr[device];
    *bytes = DDP_STATIC_TABLE_BYTES;
    return hipSuccess;
}

uint64_t claim_static_table_area(int device)
{
    return g_generation[device].fetch_add(1) + 1;
}

uint64_t static_table_generation(int device)
{
    return g_generation[device].load();
}

}  // namespace ddp
