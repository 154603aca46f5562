// The library's static table area (static_tables.hip), used by
// ddp_reducer_create_static in place of a caller-allocated workspace. Not
// part of the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

namespace ddp {

// The area on `device`, which must be the current device: its device
// address and size. The address is looked up once per device.
hipError_t static_table_area(int device, void **ptr, size_t *bytes);
// A reducer taking the area claims it: the returned generation is current
// until the next claim on the same device.
uint64_t claim_static_table_area(int device);
uint64_t static_table_generation(int device);

}  // namespace ddp
