// Scratch memory of the allocation-free forward (solattn_fwd_noalloc).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace solattn {

// Size in bytes of the file-scope device array that holds the fused
// kernel's work-queue counters for solattn_fwd_noalloc.
size_t noalloc_scratch_bytes();

// Device address of that array on the current device, looked up with
// hipGetSymbolAddress the first time a device asks and kept per device.
hipError_t noalloc_scratch(void** ptr);

}  // namespace solattn
