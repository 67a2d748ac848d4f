// zsp_entry.hpp -- helpers shared by the source files that implement entry
// points: error reporting (the thread-local message zsp_last_error()
// returns) and the gather behind zsp_gather_range.
#pragma once

#include <hip/hip_runtime.h>

#include "zsp.h"

struct zsp_plan;

namespace zsp {

zsp_status set_error(zsp_status st, const char* fmt, ...);
zsp_status set_hip_error(hipError_t e, const char* what);

// ZSP_OK if the plan has state bound on the current device, else the error.
zsp_status check_bound(const zsp_plan* P);

// Locates the no-alloc list gather's static device array on the current
// device (zsp_noalloc.hip); ZSP_OK once done.
zsp_status noalloc_setup();

// zsp_gather_range on a HIP stream (argument checks, then one launch).
zsp_status gather_range(zsp_plan* P, int32_t first_param, int32_t n_params, zsp_source src,
                        void* out, hipStream_t stream);

}  // namespace zsp
