// nb_api.hpp -- internal interface between the C ABI's argument checking and
// planning (api.cpp) and entry points that supply the workspace themselves.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#include "norm_bwd.h"

namespace nb {

// Supplies a call's workspace once its size is known and every other
// argument has been checked, before anything is launched: sets *ws and
// *ws_bytes and returns NORM_BWD_OK, or returns a status (recorded with
// report_error) and the call launches nothing. `stream` is the call's stream.
typedef int (*WorkspaceProvider)(size_t need, void** ws, size_t* ws_bytes, void* stream);

// norm_bwd_ex, with the workspace from `provider` instead of the caller's
// args->workspace when provider is non-NULL.
int run_ex(const norm_bwd_args_t* a, WorkspaceProvider provider);

// Record a failure for norm_bwd_last_error (and NORM_BWD_LOG); returns status.
int report_error(int status, const char* what);
int report_hip_error(hipError_t e, const char* where);

}  // namespace nb
