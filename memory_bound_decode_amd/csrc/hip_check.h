// HIP error attribution shared by the launchers of every HIP source.
#pragma once

#include <hip/hip_runtime.h>

#include "mbd_internal.h"

namespace mbd {

// hipGetLastError() returns (and clears) the first error recorded on the thread
// since it was last called, which may come from an earlier, unrelated HIP call
// (the caller's own work, or a previous library call).  Every device entry point
// clears that state first, so the check after its launches reports only what
// they caused.
inline void hip_clear() { (void)hipGetLastError(); }

inline mbd_status hip_check(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MBD_EHIP, "%s: %s", what, hipGetErrorString(e));
    return MBD_OK;
}

}  // namespace mbd
