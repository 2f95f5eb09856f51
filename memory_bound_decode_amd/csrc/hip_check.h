// HIP error attribution shared by the launchers of every HIP source.
#pragma once

#include <atomic>

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

// Raise a kernel's dynamic LDS limit once per process (idempotent, so a race
// between first calls only repeats the call); done holds the limit set so far.
inline mbd_status lds_limit(const void* kern, std::atomic<int>& done, size_t bytes, const char* what) {
    if (done.load(std::memory_order_acquire) >= int(bytes)) return MBD_OK;
    if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes)) != hipSuccess)
        return fail(MBD_EHIP, "cannot raise the %s LDS limit to %zu bytes", what, bytes);
    done.store(int(bytes), std::memory_order_release);
    return MBD_OK;
}

// The wave's LDS stores become visible to its other lanes' later loads.
__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace mbd
