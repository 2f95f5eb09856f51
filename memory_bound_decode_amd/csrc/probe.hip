// Streaming-read probe: the bandwidth a plain read of device memory reaches on this
// part, the practical ceiling of every weight-streaming kernel in the library (a
// decode step's time is the weight bytes it reads, [Bolt] background).  Not a step
// of the method; bench.py uses it to report each kernel against nominal HBM peak
// and against this measured ceiling.
#include <hip/hip_runtime.h>

#include "hip_check.h"
#include "mbd_internal.h"

namespace mbd {
namespace probe {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int UNROLL = 8;   // 16-byte loads in flight per thread before they are consumed

// Every thread reads UNROLL 16-byte words per round, rounds strided by the grid,
// and folds them into one word; a thread writes its fold only when it is the
// (never produced) marker value, so the loads cannot be removed yet nothing is
// stored in practice.
__global__ void stream_read_kernel(const u32x4_t* __restrict__ src, uint64_t n16, uint32_t* __restrict__ sink) {
    const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
    uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
        u32x4_t v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4_t v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace probe
}  // namespace mbd

using namespace mbd;

extern "C" {

mbd_status mbd_probe_stream_read(const void* src, uint64_t bytes, uint32_t* sink, int32_t blocks, int32_t threads,
                                 void* stream) {
    hip_clear();
    if (!src || !sink) return fail(MBD_EINVAL, "NULL argument");
    if ((reinterpret_cast<uintptr_t>(src) & 15) || bytes % 16) return fail(MBD_EALIGN, "src and bytes must be 16-byte aligned");
    if (blocks < 1 || threads < 64 || threads > 1024 || threads % 64) return fail(MBD_ESHAPE, "bad launch shape");
    hipLaunchKernelGGL(probe::stream_read_kernel, dim3(unsigned(blocks)), dim3(unsigned(threads)), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<const probe::u32x4_t*>(src), bytes / 16, sink);
    return hip_check("stream read probe launch");
}

}  // extern "C"
