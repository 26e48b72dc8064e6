// Streaming-read probe: the HBM read rate a plain kernel reaches on this
// GPU, measured next to the attention kernels as the practical ceiling of a
// scan over resident memory.  Not part of the method: it reads a buffer
// once with 16-byte loads and reduces it to one word per thread so that the
// loads cannot be removed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rbq_probe.h"

namespace {

typedef uint32_t pu32x4 __attribute__((ext_vector_type(4)));

// Each thread reads U 16-byte chunks per round, `stride` chunks apart (the
// whole grid's width), all issued before any is used; rounds advance by U
// strides.  Chunks past n16 are skipped.
template <int U, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const pu32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        pu32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const pu32x4 v = src[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" int rbq_probe_stream_read(const void* src, size_t bytes, uint32_t* sink,
                                     int32_t blocks, int32_t unroll, int32_t nontemporal,
                                     void* stream) {
    if (src == nullptr || sink == nullptr || blocks <= 0 || (bytes & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(src) & 15) != 0)
        return -1;
    const size_t n16 = bytes / 16;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)blocks), block(256);
    const pu32x4* p = reinterpret_cast<const pu32x4*>(src);
#define RBQ_PROBE_CASE(U)                                                                        \
    case U:                                                                                      \
        if (nontemporal) hipLaunchKernelGGL((stream_read_kernel<U, true>), grid, block, 0, s, p, n16, sink); \
        else hipLaunchKernelGGL((stream_read_kernel<U, false>), grid, block, 0, s, p, n16, sink); \
        break;
    switch (unroll) {
        RBQ_PROBE_CASE(1)
        RBQ_PROBE_CASE(2)
        RBQ_PROBE_CASE(4)
        RBQ_PROBE_CASE(8)
        RBQ_PROBE_CASE(16)
        default: return -1;
    }
#undef RBQ_PROBE_CASE
    return hipGetLastError() == hipSuccess ? 0 : -6;
}
