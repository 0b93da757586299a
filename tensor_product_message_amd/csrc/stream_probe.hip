// Plain HBM streams (read, write, copy) with the access shape and cache policy
// of the conv kernels' edge streams: 16-byte accesses, non-temporal, a
// grid-stride loop (4096 workgroups for reads, 16384 for writes and copies,
// the best of a sweep on MI355X).  They give the bandwidth this
// device actually sustains for each traffic mix, the practical ceiling next to
// the 8 TB/s data-sheet peak.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace ctp {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kReadBlocks = 4096;
constexpr int kWriteBlocks = 16384;

__global__ void __launch_bounds__(kProbeThreads) k_stream_read(const f4* __restrict__ a, float* __restrict__ sink,
                                                               long n4) {
    const long st = (long)gridDim.x * blockDim.x;
    f4 s = {0.0f, 0.0f, 0.0f, 0.0f};
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += st) s += __builtin_nontemporal_load(a + i);
    // the sum is consumed by a store that no finite input takes, so the loads stay
    const float t = s.x + s.y + s.z + s.w;
    if (t != t && threadIdx.x == 0) sink[0] = t;
}

__global__ void __launch_bounds__(kProbeThreads) k_stream_write(f4* __restrict__ b, long n4) {
    const long st = (long)gridDim.x * blockDim.x;
    const f4 v = {1.0f, 2.0f, 3.0f, 4.0f};
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += st) __builtin_nontemporal_store(v, b + i);
}

// four 16-byte loads in flight per lane before the stores
__global__ void __launch_bounds__(kProbeThreads) k_stream_copy(const f4* __restrict__ a, f4* __restrict__ b,
                                                               long n4) {
    const long bd = blockDim.x;
    const long st = (long)gridDim.x * bd * 4;
    long i = (long)blockIdx.x * bd * 4 + threadIdx.x;
    for (; i + 3 * bd < n4; i += st) {
        f4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(a + i + u * bd);
#pragma unroll
        for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], b + i + u * bd);
    }
    for (; i < n4; i += bd) __builtin_nontemporal_store(__builtin_nontemporal_load(a + i), b + i);
}

}  // namespace

hipError_t launch_stream_probe(int kind, const float* src, float* dst, long n_floats, hipStream_t st) {
    const long n4 = n_floats / 4;
    if (n4 == 0) return hipSuccess;
    const dim3 rgrid(kReadBlocks), wgrid(kWriteBlocks), block(kProbeThreads);
    switch (kind) {
        case 0: hipLaunchKernelGGL(k_stream_read, rgrid, block, 0, st, reinterpret_cast<const f4*>(src), dst, n4); break;
        case 1: hipLaunchKernelGGL(k_stream_write, wgrid, block, 0, st, reinterpret_cast<f4*>(dst), n4); break;
        case 2:
            hipLaunchKernelGGL(k_stream_copy, wgrid, block, 0, st, reinterpret_cast<const f4*>(src),
                               reinterpret_cast<f4*>(dst), n4);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ctp
