// Plain HBM streams (read, write, copy) with the cache policy of the conv
// kernels' edge streams: non-temporal, 16-byte or 4-byte accesses per lane, a
// grid-stride loop (4096 workgroups for reads, 16384 for writes and copies,
// the best of a sweep on MI355X).  They give the bandwidth this
// device actually sustains for each traffic mix, the practical ceiling next to
// the 8 TB/s data-sheet peak.  A fourth probe measures the fp32 FMA rate the
// vector ALUs sustain without packed instructions (the kernels are built
// without them), the arithmetic ceiling next to the derived VALU peak.
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

// The same three streams with 4-byte accesses per lane (one dword: 256 bytes
// per wave-wide instruction), the width of the conv kernels' one-channel-per-
// lane row accesses.  Reads and the copy keep kDwordDepth loads in flight per
// lane, as many bytes per lane as four 16-byte loads.
constexpr int kDwordDepth = 16;

__global__ void __launch_bounds__(kProbeThreads) k_stream_read1(const float* __restrict__ a, float* __restrict__ sink,
                                                                long n) {
    const long bd = blockDim.x;
    const long st = (long)gridDim.x * bd * kDwordDepth;
    float s[kDwordDepth];
#pragma unroll
    for (int u = 0; u < kDwordDepth; ++u) s[u] = 0.0f;
    long i = (long)blockIdx.x * bd * kDwordDepth + threadIdx.x;
    for (; i + (kDwordDepth - 1) * bd < n; i += st) {
#pragma unroll
        for (int u = 0; u < kDwordDepth; ++u) s[u] += __builtin_nontemporal_load(a + i + u * bd);
    }
    for (; i < n; i += bd) s[0] += __builtin_nontemporal_load(a + i);
    float t = 0.0f;
#pragma unroll
    for (int u = 0; u < kDwordDepth; ++u) t += s[u];
    if (t != t && threadIdx.x == 0) sink[0] = t;
}

__global__ void __launch_bounds__(kProbeThreads) k_stream_write1(float* __restrict__ b, long n) {
    const long st = (long)gridDim.x * blockDim.x;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += st) __builtin_nontemporal_store(1.0f, b + i);
}

__global__ void __launch_bounds__(kProbeThreads) k_stream_copy1(const float* __restrict__ a, float* __restrict__ b,
                                                                long n) {
    const long bd = blockDim.x;
    const long st = (long)gridDim.x * bd * kDwordDepth;
    long i = (long)blockIdx.x * bd * kDwordDepth + threadIdx.x;
    for (; i + (kDwordDepth - 1) * bd < n; i += st) {
        float v[kDwordDepth];
#pragma unroll
        for (int u = 0; u < kDwordDepth; ++u) v[u] = __builtin_nontemporal_load(a + i + u * bd);
#pragma unroll
        for (int u = 0; u < kDwordDepth; ++u) __builtin_nontemporal_store(v[u], b + i + u * bd);
    }
    for (; i < n; i += bd) __builtin_nontemporal_store(__builtin_nontemporal_load(a + i), b + i);
}

// Eight independent FMA chains per lane (enough to cover the FMA latency),
// non-packed fp32; the result is consumed by a store that no finite value
// takes.  Every workgroup runs the same work: kValuBlocks x 256 threads x
// iters x 8 FMAs.
constexpr int kValuBlocks = 2048;    // 8 waves per SIMD on 256 CUs
constexpr int kValuChains = 8;

__global__ void __launch_bounds__(kProbeThreads) k_valu_fma(float* __restrict__ sink, long iters, float a) {
    float acc[kValuChains];
#pragma unroll
    for (int k = 0; k < kValuChains; ++k) acc[k] = 1e-3f * threadIdx.x + k;
    for (long i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kValuChains; ++k) acc[k] = __builtin_fmaf(acc[k], a, 0.5f);
    }
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < kValuChains; ++k) t += acc[k];
    if (t != t && threadIdx.x == 0) sink[0] = t;
}

}  // namespace

hipError_t launch_valu_probe(long iters, float* dst, hipStream_t st) {
    if (iters == 0) return hipSuccess;
    hipLaunchKernelGGL(k_valu_fma, dim3(kValuBlocks), dim3(kProbeThreads), 0, st, dst, iters, 0.999f);
    return hipGetLastError();
}

long valu_probe_fmas(long iters) { return (long)kValuBlocks * kProbeThreads * kValuChains * iters; }

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
        case 3: hipLaunchKernelGGL(k_stream_read1, rgrid, block, 0, st, src, dst, n_floats); break;
        case 4: hipLaunchKernelGGL(k_stream_write1, wgrid, block, 0, st, dst, n_floats); break;
        case 5: hipLaunchKernelGGL(k_stream_copy1, wgrid, block, 0, st, src, dst, n_floats); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ctp
