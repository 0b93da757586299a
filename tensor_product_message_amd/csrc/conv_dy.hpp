// Harmonic gradient alone (gfx950): dY of the convolution's backward (FlashCart,
// arXiv 2610.06409, symbolic-VJP section) without dx and dw.
//
//   dY[e, l2 m2] = sum_c sum_p w[e,p,c] sum_{m1,m3} C_p[m1][m2][m3] x[j, l1 m1, c] G[i, l3 m3, c]
//
// The edge-vector VJP of the VJP needs this dY again after the forces were
// taken; the full backward would also stream dw out (a third of its bytes) and
// build T for v and dx.  Here one workgroup per receiver i keeps G[i] in
// registers, walks its in-edges in CSR order loading x[j] and w[e], forms the
// products x[m1] G[m3] per (l1, l3) group and contracts them with the
// coupling non-zeros, exactly as the backward does for dY (same operations in
// the same order, so the same bits), then sums over channels (lanes by
// fixed-order halving, waves through LDS in wave order).  No T, no LDS tables.
// Above 512 channels two channel tiles add their partial sums into a zeroed
// dY (two addends onto zero: the same bits in either order).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace ctp {
namespace conv {

constexpr int kDyMaxThreads = 512;   // channels of one tile

// dya[l2 m2] += sum_p w_p B_p[m2], B_p[m2] = sum C_p[m1][m2][m3] x[m1] g[m3],
// grouped as the backward's groups (paths reading one block of G).
template <class S>
__device__ __forceinline__ void edge_dy(const float (&xv)[S::D1], const float (&gv)[S::DO], const float (&wv)[S::P],
                                        float (&dya)[16]) {
    static_for<S::NG>([&](auto gI) __attribute__((always_inline)) {
        constexpr PathGroup pp = S::groups[decltype(gI)::value];
        constexpr int n1 = 2 * pp.l1 + 1, n3 = 2 * pp.l3 + 1;
        constexpr int o1 = pp.l1 * pp.l1, o3 = pp.o3;
        float B[kMaxL + 1][2 * kMaxL + 1];
        static_for<n1>([&](auto aI) __attribute__((always_inline)) {
            constexpr int a = decltype(aI)::value;
            float p3[n3];
#pragma unroll
            for (int b = 0; b < n3; ++b) p3[b] = xv[o1 + a] * gv[o3 + b];
            static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
                constexpr int kk = decltype(kI)::value;
                constexpr int p = pp.p[kk];
                constexpr int z0 = nz_m1_begin<S>(p, a), z1 = nz_m1_begin<S>(p, a + 1);
                static_for<z1 - z0>([&](auto zI) __attribute__((always_inline)) {
                    constexpr int n = z0 + decltype(zI)::value;
                    constexpr CgNz nzv = S::nz[n];
                    if constexpr (nz_first_m2<S>(n))
                        B[kk][nzv.m2] = nzv.c * p3[nzv.m3];
                    else
                        B[kk][nzv.m2] = __builtin_fmaf(nzv.c, p3[nzv.m3], B[kk][nzv.m2]);
                });
            });
            if constexpr (S::P >= 20) __builtin_amdgcn_sched_barrier(0);
        });
        static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
            constexpr int kk = decltype(kI)::value;
            constexpr int p = pp.p[kk];
            constexpr int n2 = 2 * S::paths[p].l2 + 1, o2 = S::paths[p].l2 * S::paths[p].l2;
#pragma unroll
            for (int b = 0; b < n2; ++b) dya[o2 + b] = __builtin_fmaf(wv[p], B[kk][b], dya[o2 + b]);
        });
        __builtin_amdgcn_sched_barrier(0);
    });
}

template <int Aux>
__device__ __forceinline__ float dy_ld(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, Aux));
}

template <class S>
__global__ void __launch_bounds__(kDyMaxThreads)
k_bwd_dy(int C, const float* __restrict__ G, const float* __restrict__ x, const float* __restrict__ w,
         const int* __restrict__ row_ptr, const int* __restrict__ senders, float* __restrict__ dy, int dy_atomic) {
    constexpr int D1 = S::D1, D2 = S::D2, DO = S::DO, P = S::P;
    __shared__ float sRed[kDyMaxThreads / 64][16];

    const int i = blockIdx.x;
    const int k0 = row_ptr[i], k1 = row_ptr[i + 1];
    if (k0 >= k1) return;   // the whole workgroup: no in-edges
    const int tid = threadIdx.x, nth = blockDim.x, nwaves = nth >> 6, ln = tid & 63;
    const int c0 = blockIdx.y * nth + tid;
    const uint32_t voff = opaque_lane(c0 < C ? (uint32_t)c0 * 4u : kOffLane);   // no channel: loads 0

    float gv[DO], xv[D1], wv[P];
    {
        const rsrc_t gr = make_row(G + (long)i * DO * C, (long)DO * C);
        const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
#pragma unroll
        for (int d = 0; d < DO; ++d) gv[d] = dy_ld<kStream>(gr, voff, (uint32_t)d * c4);
        const rsrc_t xr = make_row(x + (long)senders[k0] * D1 * C, (long)D1 * C);
        const rsrc_t wr = make_row(w + (long)k0 * P * C, (long)P * C);
#pragma unroll
        for (int d = 0; d < D1; ++d) xv[d] = dy_ld<kCached>(xr, voff, (uint32_t)d * c4);
#pragma unroll
        for (int p = 0; p < P; ++p) wv[p] = dy_ld<kStream>(wr, voff, (uint32_t)p * c4);
    }
    for (int k = k0; k < k1; ++k) {
        const bool has_next = k + 1 < k1;
        float dya[16];
#pragma unroll
        for (int d = 0; d < 16; ++d) dya[d] = 0.0f;
        edge_dy<S>(xv, gv, wv, dya);
#pragma unroll
        for (int d = 0; d < D2; ++d) pin_f32(dya[d]);
        // the next edge's rows into the registers just used (zeros after the last)
        {
            const long kn = has_next ? k + 1 : k;
            const uint32_t nvoff = has_next ? voff : kOffLane;
            const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
            const rsrc_t xr = make_row(x + (long)senders[kn] * D1 * C, (long)D1 * C);
            const rsrc_t wr = make_row(w + kn * P * C, (long)P * C);
#pragma unroll
            for (int d = 0; d < D1; ++d) xv[d] = dy_ld<kCached>(xr, nvoff, (uint32_t)d * c4);
#pragma unroll
            for (int p = 0; p < P; ++p) wv[p] = dy_ld<kStream>(wr, nvoff, (uint32_t)p * c4);
        }
        __builtin_amdgcn_sched_barrier(0);
        const float r = wave_sum16(dya, ln);
        if (sum16_holder(ln)) sRed[tid >> 6][sum16_index(ln)] = r;
        __syncthreads();
        if (tid < D2) {
            float tot = sRed[0][tid];
            for (int q = 1; q < nwaves; ++q) tot += sRed[q][tid];
            if (dy_atomic) unsafeAtomicAdd(dy + (long)k * D2 + tid, tot);
            else dy[(long)k * D2 + tid] = tot;
        }
        __syncthreads();
    }
}

template <class S>
hipError_t dy_launch(const LaunchArgs& a, hipStream_t st) {
    const int tiles = (a.C + kDyMaxThreads - 1) / kDyMaxThreads;
    const int waves = ((a.C + tiles - 1) / tiles + 63) / 64;
    if (tiles > 1) hipLaunchKernelGGL(k_fill0, dim3(1024), dim3(256), 0, st, a.dy, (long)a.n_edges * S::D2);
    hipLaunchKernelGGL((k_bwd_dy<S>), dim3(a.n_nodes, tiles), dim3(64 * waves), 0, st, a.C, a.grad, a.x, a.w,
                       a.row_ptr, a.senders, a.dy, (int)(tiles > 1));
    return hipGetLastError();
}

}  // namespace conv
}  // namespace ctp
