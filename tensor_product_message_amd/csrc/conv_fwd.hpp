// Forward kernels of the fused equivariant convolution tensor product (gfx950).
//
// Operation (e3j, arXiv 2609.35099, abstract and Table 1: message-passing
// convolution without materialised messages; FlashCart, arXiv 2610.06409,
// section 4: receiver-sorted convolution):
//
//   out[i, l3 m3, c] = sum_{e = j->i} sum_{p: l3_p = l3} w[e,p,c]
//                      sum_{m1} T_{p,e}[m1][m3] x[j, l1 m1, c],
//   T_{p,e}[m1][m3]  = sum_{m2} C_p[m1][m2][m3] Y[e, l2 m2].
//
// Layout: x[N][D1][C], out[N][DO][C], w[E][P][C] (channel fastest, so every
// wave-wide access is a contiguous run of C floats), Y[E][D2] or vec[E][3];
// edges in CSR-by-receiver order.  S = Spec<L1, L2, L3, V> fixes the degrees
// of x, Y and out and the path variant at compile time.
//
// Mapping: one workgroup per receiver and channel tile, one channel per lane.
// Per edge, T_{p,e} is shared by every channel: the workgroup builds it once
// in LDS (lane-parallel, <= 2 terms per entry) and every lane reads it by
// broadcast.  The path loops are unrolled over the constexpr tables, so each
// coupling coefficient is an instruction constant and every partial sum lives
// in registers.
//
// Determinism: the CSR forward sums edges and paths in a fixed order.  Small
// grids (SPLIT) divide each edge list between two workgroups whose two partial
// sums meet by fp32 atomics onto zero, which gives the same bits in either
// order.  The edge-parallel atomic forward exists only as a comparison.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace ctp {
namespace conv {

constexpr int kMaxThreads = 256;   // forward workgroups

// ------------------------------------------------------------ per-edge building blocks

// acc[l3 m3] += sum_p w_p * (T_p^T x[l1])[m3] for one edge and CPL channels.
template <class S, int CPL>
__device__ __forceinline__ void edge_forward(float (&acc)[S::DO][CPL], const float (&xv)[S::D1][CPL],
                                             const float (&wv)[S::P][CPL], const float* sT) {
    static_for<S::P>([&](auto pI) __attribute__((always_inline)) {
        constexpr int p = decltype(pI)::value;
        constexpr PathL q = S::paths[p];
        constexpr int n1 = 2 * q.l1 + 1, n3 = 2 * q.l3 + 1;
        constexpr int o1 = q.l1 * q.l1, o3 = S::out_off[p];   // o3: first output component of path p
        constexpr int t0 = S::slot_begin[p], t1 = S::slot_begin[p + 1];
        if constexpr (n1 <= n3) {
            // scale x by w first: n1 products, then one FMA per slot
            float xs[n1][CPL];
#pragma unroll
            for (int a = 0; a < n1; ++a)
#pragma unroll
                for (int c = 0; c < CPL; ++c) xs[a][c] = wv[p][c] * xv[o1 + a][c];
            static_for<t1 - t0>([&](auto tI) __attribute__((always_inline)) {
                constexpr int t = t0 + decltype(tI)::value;
                constexpr TSlot s = S::slots[t];
                const float tv = slot_value<t>(sT);
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    acc[o3 + s.m3][c] = __builtin_fmaf(tv, xs[s.m1][c], acc[o3 + s.m3][c]);
            });
        } else {
            // contract T with x first: one FMA per slot, then n3 FMAs with w
            float u[n3][CPL];
            static_for<t1 - t0>([&](auto tI) __attribute__((always_inline)) {
                constexpr int t = t0 + decltype(tI)::value;
                constexpr TSlot s = S::slots[t];
                const float tv = slot_value<t>(sT);
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    if constexpr (first_m3<S>(t))
                        u[s.m3][c] = tv * xv[o1 + s.m1][c];
                    else
                        u[s.m3][c] = __builtin_fmaf(tv, xv[o1 + s.m1][c], u[s.m3][c]);
                }
            });
#pragma unroll
            for (int k = 0; k < n3; ++k)
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[o3 + k][c] = __builtin_fmaf(wv[p][c], u[k][c], acc[o3 + k][c]);
        }
    });
}

template <class S, int CPL>
__device__ __forceinline__ void load_edge_operands(float (&xv)[S::D1][CPL], float (&wv)[S::P][CPL],
                                                   const float* __restrict__ x, const float* __restrict__ w,
                                                   long j, long e, int C, uint32_t voff) {
    const rsrc_t xr = make_row(x + j * S::D1 * C, (long)S::D1 * C);
    const rsrc_t wr = make_row(w + e * S::P * C, (long)S::P * C);
    const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
#pragma unroll
    for (int d = 0; d < S::D1; ++d) bload<CPL>(xr, voff, (uint32_t)d * c4, xv[d]);
#pragma unroll
    for (int p = 0; p < S::P; ++p) bload<CPL, kStream>(wr, voff, (uint32_t)p * c4, wv[p]);
}

// ------------------------------------------------------------ K1: CSR forward (deterministic)
//
// Rotating prefetch through a window of R w registers (R divides P): path p
// reads slot p % R, and right after it has consumed w[e, p] that slot receives
// the row R paths ahead, w[e, p + R] or, past the edge's last path,
// w[e+1, p + R - P].  With R = P every load has a whole edge of arithmetic to
// arrive; with R = P/2 half an edge, for half the registers (at lmax 3:
// 77 instead of 110 VGPRs, six waves per SIMD instead of four, measured 2%
// faster; a window of two paths was 15% slower).  Each x block is refilled
// with the next sender's row after its last use.  The next edge's Y is
// loaded early and its T is built into the other LDS buffer after compute.

// Window of w registers: half the paths when there are enough of them (P even
// and at least 32) for half an edge of arithmetic to cover a load, else all.
template <class S>
constexpr int fwd_window() {
    return (S::P >= 32 && S::P % 2 == 0) ? S::P / 2 : S::P;
}

template <class S>
constexpr bool last_path_of_l1(int p) {
    return p + 1 == S::P || S::paths[p + 1].l1 != S::paths[p].l1;
}

// Path loop of one edge with refills for the next edge.
// cw: the current edge's w row; nx, nw: the next edge's x and w rows (nvoff:
// out of range after the last edge, so those loads return 0).
template <class S, int CPL>
__device__ __forceinline__ void edge_forward_refill(float (&acc)[S::DO][CPL], float (&xv)[S::D1][CPL],
                                                    float (&wv)[fwd_window<S>()][CPL], const float* sT,
                                                    rsrc_t cw, uint32_t voff, rsrc_t nx, rsrc_t nw,
                                                    uint32_t nvoff, int C) {
    constexpr int R = fwd_window<S>();
    static_assert(S::P % R == 0, "the window must divide the path count");
    static_for<S::P>([&](auto pI) __attribute__((always_inline)) {
        constexpr int p = decltype(pI)::value;
        constexpr PathL q = S::paths[p];
        constexpr int n1 = 2 * q.l1 + 1, n3 = 2 * q.l3 + 1;
        constexpr int o1 = q.l1 * q.l1, o3 = S::out_off[p];   // o3: first output component of path p
        constexpr int t0 = S::slot_begin[p], t1 = S::slot_begin[p + 1];
        if constexpr (n1 <= n3) {
            float xs[n1][CPL];
#pragma unroll
            for (int a = 0; a < n1; ++a)
#pragma unroll
                for (int c = 0; c < CPL; ++c) xs[a][c] = wv[p % R][c] * xv[o1 + a][c];
            static_for<t1 - t0>([&](auto tI) __attribute__((always_inline)) {
                constexpr int t = t0 + decltype(tI)::value;
                constexpr TSlot s = S::slots[t];
                const float tv = slot_value<t>(sT);
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    acc[o3 + s.m3][c] = __builtin_fmaf(tv, xs[s.m1][c], acc[o3 + s.m3][c]);
            });
        } else {
            float u[n3][CPL];
            static_for<t1 - t0>([&](auto tI) __attribute__((always_inline)) {
                constexpr int t = t0 + decltype(tI)::value;
                constexpr TSlot s = S::slots[t];
                const float tv = slot_value<t>(sT);
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    if constexpr (first_m3<S>(t))
                        u[s.m3][c] = tv * xv[o1 + s.m1][c];
                    else
                        u[s.m3][c] = __builtin_fmaf(tv, xv[o1 + s.m1][c], u[s.m3][c]);
                }
            });
#pragma unroll
            for (int k = 0; k < n3; ++k)
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[o3 + k][c] = __builtin_fmaf(wv[p % R][c], u[k][c], acc[o3 + k][c]);
        }
        // keep this path's arithmetic here (pure code would otherwise sink to the loop latch)
#pragma unroll
        for (int k = 0; k < n3; ++k)
#pragma unroll
            for (int c = 0; c < CPL; ++c) pin_f32(acc[o3 + k][c]);
        // refills: w R paths ahead (this edge's row, else the next edge's), x
        // blocks for the next edge after their last use
        const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
        if constexpr (p + R < S::P)
            bload<CPL, kStream>(cw, voff, (uint32_t)(p + R) * c4, wv[p % R]);
        else
            bload<CPL, kStream>(nw, nvoff, (uint32_t)(p + R - S::P) * c4, wv[p % R]);
        if constexpr (last_path_of_l1<S>(p)) {
#pragma unroll
            for (int a = 0; a < n1; ++a) bload<CPL>(nx, nvoff, (uint32_t)(o1 + a) * c4, xv[o1 + a]);
        }
        // nothing but LDS reads (the next path's T entries) may move across
        __builtin_amdgcn_sched_barrier(0x100);
    });
}

// SPLIT (small grids): blockIdx.z picks one half of the row's edges, and the
// two halves add their sums into a zeroed out with fp32 atomics.  With exactly
// two addends onto zero the result is the same in either order, so the
// output stays bitwise reproducible.
template <class S, int CPL, bool VEC, bool SPLIT>
__global__ void __launch_bounds__(kMaxThreads) __attribute__((amdgpu_waves_per_eu(1, 8)))
k_fwd_csr(int C, const float* __restrict__ x, const float* __restrict__ yv, const float* __restrict__ w,
          const int* __restrict__ row_ptr, const int* __restrict__ senders, float* __restrict__ out) {
    constexpr int D1 = S::D1, D2 = S::D2, D3 = S::DO, P = S::P, NT = S::NT, NTP = (NT + 3) & ~3;
    __shared__ __attribute__((aligned(16))) float sT[2][NTP];
    __shared__ float sY[2][16];
    __shared__ SlotDev sTab[NT];
    __shared__ ShCoef sSh[VEC ? 16 : 1];   // harmonic coefficients, read per edge from LDS

    const int i = blockIdx.x;
    const int tid = threadIdx.x, nth = blockDim.x;
    // lane owns channels c0 .. c0 + CPL - 1 (a wave covers 64 * CPL channels)
    const int c0 = blockIdx.y * nth * CPL + (tid >> 6) * 64 * CPL + (tid & 63) * CPL;
    const uint32_t voff = opaque_lane(c0 < C ? (uint32_t)c0 * 4u : kOffLane);

    float acc[D3][CPL];
#pragma unroll
    for (int d = 0; d < D3; ++d)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[d][c] = 0.0f;

    int e0 = row_ptr[i], e1 = row_ptr[i + 1];
    if constexpr (SPLIT) {
        const int mid = e0 + (e1 - e0 + 1) / 2;
        if (blockIdx.z == 0) e1 = mid; else e0 = mid;
    }
    if (e0 < e1) {
        {
            const SlotDev* tab = slot_tab<S>();
            for (int t = tid; t < NT; t += nth) sTab[t] = tab[t];
            if constexpr (VEC)
                if (tid < 16) sSh[tid] = sh_tab().k[tid];
        }
        constexpr int R = fwd_window<S>();
        float xv[D1][CPL], wv[R][CPL];
        {
            // the first edge's x row and the first R paths of its w row
            const rsrc_t xr = make_row(x + (long)senders[e0] * D1 * C, (long)D1 * C);
            const rsrc_t wr = make_row(w + (long)e0 * P * C, (long)P * C);
            const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
#pragma unroll
            for (int d = 0; d < D1; ++d) bload<CPL>(xr, voff, (uint32_t)d * c4, xv[d]);
#pragma unroll
            for (int p = 0; p < R; ++p) bload<CPL, kStream>(wr, voff, (uint32_t)p * c4, wv[p]);
        }
        const float y0 = sh_value<D2, VEC>(yv, e0, tid);
        if (tid < D2) sY[0][tid] = y0;
        __syncthreads();
        build_T_lds<S>(sT[0], sY[0], sTab, tid, nth);
        __syncthreads();
        for (int e = e0; e < e1; ++e) {
            const int buf = (e - e0) & 1;
            const bool has_next = e + 1 < e1;
            const long en = has_next ? e + 1 : e;
            const long jn = senders[en];
            const rsrc_t nx = make_row(x + jn * D1 * C, (long)D1 * C);
            const rsrc_t nw = make_row(w + en * P * C, (long)P * C);
            const uint32_t nvoff = has_next ? voff : kOffLane;
            float ynext;
            if constexpr (VEC) {
                const float* vp = yv + 3 * en;
                ynext = tid < D2 ? sh_component_c(tid, sSh[tid < D2 ? tid : 0], vp[0], vp[1], vp[2]) : 0.0f;
            } else {
                ynext = sh_value<D2, VEC>(yv, en, tid);
            }
            const rsrc_t cw = make_row(w + (long)e * P * C, (long)P * C);
            edge_forward_refill<S, CPL>(acc, xv, wv, sT[buf], cw, voff, nx, nw, nvoff, C);
            if (has_next) {
                if (tid < D2) sY[buf ^ 1][tid] = ynext;
                __syncthreads();
                build_T_lds<S>(sT[buf ^ 1], sY[buf ^ 1], sTab, tid, nth);
                __syncthreads();
            }
        }
    }
    if constexpr (SPLIT) {
        if (e0 < e1 && c0 < C) {
            float* o = out + (long)i * D3 * C + c0;
#pragma unroll
            for (int d = 0; d < D3; ++d)
#pragma unroll
                for (int c = 0; c < CPL; ++c) unsafeAtomicAdd(o + (long)d * C + c, acc[d][c]);
        }
    } else {
        const rsrc_t orow = make_row(out + (long)i * D3 * C, (long)D3 * C);
#pragma unroll
        for (int d = 0; d < D3; ++d) bstore<CPL, kStream>(orow, voff, (uint32_t)(d * C * 4), acc[d]);
    }
}

// ------------------------------------------------------------ K2: edge-parallel atomic forward (comparison)

template <class S, int CPL, bool VEC>
__global__ void __launch_bounds__(kMaxThreads)
k_fwd_atomic(int n_nodes, int C, const float* __restrict__ x, const float* __restrict__ yv,
             const float* __restrict__ w, const int* __restrict__ row_ptr, const int* __restrict__ senders,
             float* __restrict__ out) {
    constexpr int D2 = S::D2, D3 = S::DO, NT = S::NT, NTP = (NT + 3) & ~3;
    __shared__ __attribute__((aligned(16))) float sT[NTP];
    __shared__ float sY[16];

    const long e = blockIdx.x;
    const int tid = threadIdx.x, nth = blockDim.x;
    const int c0 = blockIdx.y * nth * CPL + (tid >> 6) * 64 * CPL + (tid & 63) * CPL;
    const bool active = c0 < C;
    const uint32_t voff = opaque_lane(active ? (uint32_t)c0 * 4u : kOffLane);

    // receiver of edge e: last i with row_ptr[i] <= e
    int lo = 0, hi = n_nodes;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (row_ptr[mid] <= e) lo = mid; else hi = mid;
    }
    const int i = lo;

    float xv[S::D1][CPL], wv[S::P][CPL];
    load_edge_operands<S, CPL>(xv, wv, x, w, senders[e], e, C, voff);
    {
        const float y0 = sh_value<D2, VEC>(yv, e, tid);
        if (tid < D2) sY[tid] = y0;
    }
    __syncthreads();
    build_T_lds<S>(sT, sY, slot_tab<S>(), tid, nth);
    __syncthreads();
    float acc[D3][CPL];
#pragma unroll
    for (int d = 0; d < D3; ++d)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[d][c] = 0.0f;
    edge_forward<S, CPL>(acc, xv, wv, sT);
    if (active) {
        float* o = out + (long)i * D3 * C + c0;
#pragma unroll
        for (int d = 0; d < D3; ++d)
#pragma unroll
            for (int c = 0; c < CPL; ++c) unsafeAtomicAdd(o + (long)d * C + c, acc[d][c]);
    }
}

// ------------------------------------------------------------ launchers

struct ChanMap {
    int waves, tiles;   // waves per workgroup, channel tiles (grid.y); one channel per lane
};

// Channels over workgroups of at most max_waves waves.  The kernels also take
// two adjacent channels per lane (CPL = 2: half the T reads per channel, twice
// the registers); that measured 1-2% slower in the CSR forward and twice as
// slow in the atomic one, so every launch uses CPL = 1.
inline ChanMap chan_map(int C, int max_waves) {
    ChanMap m{};
    const int need = (C + 63) / 64;
    m.waves = need < max_waves ? need : max_waves;
    m.tiles = (need + m.waves - 1) / m.waves;
    return m;
}

// Grids with fewer waves than 4 per SIMD split every edge list in two (SPLIT).
constexpr long kSplitBelowWaves = 4L * 1024;

template <class S, bool SPLIT>
hipError_t fwd_csr_launch(const LaunchArgs& a, const ChanMap& m, hipStream_t st) {
    const dim3 grid(a.n_nodes, m.tiles, SPLIT ? 2 : 1), block(64 * m.waves);
    if (SPLIT) {
        const long n = (long)a.n_nodes * S::DO * a.C;
        hipLaunchKernelGGL(k_fill0, dim3(1024), dim3(256), 0, st, a.out, n);
    }
    if (a.vec_mode)
        hipLaunchKernelGGL((k_fwd_csr<S, 1, true, SPLIT>), grid, block, 0, st, a.C, a.x, a.y, a.w, a.row_ptr,
                           a.senders, a.out);
    else
        hipLaunchKernelGGL((k_fwd_csr<S, 1, false, SPLIT>), grid, block, 0, st, a.C, a.x, a.y, a.w, a.row_ptr,
                           a.senders, a.out);
    return hipGetLastError();
}

template <class S>
hipError_t fwd_launch(const LaunchArgs& a, hipStream_t st) {
    const ChanMap m = chan_map(a.C, kMaxThreads / 64);
    if (a.algo == 0) {
        if constexpr (S::V == kVariantSummed)
            if ((long)a.n_nodes * m.tiles * m.waves < kSplitBelowWaves) return fwd_csr_launch<S, true>(a, m, st);
        return fwd_csr_launch<S, false>(a, m, st);
    }
    const long n = (long)a.n_nodes * S::DO * a.C;
    hipLaunchKernelGGL(k_fill0, dim3(1024), dim3(256), 0, st, a.out, n);
    if (a.n_edges > 0) {
        const dim3 grid(a.n_edges, m.tiles), block(64 * m.waves);
        if (a.vec_mode)
            hipLaunchKernelGGL((k_fwd_atomic<S, 1, true>), grid, block, 0, st, a.n_nodes, a.C, a.x, a.y, a.w,
                               a.row_ptr, a.senders, a.out);
        else
            hipLaunchKernelGGL((k_fwd_atomic<S, 1, false>), grid, block, 0, st, a.n_nodes, a.C, a.x, a.y, a.w,
                               a.row_ptr, a.senders, a.out);
    }
    return hipGetLastError();
}

}  // namespace conv
}  // namespace ctp
