// HIP kernels of the fused equivariant convolution tensor product (gfx950).
//
// Operation (e3j, arXiv 2609.35099, abstract and Table 1: message-passing
// convolution without materialised messages; FlashCart, arXiv 2610.06409,
// receiver-sorted convolution and its VJP):
//
//   out[i, l3 m3, c] = sum_{e = j->i} sum_{p: l3_p = l3} w[e,p,c]
//                      sum_{m1} T_{p,e}[m1][m3] x[j, l1 m1, c],
//   T_{p,e}[m1][m3]  = sum_{m2} C_p[m1][m2][m3] Y[e, l2 m2].
//
// Layout: x[N][D1][C], out[N][D3][C], w[E][P][C] (channel fastest, so every
// wave-wide access is a contiguous run of C floats), Y[E][D2] or vec[E][3];
// edges in CSR-by-receiver order.
//
// Mapping: one workgroup per receiver (forward) or sender (backward) and per
// channel tile; a lane owns CPL consecutive channels (CPL = 1 or 2), so every
// wave-wide access covers 64 * CPL contiguous floats with one dword or dwordx2
// per lane.  Per edge, T_{p,e} is
// shared by every channel: the workgroup builds it once in LDS (lane-parallel,
// <= 2 terms per entry) and every lane then reads it by broadcast.  The path
// loops are unrolled at compile time over the constexpr tables, so each
// coupling coefficient is an instruction constant and every partial sum lives
// in registers.  The path variant V (all paths summed per l3, or MACE's
// natural-parity paths with one output slot each) is a template parameter.
//
// Determinism: the CSR forward and the sender-sorted backward sum edges and
// paths in a fixed order.  Small grids (SPLIT) divide each edge list between
// two workgroups whose two partial sums meet by fp32 atomics onto zero, which
// gives the same bits in either order.  The edge-parallel atomic forward
// exists only as a comparison.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace ctp {

__constant__ SlotTab<0> kSlot0 = make_slot_tab<0>();
__constant__ SlotTab<1> kSlot1 = make_slot_tab<1>();
__constant__ SlotTab<2> kSlot2 = make_slot_tab<2>();
__constant__ SlotTab<3> kSlot3 = make_slot_tab<3>();
__constant__ ShTab kShTab = make_sh_tab();

template <> __device__ __forceinline__ const SlotDev* slot_tab<0>() { return kSlot0.s; }
template <> __device__ __forceinline__ const SlotDev* slot_tab<1>() { return kSlot1.s; }
template <> __device__ __forceinline__ const SlotDev* slot_tab<2>() { return kSlot2.s; }
template <> __device__ __forceinline__ const SlotDev* slot_tab<3>() { return kSlot3.s; }
__constant__ SlotTab<0, kVariantSlots> kSlotM0 = make_slot_tab<0, kVariantSlots>();
__constant__ SlotTab<1, kVariantSlots> kSlotM1 = make_slot_tab<1, kVariantSlots>();
__constant__ SlotTab<2, kVariantSlots> kSlotM2 = make_slot_tab<2, kVariantSlots>();
__constant__ SlotTab<3, kVariantSlots> kSlotM3 = make_slot_tab<3, kVariantSlots>();
template <> __device__ __forceinline__ const SlotDev* slot_tab<0, kVariantSlots>() { return kSlotM0.s; }
template <> __device__ __forceinline__ const SlotDev* slot_tab<1, kVariantSlots>() { return kSlotM1.s; }
template <> __device__ __forceinline__ const SlotDev* slot_tab<2, kVariantSlots>() { return kSlotM2.s; }
template <> __device__ __forceinline__ const SlotDev* slot_tab<3, kVariantSlots>() { return kSlotM3.s; }
__device__ __forceinline__ const ShTab& sh_tab() { return kShTab; }

constexpr int kMaxThreads = 256;     // forward workgroups
constexpr int kBwdMaxThreads = 512;  // backward: all channels of one sender
#ifndef FWD_WPE
#define FWD_WPE 1
#endif
#ifndef BWD_WPE
#define BWD_WPE 3
#endif

// ------------------------------------------------------------ per-edge building blocks

// Y of edge e into sY (lanes < D2): read (Y mode) or evaluated from vec.
template <int D2, bool VEC>
__device__ __forceinline__ void stage_sh(float* sY, const float* __restrict__ yv, long e, int tid) {
    if (tid < D2) {
        if constexpr (VEC) {
            const float* v = yv + 3 * e;
            sY[tid] = sh_component(tid, v[0], v[1], v[2]);
        } else {
            sY[tid] = yv[e * D2 + tid];
        }
    }
}

// T_{p,e} for all paths into sT, lane-parallel over the slots.
template <int L, int V>
__device__ __forceinline__ void build_T(float* sT, const float* sY, int tid, int nth) {
    constexpr int NT = Spec<L, L, L, V>::NT;
    const SlotDev* tab = slot_tab<L, V>();
    for (int t = tid; t < NT; t += nth) {
        const SlotDev s = tab[t];
        sT[t] = s.c1 * sY[s.yy & 0xff] + s.c2 * sY[s.yy >> 8];
    }
}

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
// Rotating prefetch: right after path p of edge e has consumed w[e, p], the
// same registers receive w[e+1, p]; each x block is refilled with the next
// sender's row after its last use.  Every load thus has about one edge of
// arithmetic to arrive, with no second register set.  The next edge's Y is
// loaded early and its T is built into the other LDS buffer after compute.

template <class S>
constexpr bool last_path_of_l1(int p) {
    return p + 1 == S::P || S::paths[p + 1].l1 != S::paths[p].l1;
}

// Path loop of one edge with refills for the next edge.
template <class S, int CPL>
__device__ __forceinline__ void edge_forward_refill(float (&acc)[S::DO][CPL], float (&xv)[S::D1][CPL],
                                                    float (&wv)[S::P][CPL], const float* sT, rsrc_t nx,
                                                    rsrc_t nw, uint32_t nvoff, int C) {
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
        // keep this path's arithmetic here (pure code would otherwise sink to the loop latch)
#pragma unroll
        for (int k = 0; k < n3; ++k)
#pragma unroll
            for (int c = 0; c < CPL; ++c) pin_f32(acc[o3 + k][c]);
        // refills for the next edge (loads return 0 when there is none)
        const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
        bload<CPL, kStream>(nw, nvoff, (uint32_t)p * c4, wv[p]);
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
template <int L, int CPL, bool VEC, int V, bool SPLIT>
__global__ void __launch_bounds__(kMaxThreads) __attribute__((amdgpu_waves_per_eu(FWD_WPE, 8)))
k_fwd_csr(int C, const float* __restrict__ x, const float* __restrict__ yv, const float* __restrict__ w,
          const int* __restrict__ row_ptr, const int* __restrict__ senders, float* __restrict__ out) {
    using S = Spec<L, L, L, V>;
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
            const SlotDev* tab = slot_tab<L, V>();
            for (int t = tid; t < NT; t += nth) sTab[t] = tab[t];
            if constexpr (VEC)
                if (tid < 16) sSh[tid] = sh_tab().k[tid];
        }
        float xv[D1][CPL], wv[P][CPL];
        load_edge_operands<S, CPL>(xv, wv, x, w, senders[e0], e0, C, voff);
        const float y0 = sh_value<D2, VEC>(yv, e0, tid);
        if (tid < D2) sY[0][tid] = y0;
        __syncthreads();
        build_T_lds<L, V>(sT[0], sY[0], sTab, tid, nth);
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
            edge_forward_refill<S, CPL>(acc, xv, wv, sT[buf], nx, nw, nvoff, C);
            if (has_next) {
                if (tid < D2) sY[buf ^ 1][tid] = ynext;
                __syncthreads();
                build_T_lds<L, V>(sT[buf ^ 1], sY[buf ^ 1], sTab, tid, nth);
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

__global__ void k_zero(float* __restrict__ p, long n) {
    long k = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long stride = (long)gridDim.x * blockDim.x;
    for (; k < n; k += stride) p[k] = 0.0f;
}

template <int L, int CPL, bool VEC, int V>
__global__ void __launch_bounds__(kMaxThreads)
k_fwd_atomic(int n_nodes, int C, const float* __restrict__ x, const float* __restrict__ yv,
             const float* __restrict__ w, const int* __restrict__ row_ptr, const int* __restrict__ senders,
             float* __restrict__ out) {
    using S = Spec<L, L, L, V>;
    constexpr int D2 = S::D2, D3 = S::DO, NTP = (S::NT + 3) & ~3;
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
    stage_sh<D2, VEC>(sY, yv, e, tid);
    __syncthreads();
    build_T<L, V>(sT, sY, tid, nth);
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

// ------------------------------------------------------------ K3: sender-sorted backward (deterministic)
//
// For sender j and each out-edge e = j -> i (sender-sorted, stable in CSR id):
//   v_p[m1]      = sum_m3 T_p[m1][m3] G[i, l3 m3]
//   dw[e,p]      = sum_m1 x[j, l1 m1] v_p[m1]
//   dx[j, l1 m1] += w_p v_p[m1]                      (registers; stored once)
//   B_p[m2]      = sum_{m1,m3} C_p[m1][m2][m3] x[j, l1 m1] G[i, l3 m3]
//   dY[e, l2 m2] = sum_c sum_p w_p B_p[m2]           (lanes, then waves, fixed order)
// With VEC, dvec[e] = J(vec_e)^T dY[e] instead of dY.

// G row of receiver i and w row of edge e, CPL channels per lane.
template <class S, int CPL>
__device__ __forceinline__ void load_bwd_operands(float (&gv)[S::DO][CPL], float (&wv)[S::P][CPL],
                                                  const float* __restrict__ G, const float* __restrict__ w, long i,
                                                  long e, int C, uint32_t voff) {
    const rsrc_t gr = make_row(G + i * S::DO * C, (long)S::DO * C);
    const rsrc_t wr = make_row(w + e * S::P * C, (long)S::P * C);
    const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
#pragma unroll
    for (int d = 0; d < S::DO; ++d) bload<CPL>(gr, voff, (uint32_t)d * c4, gv[d]);
#pragma unroll
    for (int p = 0; p < S::P; ++p) bload<CPL, kStream>(wr, voff, (uint32_t)p * c4, wv[p]);
}

// One edge of the backward, given T = T(Y_e) in LDS, the sender's row x, the
// receiver's row g of G and the edge's row w (one channel set per lane):
//   v_p = T_p^T g,  dw[e,p] = x . v_p (stored through dwr),  dxa += w_p v_p,
//   dya[l2 m2] += sum_p w_p B_p[m2],  B_p[m2] = sum C_p[m1][m2][m3] x[m1] g[m3].
// Work is grouped by the paths that read one block of G: for each group, v_p,
// dw_p and dx for its paths, then B_p from the products x[l1 m1] g[l3 m3]
// formed m1 by m1 and shared by the group's paths.  A scheduling barrier after
// each group bounds register lifetimes.  k_bwd_sender keeps an inline copy of
// this loop: through the call the compiler's schedule for it needs 134 VGPRs
// at L=3 instead of 122, one wave fewer per SIMD.
template <int L, class S, int CPL>
__device__ __forceinline__ void edge_backward(const float* T, const float (&xv)[S::D1][CPL],
                                              const float (&gv)[S::DO][CPL], const float (&wv)[S::P][CPL],
                                              rsrc_t dwr, uint32_t voff, int C, float (&dxa)[S::D1][CPL],
                                              float (&dya)[16]) {
    static_for<S::NG>([&](auto gI) __attribute__((always_inline)) {
        constexpr PathGroup pp = S::groups[decltype(gI)::value];
        constexpr int l1 = pp.l1, l3 = pp.l3;
        constexpr int n1 = 2 * l1 + 1, n3 = 2 * l3 + 1;
        constexpr int o1 = l1 * l1, o3 = pp.o3;   // o3: the group's block of G
        // (a) v_p = T_p^T g, dw_p = x . v_p, dx += w_p v_p
        static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
            constexpr int p = pp.p[decltype(kI)::value];
            constexpr int t0 = S::slot_begin[p], t1 = S::slot_begin[p + 1];
            float v[n1][CPL];
            static_for<t1 - t0>([&](auto tI) __attribute__((always_inline)) {
                constexpr int t = t0 + decltype(tI)::value;
                constexpr TSlot s = S::slots[t];
                const float tv = slot_value<t>(T);
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    if constexpr (first_m1<S>(t))
                        v[s.m1][c] = tv * gv[o3 + s.m3][c];
                    else
                        v[s.m1][c] = __builtin_fmaf(tv, gv[o3 + s.m3][c], v[s.m1][c]);
                }
            });
            float dwv[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                dwv[c] = xv[o1][c] * v[0][c];
#pragma unroll
                for (int a = 1; a < n1; ++a) dwv[c] = __builtin_fmaf(xv[o1 + a][c], v[a][c], dwv[c]);
            }
            bstore<CPL, kStream>(dwr, voff, (uint32_t)p * opaque_u32((uint32_t)C * 4u), dwv);
#pragma unroll
            for (int a = 0; a < n1; ++a)
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    dxa[o1 + a][c] = __builtin_fmaf(wv[p][c], v[a][c], dxa[o1 + a][c]);
                    pin_f32(dxa[o1 + a][c]);
                }
            if constexpr (L >= 3) __builtin_amdgcn_sched_barrier(0);
        });
        __builtin_amdgcn_sched_barrier(0);
        // (b) B_p[m2] = sum C_p[m1][m2][m3] x[m1] g[m3], m1 outermost
        float B[kMaxL + 1][2 * kMaxL + 1][CPL];
        static_for<n1>([&](auto aI) __attribute__((always_inline)) {
            constexpr int a = decltype(aI)::value;
            float p3[n3][CPL];
#pragma unroll
            for (int b = 0; b < n3; ++b)
#pragma unroll
                for (int c = 0; c < CPL; ++c) p3[b][c] = xv[o1 + a][c] * gv[o3 + b][c];
            static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
                constexpr int kk = decltype(kI)::value;
                constexpr int p = pp.p[kk];
                constexpr int z0 = nz_m1_begin<S>(p, a), z1 = nz_m1_begin<S>(p, a + 1);
                static_for<z1 - z0>([&](auto zI) __attribute__((always_inline)) {
                    constexpr int n = z0 + decltype(zI)::value;
                    constexpr CgNz nzv = S::nz[n];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        if constexpr (nz_first_m2<S>(n))
                            B[kk][nzv.m2][c] = nzv.c * p3[nzv.m3][c];
                        else
                            B[kk][nzv.m2][c] = __builtin_fmaf(nzv.c, p3[nzv.m3][c], B[kk][nzv.m2][c]);
                    }
                });
            });
            if constexpr (L >= 3) __builtin_amdgcn_sched_barrier(0);
        });
        // (c) dY partial sums
        static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
            constexpr int kk = decltype(kI)::value;
            constexpr int p = pp.p[kk];
            constexpr int n2 = 2 * S::paths[p].l2 + 1, o2 = S::paths[p].l2 * S::paths[p].l2;
#pragma unroll
            for (int b = 0; b < n2; ++b)
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    dya[o2 + b] = __builtin_fmaf(wv[p][c], B[kk][b][c], dya[o2 + b]);
        });
        __builtin_amdgcn_sched_barrier(0);
    });
}

// After an edge: dY summed over the workgroup's channels (lanes by fixed-order
// halving, then waves through LDS in wave order) while T of the next edge is
// built into Tn from its harmonics ynext (staged in Yn); wave 0 stores dY of
// edge e_cur, or with VEC dvec = J(vec)^T dY.  tt is the thread index.
template <int L, int V, bool VEC>
__device__ __forceinline__ void edge_dy_finish(const float (&dya)[16], float (*sRed)[16], float* Tn, float* Yn,
                                               const SlotDev* sTab, const ShCoef* sSh, bool has_next, float ynext,
                                               int tt, int nth, int nwaves, const float* __restrict__ yv, long e_cur,
                                               float* __restrict__ dyv) {
    constexpr int D2 = (L + 1) * (L + 1);
    const int ln = tt & 63;
    // dY: lanes (fixed-order halving), then waves (LDS, fixed order)
    const float r = wave_sum16(dya, ln);
    if (sum16_holder(ln)) sRed[tt >> 6][sum16_index(ln)] = r;
    if (has_next && tt < D2) Yn[tt] = ynext;
    __syncthreads();
    if (has_next) build_T_lds<L, V>(Tn, Yn, sTab, tt, nth);
    float tot = 0.0f;
    if (tt < D2) {
        tot = sRed[0][tt];
        for (int q = 1; q < nwaves; ++q) tot += sRed[q][tt];
    }
    if constexpr (VEC) {
        // dvec = (I - r r^T)/|v| * sum_k dY_k grad Y_k(r), lanes < D2 of wave 0
        if (tt < 64) {
            const float* vp = yv + 3 * e_cur;
            const float vx = vp[0], vy = vp[1], vz = vp[2];
            const float n2 = vx * vx + vy * vy + vz * vz;
            const float inv = n2 > 0.0f ? 1.0f / sqrtf(n2) : 0.0f;
            const float rx = vx * inv, ry = vy * inv, rz = vz * inv;
            float g[3] = {0.0f, 0.0f, 0.0f};
            if (ln < D2) {
                sh_component_grad_c(sSh[ln], rx, ry, rz, g);
                g[0] *= tot; g[1] *= tot; g[2] *= tot;
            }
            const float gx = lane_value(wave_sum_to_last(g[0]), 63);
            const float gy = lane_value(wave_sum_to_last(g[1]), 63);
            const float gz = lane_value(wave_sum_to_last(g[2]), 63);
            const float rg = rx * gx + ry * gy + rz * gz;
            if (ln < 3) {
                const float gl = ln == 0 ? gx : (ln == 1 ? gy : gz);
                const float rl = ln == 0 ? rx : (ln == 1 ? ry : rz);
                dyv[3 * e_cur + ln] = (gl - rg * rl) * inv;
            }
        }
    } else {
        if (tt < D2) dyv[e_cur * D2 + tt] = tot;
    }
}

// Harmonics of edge e for the next T build: lane tt < D2 gets Y_e[tt] (from
// vec and the LDS coefficient copy with VEC, else a buffer load); others 0.
template <int D2, bool VEC>
__device__ __forceinline__ float next_y(const float* __restrict__ yv, long e, int tt, const ShCoef* sSh) {
    if constexpr (VEC) {
        const float* vp = yv + 3 * e;
        return tt < D2 ? sh_component_c(tt, sSh[tt < D2 ? tt : 0], vp[0], vp[1], vp[2]) : 0.0f;
    } else {
        return sh_load<D2, VEC>(yv, e, tt);
    }
}

// With one G slot per path (variant 1) the G row alone is D_out registers per
// channel, so that variant may take two waves per SIMD instead of spilling.
// SPLIT (small grids): blockIdx.y picks one half of the sender's out-edges;
// dx is added with fp32 atomics into a zeroed dx (two addends: order-free).
template <int L, int CPL, bool VEC, int V, bool SPLIT>
__global__ void __launch_bounds__(kBwdMaxThreads)
__attribute__((amdgpu_waves_per_eu(V == kVariantSlots ? 2 : BWD_WPE, 8)))
k_bwd_sender(int C, const float* __restrict__ G, const float* __restrict__ x, const float* __restrict__ yv,
             const float* __restrict__ w, const int* __restrict__ send_ptr, const int* __restrict__ send_perm,
             const int* __restrict__ send_recv, float* __restrict__ dx, float* __restrict__ dw,
             float* __restrict__ dyv) {
    using S = Spec<L, L, L, V>;
    constexpr int D1 = S::D1, D2 = S::D2, D3 = S::DO, P = S::P, NT = S::NT, NTP = (NT + 3) & ~3;
    __shared__ __attribute__((aligned(16))) float sT[2][NTP];
    __shared__ float sY[2][16];
    __shared__ float sRed[kBwdMaxThreads / 64][16];
    __shared__ SlotDev sTab[NT];
    __shared__ ShCoef sSh[VEC ? 16 : 1];   // harmonic coefficients, read per edge from LDS

    const int j = blockIdx.x;
    const int tid = threadIdx.x, nth = blockDim.x;
    const int nwaves = nth >> 6;
    const int c0 = tid * CPL;
    const uint32_t voff = opaque_lane(c0 < C ? (uint32_t)c0 * 4u : kOffLane);   // no channel: loads 0, stores dropped

    float xv[D1][CPL], dxa[D1][CPL];
    {
        const rsrc_t xr = make_row(x + (long)j * D1 * C, (long)D1 * C);
#pragma unroll
        for (int d = 0; d < D1; ++d) {
            bload<CPL, kStream>(xr, voff, (uint32_t)(d * C * 4), xv[d]);
#pragma unroll
            for (int c = 0; c < CPL; ++c) dxa[d][c] = 0.0f;
        }
    }

    int k0 = send_ptr[j], k1 = send_ptr[j + 1];
    if constexpr (SPLIT) {
        const int mid = k0 + (k1 - k0 + 1) / 2;
        if (blockIdx.y == 0) k1 = mid; else k0 = mid;
    }
    if (k0 < k1) {
        {
            const SlotDev* tab = slot_tab<L, V>();
            for (int t = tid; t < NT; t += nth) sTab[t] = tab[t];
            if constexpr (VEC)
                if (tid < 16) sSh[tid] = sh_tab().k[tid];
        }
        float gv[D3][CPL], wv[P][CPL];
        long e = send_perm[k0];
        const float y0 = sh_load<D2, VEC>(yv, e, tid);
        load_bwd_operands<S, CPL>(gv, wv, G, w, send_recv[k0], e, C, voff);
        if (tid < D2) sY[0][tid] = y0;
        __syncthreads();
        build_T_lds<L, V>(sT[0], sY[0], sTab, tid, nth);
        __syncthreads();

        // Per out-edge k: compute with T(k) and the rows already in registers;
        // then load the rows of edge k+1 into the same registers, reduce dY,
        // and build T(k+1) in the other buffer while those loads are in flight.
        for (int k = k0; k < k1; ++k) {
            const int buf = (k - k0) & 1;
            const bool has_next = k + 1 < k1;
            const float* T = sT[buf];

            // Work grouped by (l1, l3): for each pair, v_p, dw_p and dx for its
            // paths, then B_p from the products x[l1 m1] g[l3 m3] formed m1 by m1
            // and shared by the pair's paths.  A scheduling barrier after each
            // pair bounds register lifetimes.
            const rsrc_t dwr = make_row(dw + e * P * C, (long)P * C);
            float dya[16];
#pragma unroll
            for (int d = 0; d < 16; ++d) dya[d] = 0.0f;
            static_for<S::NG>([&](auto gI) __attribute__((always_inline)) {
                constexpr PathGroup pp = S::groups[decltype(gI)::value];
                constexpr int l1 = pp.l1, l3 = pp.l3;
                {
                    {
                        constexpr int n1 = 2 * l1 + 1, n3 = 2 * l3 + 1;
                        constexpr int o1 = l1 * l1, o3 = pp.o3;   // o3: the group's block of G
                        // (a) v_p = T_p^T g, dw_p = x . v_p, dx += w_p v_p
                        static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
                            constexpr int p = pp.p[decltype(kI)::value];
                            constexpr int t0 = S::slot_begin[p], t1 = S::slot_begin[p + 1];
                            float v[n1][CPL];
                            static_for<t1 - t0>([&](auto tI) __attribute__((always_inline)) {
                                constexpr int t = t0 + decltype(tI)::value;
                                constexpr TSlot s = S::slots[t];
                                const float tv = slot_value<t>(T);
#pragma unroll
                                for (int c = 0; c < CPL; ++c) {
                                    if constexpr (first_m1<S>(t))
                                        v[s.m1][c] = tv * gv[o3 + s.m3][c];
                                    else
                                        v[s.m1][c] = __builtin_fmaf(tv, gv[o3 + s.m3][c], v[s.m1][c]);
                                }
                            });
                            float dwv[CPL];
#pragma unroll
                            for (int c = 0; c < CPL; ++c) {
                                dwv[c] = xv[o1][c] * v[0][c];
#pragma unroll
                                for (int a = 1; a < n1; ++a) dwv[c] = __builtin_fmaf(xv[o1 + a][c], v[a][c], dwv[c]);
                            }
                            bstore<CPL, kStream>(dwr, voff, (uint32_t)p * opaque_u32((uint32_t)C * 4u), dwv);
#pragma unroll
                            for (int a = 0; a < n1; ++a)
#pragma unroll
                                for (int c = 0; c < CPL; ++c) {
                                    dxa[o1 + a][c] = __builtin_fmaf(wv[p][c], v[a][c], dxa[o1 + a][c]);
                                    pin_f32(dxa[o1 + a][c]);
                                }
                            if constexpr (L >= 3) __builtin_amdgcn_sched_barrier(0);
                        });
                        __builtin_amdgcn_sched_barrier(0);
                        // (b) B_p[m2] = sum C_p[m1][m2][m3] x[m1] g[m3], m1 outermost
                        float B[kMaxL + 1][2 * kMaxL + 1][CPL];
                        static_for<n1>([&](auto aI) __attribute__((always_inline)) {
                            constexpr int a = decltype(aI)::value;
                            float p3[n3][CPL];
#pragma unroll
                            for (int b = 0; b < n3; ++b)
#pragma unroll
                                for (int c = 0; c < CPL; ++c) p3[b][c] = xv[o1 + a][c] * gv[o3 + b][c];
                            static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
                                constexpr int kk = decltype(kI)::value;
                                constexpr int p = pp.p[kk];
                                constexpr int z0 = nz_m1_begin<S>(p, a), z1 = nz_m1_begin<S>(p, a + 1);
                                static_for<z1 - z0>([&](auto zI) __attribute__((always_inline)) {
                                    constexpr int n = z0 + decltype(zI)::value;
                                    constexpr CgNz nzv = S::nz[n];
#pragma unroll
                                    for (int c = 0; c < CPL; ++c) {
                                        if constexpr (nz_first_m2<S>(n))
                                            B[kk][nzv.m2][c] = nzv.c * p3[nzv.m3][c];
                                        else
                                            B[kk][nzv.m2][c] = __builtin_fmaf(nzv.c, p3[nzv.m3][c], B[kk][nzv.m2][c]);
                                    }
                                });
                            });
                            if constexpr (L >= 3) __builtin_amdgcn_sched_barrier(0);
                        });
                        // (c) dY partial sums
                        static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
                            constexpr int kk = decltype(kI)::value;
                            constexpr int p = pp.p[kk];
                            constexpr int n2 = 2 * S::paths[p].l2 + 1, o2 = S::paths[p].l2 * S::paths[p].l2;
#pragma unroll
                            for (int b = 0; b < n2; ++b)
#pragma unroll
                                for (int c = 0; c < CPL; ++c)
                                    dya[o2 + b] = __builtin_fmaf(wv[p][c], B[kk][b][c], dya[o2 + b]);
                        });
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            });

            // rows of the next edge into the registers just freed (unconditional:
            // after the last edge the loads use an out-of-range offset and return 0).
            // The dY sums are pinned first so the loads cannot be hoisted into the
            // arithmetic above, where their registers would still be in use.
#pragma unroll
            for (int d = 0; d < D2; ++d) pin_f32(dya[d]);
            const long e_cur = e;
            const int kn = has_next ? k + 1 : k;
            e = send_perm[kn];
            // A fresh copy of the thread index each edge keeps the address
            // arithmetic below from being hoisted out of the loop, where it would
            // hold registers through the arithmetic above.
            const int tt = (int)opaque_lane((uint32_t)tid);
            const int ln = tt & 63;
            float ynext;
            if constexpr (VEC) {
                const float* vp = yv + 3 * e;
                ynext = tt < D2 ? sh_component_c(tt, sSh[tt < D2 ? tt : 0], vp[0], vp[1], vp[2]) : 0.0f;
            } else {
                ynext = sh_load<D2, VEC>(yv, e, tt);
            }
            load_bwd_operands<S, CPL>(gv, wv, G, w, send_recv[kn], e, C, has_next ? voff : kOffLane);
            __builtin_amdgcn_sched_barrier(0);

            // dY: lanes (fixed-order halving), then waves (LDS, fixed order)
            const float r = wave_sum16(dya, ln);
            if (sum16_holder(ln)) sRed[tt >> 6][sum16_index(ln)] = r;
            if (has_next && tt < D2) sY[buf ^ 1][tt] = ynext;
            __syncthreads();
            if (has_next) build_T_lds<L, V>(sT[buf ^ 1], sY[buf ^ 1], sTab, tt, nth);
            float tot = 0.0f;
            if (tt < D2) {
                tot = sRed[0][tt];
                for (int q = 1; q < nwaves; ++q) tot += sRed[q][tt];
            }
            if constexpr (VEC) {
                // dvec = (I - r r^T)/|v| * sum_k dY_k grad Y_k(r), lanes < D2 of wave 0
                if (tt < 64) {
                    const float* vp = yv + 3 * e_cur;
                    const float vx = vp[0], vy = vp[1], vz = vp[2];
                    const float n2 = vx * vx + vy * vy + vz * vz;
                    const float inv = n2 > 0.0f ? 1.0f / sqrtf(n2) : 0.0f;
                    const float rx = vx * inv, ry = vy * inv, rz = vz * inv;
                    float g[3] = {0.0f, 0.0f, 0.0f};
                    if (ln < D2) {
                        sh_component_grad_c(sSh[ln], rx, ry, rz, g);
                        g[0] *= tot; g[1] *= tot; g[2] *= tot;
                    }
                    const float gx = lane_value(wave_sum_to_last(g[0]), 63);
                    const float gy = lane_value(wave_sum_to_last(g[1]), 63);
                    const float gz = lane_value(wave_sum_to_last(g[2]), 63);
                    const float rg = rx * gx + ry * gy + rz * gz;
                    if (ln < 3) {
                        const float gl = ln == 0 ? gx : (ln == 1 ? gy : gz);
                        const float rl = ln == 0 ? rx : (ln == 1 ? ry : rz);
                        dyv[3 * e_cur + ln] = (gl - rg * rl) * inv;
                    }
                }
            } else {
                if (tt < D2) dyv[e_cur * D2 + tt] = tot;
            }
            __syncthreads();
        }
    }

    if constexpr (SPLIT) {
        if (k0 < k1 && c0 < C) {
            float* o = dx + (long)j * D1 * C + c0;
#pragma unroll
            for (int d = 0; d < D1; ++d)
#pragma unroll
                for (int c = 0; c < CPL; ++c) unsafeAtomicAdd(o + (long)d * C + c, dxa[d][c]);
        }
    } else {
        const rsrc_t dxr = make_row(dx + (long)j * D1 * C, (long)D1 * C);
#pragma unroll
        for (int d = 0; d < D1; ++d) bstore<CPL, kStream>(dxr, voff, (uint32_t)(d * C * 4), dxa[d]);
    }
}

// ------------------------------------------------------------ K3m: receiver-major backward with edge messages
//
// The same products as K3 with the roles of the two nodes exchanged: one
// workgroup per receiver i keeps G[i] in registers and walks its in-edges in
// CSR order, loading x[j] and w[e] per edge.  dw[e] and dY[e] are stored as in
// K3; the edge's message msg[e, l1 m1] = sum_p w_p v_p[m1] goes to a workspace
// row e, and k_msg_sum then forms dx[j] as the sum of the messages of j's
// out-edges in sender-sorted order (fixed, so reproducible).  G is read once
// per receiver instead of once per edge, which pays when G's rows are much
// wider than x's (one output slot per path: 99 against 16 components at L=3).

// x row of sender j and w row of edge e, CPL channels per lane.
template <class S, int CPL>
__device__ __forceinline__ void load_recv_operands(float (&xv)[S::D1][CPL], float (&wv)[S::P][CPL],
                                                   const float* __restrict__ x, const float* __restrict__ w, long j,
                                                   long e, int C, uint32_t voff) {
    const rsrc_t xr = make_row(x + j * S::D1 * C, (long)S::D1 * C);
    const rsrc_t wr = make_row(w + e * S::P * C, (long)S::P * C);
    const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
#pragma unroll
    for (int d = 0; d < S::D1; ++d) bload<CPL>(xr, voff, (uint32_t)d * c4, xv[d]);
#pragma unroll
    for (int p = 0; p < S::P; ++p) bload<CPL, kStream>(wr, voff, (uint32_t)p * c4, wv[p]);
}

template <int L, bool VEC, int V>
__global__ void __launch_bounds__(kBwdMaxThreads)
__attribute__((amdgpu_waves_per_eu(V == kVariantSlots ? 2 : BWD_WPE, 8)))
k_bwd_recv(int C, const float* __restrict__ G, const float* __restrict__ x, const float* __restrict__ yv,
           const float* __restrict__ w, const int* __restrict__ row_ptr, const int* __restrict__ senders,
           float* __restrict__ msg, float* __restrict__ dw, float* __restrict__ dyv) {
    constexpr int CPL = 1;
    using S = Spec<L, L, L, V>;
    constexpr int D1 = S::D1, D2 = S::D2, D3 = S::DO, P = S::P, NT = S::NT, NTP = (NT + 3) & ~3;
    __shared__ __attribute__((aligned(16))) float sT[2][NTP];
    __shared__ float sY[2][16];
    __shared__ float sRed[kBwdMaxThreads / 64][16];
    __shared__ SlotDev sTab[NT];
    __shared__ ShCoef sSh[VEC ? 16 : 1];

    const int i = blockIdx.x;
    const int k0 = row_ptr[i], k1 = row_ptr[i + 1];
    if (k0 >= k1) return;   // the whole workgroup: no in-edges, nothing to store
    const int tid = threadIdx.x, nth = blockDim.x;
    const int nwaves = nth >> 6;
    const uint32_t voff = opaque_lane(tid < C ? (uint32_t)tid * 4u : kOffLane);   // no channel: loads 0, stores dropped

    float gv[D3][CPL];
    {
        const rsrc_t gr = make_row(G + (long)i * D3 * C, (long)D3 * C);
#pragma unroll
        for (int d = 0; d < D3; ++d) bload<CPL, kStream>(gr, voff, (uint32_t)(d * C * 4), gv[d]);
    }
    {
        const SlotDev* tab = slot_tab<L, V>();
        for (int t = tid; t < NT; t += nth) sTab[t] = tab[t];
        if constexpr (VEC)
            if (tid < 16) sSh[tid] = sh_tab().k[tid];
    }
    float xv[D1][CPL], wv[P][CPL];
    long e = k0;
    const float y0 = sh_load<D2, VEC>(yv, e, tid);
    load_recv_operands<S, CPL>(xv, wv, x, w, senders[k0], e, C, voff);
    if (tid < D2) sY[0][tid] = y0;
    __syncthreads();
    build_T_lds<L, V>(sT[0], sY[0], sTab, tid, nth);
    __syncthreads();

    // Per in-edge: products with T(e) and the rows in registers, the message
    // stored, then the next edge's rows loaded while dY is reduced and T(e+1)
    // built in the other buffer.
    for (int k = k0; k < k1; ++k) {
        const int buf = (k - k0) & 1;
        const bool has_next = k + 1 < k1;
        float mx[D1][CPL], dya[16];
#pragma unroll
        for (int d = 0; d < D1; ++d) mx[d][0] = 0.0f;
#pragma unroll
        for (int d = 0; d < 16; ++d) dya[d] = 0.0f;
        edge_backward<L, S, CPL>(sT[buf], xv, gv, wv, make_row(dw + e * P * C, (long)P * C), voff, C, mx, dya);
        {
            const rsrc_t mr = make_row(msg + e * D1 * C, (long)D1 * C);
#pragma unroll
            for (int d = 0; d < D1; ++d) bstore<CPL, kStream>(mr, voff, (uint32_t)(d * C * 4), mx[d]);
        }
#pragma unroll
        for (int d = 0; d < D2; ++d) pin_f32(dya[d]);
        const long e_cur = e;
        e = has_next ? k + 1 : k;
        const int tt = (int)opaque_lane((uint32_t)tid);
        const float ynext = next_y<D2, VEC>(yv, e, tt, sSh);
        load_recv_operands<S, CPL>(xv, wv, x, w, senders[e], e, C, has_next ? voff : kOffLane);
        __builtin_amdgcn_sched_barrier(0);
        edge_dy_finish<L, V, VEC>(dya, sRed, sT[buf ^ 1], sY[buf ^ 1], sTab, sSh, has_next, ynext, tt, nth, nwaves,
                                  yv, e_cur, dyv);
        __syncthreads();
    }
}

// dx[j] = sum over j's out-edges k (sender-sorted order) of msg[send_perm[k]]:
// one workgroup per (sender, span of the row); each thread owns R vectors of
// VW floats, 256 * VW floats apart, and keeps U edges' loads in flight;
// additions run in edge order.
template <int VW, int U, int R>
__global__ void __launch_bounds__(256)
k_msg_sum(long row, const float* __restrict__ msg, const int* __restrict__ send_ptr,
          const int* __restrict__ send_perm, float* __restrict__ dx) {
    using vec_t = float __attribute__((ext_vector_type(VW)));
    const int j = blockIdx.x;
    const long t = ((long)blockIdx.y * 256 * R + threadIdx.x) * VW;
    if (t >= row) return;
    const int k0 = send_ptr[j], k1 = send_ptr[j + 1];
    bool ok[R];
    vec_t acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        ok[r] = t + (long)r * 256 * VW < row;
        acc[r] = (vec_t)0.0f;
    }
    auto ld = [&](int k, int r) {
        return __builtin_nontemporal_load(
            reinterpret_cast<const vec_t*>(msg + (long)send_perm[k] * row + t + (long)r * 256 * VW));
    };
    int k = k0;
    for (; k + U <= k1; k += U) {
        vec_t m[U][R];
#pragma unroll
        for (int q = 0; q < U; ++q)
#pragma unroll
            for (int r = 0; r < R; ++r) m[q][r] = ok[r] ? ld(k + q, r) : (vec_t)0.0f;
#pragma unroll
        for (int q = 0; q < U; ++q)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] += m[q][r];
    }
    for (; k < k1; ++k)
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (ok[r]) acc[r] += ld(k, r);
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (ok[r]) *reinterpret_cast<vec_t*>(dx + (long)j * row + t + (long)r * 256 * VW) = acc[r];
}

// ------------------------------------------------------------ standalone harmonics (vec -> Y, dY -> dvec)

template <int L>
__global__ void k_sh(long n_edges, const float* __restrict__ vec, float* __restrict__ Y) {
    constexpr int D = (L + 1) * (L + 1);
    const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_edges * D) return;
    const long e = t / D;
    const int k = static_cast<int>(t - e * D);
    Y[t] = sh_component(k, vec[3 * e], vec[3 * e + 1], vec[3 * e + 2]);
}

template <int L>
__global__ void k_sh_bwd(long n_edges, const float* __restrict__ vec, const float* __restrict__ dY,
                         float* __restrict__ dvec) {
    constexpr int D = (L + 1) * (L + 1);
    const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n_edges) return;
    const float vx = vec[3 * e], vy = vec[3 * e + 1], vz = vec[3 * e + 2];
    const float n2 = vx * vx + vy * vy + vz * vz;
    if (n2 == 0.0f) {
        dvec[3 * e] = dvec[3 * e + 1] = dvec[3 * e + 2] = 0.0f;
        return;
    }
    const float inv = 1.0f / sqrtf(n2);
    const float rx = vx * inv, ry = vy * inv, rz = vz * inv;
    float gx = 0.0f, gy = 0.0f, gz = 0.0f;
#pragma unroll
    for (int k = 0; k < D; ++k) {
        float g[3];
        sh_component_grad(k, rx, ry, rz, g);
        const float d = dY[e * D + k];
        gx = __builtin_fmaf(d, g[0], gx);
        gy = __builtin_fmaf(d, g[1], gy);
        gz = __builtin_fmaf(d, g[2], gz);
    }
    const float rg = rx * gx + ry * gy + rz * gz;
    dvec[3 * e] = (gx - rg * rx) * inv;
    dvec[3 * e + 1] = (gy - rg * ry) * inv;
    dvec[3 * e + 2] = (gz - rg * rz) * inv;
}

// Second-order terms for edge vectors (the VJP of the backward when the
// harmonics are evaluated from vec; r = v/|v|, n = |v|, P = I - r r^T):
//   aY[e, k] = (J a)_k = g_k . P a / n                       (k_sh_jvp)
//   gvec[e]  = J^T gY + d/dv < J a, dY >                     (k_sh_bwd_bwd)
// with g_k, H_k the gradient and Hessian of Y_k's polynomial form in r.  For
// u = sum dY_k g_k, M = sum dY_k H_k and f = u . P a:
//   d/dv < J a, dY > = (P grad_r f - f r) / n^2,
//   grad_r f = M a - (r . a)(M r + u) - (u . r) a.
template <int L>
__global__ void k_sh_jvp(long n_edges, const float* __restrict__ vec, const float* __restrict__ a,
                         float* __restrict__ aY) {
    constexpr int D = (L + 1) * (L + 1);
    const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_edges * D) return;
    const long e = t / D;
    const int k = static_cast<int>(t - e * D);
    const float vx = vec[3 * e], vy = vec[3 * e + 1], vz = vec[3 * e + 2];
    const float n2 = vx * vx + vy * vy + vz * vz;
    if (n2 == 0.0f) {
        aY[t] = 0.0f;
        return;
    }
    const float inv = 1.0f / sqrtf(n2);
    const float rx = vx * inv, ry = vy * inv, rz = vz * inv;
    const float ax = a[3 * e], ay = a[3 * e + 1], az = a[3 * e + 2];
    float g[3];
    sh_component_grad(k, rx, ry, rz, g);
    const float ga = g[0] * ax + g[1] * ay + g[2] * az;
    const float gr = g[0] * rx + g[1] * ry + g[2] * rz;
    const float ra = rx * ax + ry * ay + rz * az;
    aY[t] = (ga - gr * ra) * inv;
}

template <int L>
__global__ void k_sh_bwd_bwd(long n_edges, const float* __restrict__ vec, const float* __restrict__ dY,
                             const float* __restrict__ a, const float* __restrict__ gY, float* __restrict__ gvec) {
    constexpr int D = (L + 1) * (L + 1);
    const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n_edges) return;
    const float vx = vec[3 * e], vy = vec[3 * e + 1], vz = vec[3 * e + 2];
    const float n2 = vx * vx + vy * vy + vz * vz;
    if (n2 == 0.0f) {
        gvec[3 * e] = gvec[3 * e + 1] = gvec[3 * e + 2] = 0.0f;
        return;
    }
    const float inv = 1.0f / sqrtf(n2);
    const float r[3] = {vx * inv, vy * inv, vz * inv};
    const float av[3] = {a[3 * e], a[3 * e + 1], a[3 * e + 2]};
    float wv[3] = {0.0f, 0.0f, 0.0f}, u[3] = {0.0f, 0.0f, 0.0f};
    float M[6] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};   // xx, xy, yy, xz, yz, zz
#pragma unroll
    for (int k = 0; k < D; ++k) {
        float g[3], h[6];
        sh_component_hess(k, r[0], r[1], r[2], g, h);
        const float gy = gY[e * D + k], dy = dY[e * D + k];
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            wv[i] = __builtin_fmaf(gy, g[i], wv[i]);
            u[i] = __builtin_fmaf(dy, g[i], u[i]);
        }
#pragma unroll
        for (int i = 0; i < 6; ++i) M[i] = __builtin_fmaf(dy, h[i], M[i]);
    }
    auto mul = [&](const float* q, float* o) {
        o[0] = M[0] * q[0] + M[1] * q[1] + M[3] * q[2];
        o[1] = M[1] * q[0] + M[2] * q[1] + M[4] * q[2];
        o[2] = M[3] * q[0] + M[4] * q[1] + M[5] * q[2];
    };
    const float wr = wv[0] * r[0] + wv[1] * r[1] + wv[2] * r[2];
    const float ur = u[0] * r[0] + u[1] * r[1] + u[2] * r[2];
    const float ra = r[0] * av[0] + r[1] * av[1] + r[2] * av[2];
    const float f = (u[0] * av[0] + u[1] * av[1] + u[2] * av[2]) - ur * ra;
    float Ma[3], Mr[3], df[3];
    mul(av, Ma);
    mul(r, Mr);
#pragma unroll
    for (int i = 0; i < 3; ++i) df[i] = Ma[i] - ra * (Mr[i] + u[i]) - ur * av[i];
    const float dfr = df[0] * r[0] + df[1] * r[1] + df[2] * r[2];
    const float inv2 = inv * inv;
#pragma unroll
    for (int i = 0; i < 3; ++i)
        gvec[3 * e + i] = (wv[i] - wr * r[i]) * inv + (df[i] - dfr * r[i] - f * r[i]) * inv2;
}

// ------------------------------------------------------------ launchers

namespace {

struct ChanMap {
    int cpl, waves, tiles;   // channels per lane, waves per workgroup, channel tiles (grid.y)
};

// One channel per lane.  The kernels also take two adjacent channels per lane
// (CPL = 2: half the T reads and loop control per channel, twice the
// registers); measured at C = 128-1024 that was 1-2% slower in the CSR
// forward and twice as slow in the atomic one, so every launch uses CPL = 1.
ChanMap chan_map(int C, int max_waves) {
    ChanMap m{};
    m.cpl = 1;
    const int per_wave = 64 * m.cpl;
    const int need = (C + per_wave - 1) / per_wave;
    m.waves = need < max_waves ? need : max_waves;
    m.tiles = (need + m.waves - 1) / m.waves;
    return m;
}

// Grids with fewer waves than 4 per SIMD split every edge list in two (SPLIT).
constexpr long kSplitBelowWaves = 4L * 1024;

template <int L, int CPL, int V, bool SPLIT>
hipError_t fwd_csr_launch(const LaunchArgs& a, const ChanMap& m, hipStream_t st) {
    const dim3 grid(a.n_nodes, m.tiles, SPLIT ? 2 : 1), block(64 * m.waves);
    if (SPLIT) {
        const long n = (long)a.n_nodes * Spec<L, L, L, V>::DO * a.C;
        hipLaunchKernelGGL(k_zero, dim3(1024), dim3(256), 0, st, a.out, n);
    }
    if (a.vec_mode)
        hipLaunchKernelGGL((k_fwd_csr<L, CPL, true, V, SPLIT>), grid, block, 0, st, a.C, a.x, a.y, a.w, a.row_ptr,
                           a.senders, a.out);
    else
        hipLaunchKernelGGL((k_fwd_csr<L, CPL, false, V, SPLIT>), grid, block, 0, st, a.C, a.x, a.y, a.w, a.row_ptr,
                           a.senders, a.out);
    return hipGetLastError();
}

template <int L, int CPL, int V>
hipError_t fwd_dispatch(const LaunchArgs& a, const ChanMap& m, hipStream_t st) {
    dim3 block(64 * m.waves);
    if (a.algo == 0) {
        const bool split = CPL == 1 && V == kVariantSummed && (long)a.n_nodes * m.tiles * m.waves < kSplitBelowWaves;
        if constexpr (CPL == 1 && V == kVariantSummed)
            if (split) return fwd_csr_launch<L, CPL, V, true>(a, m, st);
        return fwd_csr_launch<L, CPL, V, false>(a, m, st);
    } else {
        const long n = (long)a.n_nodes * Spec<L, L, L, V>::DO * a.C;
        hipLaunchKernelGGL(k_zero, dim3(1024), dim3(256), 0, st, a.out, n);
        if (a.n_edges > 0) {
            dim3 grid(a.n_edges, m.tiles);
            if (a.vec_mode)
                hipLaunchKernelGGL((k_fwd_atomic<L, CPL, true, V>), grid, block, 0, st, a.n_nodes, a.C, a.x, a.y,
                                   a.w, a.row_ptr, a.senders, a.out);
            else
                hipLaunchKernelGGL((k_fwd_atomic<L, CPL, false, V>), grid, block, 0, st, a.n_nodes, a.C, a.x, a.y,
                                   a.w, a.row_ptr, a.senders, a.out);
        }
    }
    return hipGetLastError();
}

template <int L, int CPL, int V, bool SPLIT>
hipError_t bwd_launch(const LaunchArgs& a, const ChanMap& m, hipStream_t st) {
    const dim3 grid(a.n_nodes, SPLIT ? 2 : 1), block(64 * m.waves);
    if (SPLIT) {
        const long n = (long)a.n_nodes * Spec<L, L, L, V>::D1 * a.C;
        hipLaunchKernelGGL(k_zero, dim3(1024), dim3(256), 0, st, a.dx, n);
    }
    if (a.vec_mode)
        hipLaunchKernelGGL((k_bwd_sender<L, CPL, true, V, SPLIT>), grid, block, 0, st, a.C, a.grad, a.x, a.y, a.w,
                           a.send_ptr, a.send_perm, a.send_recv, a.dx, a.dw, a.dy);
    else
        hipLaunchKernelGGL((k_bwd_sender<L, CPL, false, V, SPLIT>), grid, block, 0, st, a.C, a.grad, a.x, a.y, a.w,
                           a.send_ptr, a.send_perm, a.send_recv, a.dx, a.dw, a.dy);
    return hipGetLastError();
}

template <int L, int CPL, int V>
hipError_t bwd_dispatch(const LaunchArgs& a, const ChanMap& m, hipStream_t st) {
    static_assert(CPL == 1, "the backward maps one channel per lane");
    if constexpr (V == kVariantSummed)
        if ((long)a.n_nodes * m.waves < kSplitBelowWaves) return bwd_launch<L, CPL, V, true>(a, m, st);
    return bwd_launch<L, CPL, V, false>(a, m, st);
}

template <int L>
hipError_t fwd_L(const LaunchArgs& a, hipStream_t st) {
    const ChanMap m = chan_map(a.C, kMaxThreads / 64);
    if (a.variant == kVariantSlots) return fwd_dispatch<L, 1, kVariantSlots>(a, m, st);
    return fwd_dispatch<L, 1, kVariantSummed>(a, m, st);
}

ChanMap bwd_chan_map(int C) {
    ChanMap m{};
    m.cpl = 1;
    m.waves = (C + 63) / 64;
    m.tiles = 1;
    return m;
}

template <int L>
hipError_t bwd_L(const LaunchArgs& a, hipStream_t st) {
    if (a.variant == kVariantSlots) return bwd_dispatch<L, 1, kVariantSlots>(a, bwd_chan_map(a.C), st);
    return bwd_dispatch<L, 1, kVariantSummed>(a, bwd_chan_map(a.C), st);
}

template <int L, int V>
hipError_t bwd_msg_L(const LaunchArgs& a, float* msg, hipStream_t st) {
    const ChanMap m = bwd_chan_map(a.C);
    if (a.n_edges > 0) {
        const dim3 grid(a.n_nodes), block(64 * m.waves);
        if (a.vec_mode)
            hipLaunchKernelGGL((k_bwd_recv<L, true, V>), grid, block, 0, st, a.C, a.grad, a.x, a.y, a.w, a.row_ptr,
                               a.senders, msg, a.dw, a.dy);
        else
            hipLaunchKernelGGL((k_bwd_recv<L, false, V>), grid, block, 0, st, a.C, a.grad, a.x, a.y, a.w,
                               a.row_ptr, a.senders, msg, a.dw, a.dy);
    }
    // dx rows of senders without out-edges come out zero
    const long row = (long)Spec<L, L, L, V>::D1 * a.C;
    // four edges in flight, one vector per thread: eight or sixteen edges, or
    // two vectors per thread, measured the same at lmax 3, C 128
    constexpr int kU = 4, kR = 1;
    if (row % 4 == 0)
        hipLaunchKernelGGL((k_msg_sum<4, kU, kR>), dim3(a.n_nodes, (unsigned)((row + 1024 * kR - 1) / (1024 * kR))),
                           dim3(256), 0, st, row, msg, a.send_ptr, a.send_perm, a.dx);
    else
        hipLaunchKernelGGL((k_msg_sum<1, kU, kR>), dim3(a.n_nodes, (unsigned)((row + 256 * kR - 1) / (256 * kR))),
                           dim3(256), 0, st, row, msg, a.send_ptr, a.send_perm, a.dx);
    return hipGetLastError();
}

template <int L>
hipError_t bwd_msg_V(const LaunchArgs& a, float* msg, hipStream_t st) {
    if (a.variant == kVariantSlots) return bwd_msg_L<L, kVariantSlots>(a, msg, st);
    return bwd_msg_L<L, kVariantSummed>(a, msg, st);
}

}  // namespace

bool bwd_supports_channels(int C) {
    // the backward keeps all channels of a sender in one workgroup (deterministic dY)
    return bwd_chan_map(C).waves <= kBwdMaxThreads / 64;
}

hipError_t launch_fwd(const LaunchArgs& a, hipStream_t st) {
    if (a.n_nodes == 0) return hipSuccess;
    if (a.algo == 2) return launch_fwd_frame(a, st);
    switch (a.L) {
        case 0: return fwd_L<0>(a, st);
        case 1: return fwd_L<1>(a, st);
        case 2: return fwd_L<2>(a, st);
        case 3: return fwd_L<3>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd(const LaunchArgs& a, hipStream_t st) {
    if (a.n_nodes == 0) return hipSuccess;
    switch (a.L) {
        case 0: return bwd_L<0>(a, st);
        case 1: return bwd_L<1>(a, st);
        case 2: return bwd_L<2>(a, st);
        case 3: return bwd_L<3>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_msg(const LaunchArgs& a, float* msg, hipStream_t st) {
    if (a.n_nodes == 0) return hipSuccess;
    switch (a.L) {
        case 0: return bwd_msg_V<0>(a, msg, st);
        case 1: return bwd_msg_V<1>(a, msg, st);
        case 2: return bwd_msg_V<2>(a, msg, st);
        case 3: return bwd_msg_V<3>(a, msg, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_sh(int L, long n_edges, const float* vec, float* Y, hipStream_t st) {
    if (n_edges == 0) return hipSuccess;
    const long D = (long)(L + 1) * (L + 1);
    const long n = n_edges * D;
    const dim3 block(256), grid((unsigned)((n + 255) / 256));
    switch (L) {
        case 0: hipLaunchKernelGGL(k_sh<0>, grid, block, 0, st, n_edges, vec, Y); break;
        case 1: hipLaunchKernelGGL(k_sh<1>, grid, block, 0, st, n_edges, vec, Y); break;
        case 2: hipLaunchKernelGGL(k_sh<2>, grid, block, 0, st, n_edges, vec, Y); break;
        case 3: hipLaunchKernelGGL(k_sh<3>, grid, block, 0, st, n_edges, vec, Y); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_sh_bwd(int L, long n_edges, const float* vec, const float* dY, float* dvec, hipStream_t st) {
    if (n_edges == 0) return hipSuccess;
    const dim3 block(256), grid((unsigned)((n_edges + 255) / 256));
    switch (L) {
        case 0: hipLaunchKernelGGL(k_sh_bwd<0>, grid, block, 0, st, n_edges, vec, dY, dvec); break;
        case 1: hipLaunchKernelGGL(k_sh_bwd<1>, grid, block, 0, st, n_edges, vec, dY, dvec); break;
        case 2: hipLaunchKernelGGL(k_sh_bwd<2>, grid, block, 0, st, n_edges, vec, dY, dvec); break;
        case 3: hipLaunchKernelGGL(k_sh_bwd<3>, grid, block, 0, st, n_edges, vec, dY, dvec); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_sh_jvp(int L, long n_edges, const float* vec, const float* a, float* aY, hipStream_t st) {
    if (n_edges == 0) return hipSuccess;
    const long n = n_edges * (L + 1) * (L + 1);
    const dim3 block(256), grid((unsigned)((n + 255) / 256));
    switch (L) {
        case 0: hipLaunchKernelGGL(k_sh_jvp<0>, grid, block, 0, st, n_edges, vec, a, aY); break;
        case 1: hipLaunchKernelGGL(k_sh_jvp<1>, grid, block, 0, st, n_edges, vec, a, aY); break;
        case 2: hipLaunchKernelGGL(k_sh_jvp<2>, grid, block, 0, st, n_edges, vec, a, aY); break;
        case 3: hipLaunchKernelGGL(k_sh_jvp<3>, grid, block, 0, st, n_edges, vec, a, aY); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_sh_bwd_bwd(int L, long n_edges, const float* vec, const float* dY, const float* a, const float* gY,
                             float* gvec, hipStream_t st) {
    if (n_edges == 0) return hipSuccess;
    const dim3 block(256), grid((unsigned)((n_edges + 255) / 256));
    switch (L) {
        case 0: hipLaunchKernelGGL(k_sh_bwd_bwd<0>, grid, block, 0, st, n_edges, vec, dY, a, gY, gvec); break;
        case 1: hipLaunchKernelGGL(k_sh_bwd_bwd<1>, grid, block, 0, st, n_edges, vec, dY, a, gY, gvec); break;
        case 2: hipLaunchKernelGGL(k_sh_bwd_bwd<2>, grid, block, 0, st, n_edges, vec, dY, a, gY, gvec); break;
        case 3: hipLaunchKernelGGL(k_sh_bwd_bwd<3>, grid, block, 0, st, n_edges, vec, dY, a, gY, gvec); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ctp
