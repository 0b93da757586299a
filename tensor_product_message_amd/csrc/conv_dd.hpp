// VJP of the VJP of the convolution tensor product (gfx950), Y given.
//
// The backward maps (x, w, Y, G) to (dx, dw, dY).  For cotangents (ax, aw, aY)
// of those outputs, L2 = <ax, dx> + <aw, dw> + <aY, dY>, and because the
// forward F(x, w, Y) is trilinear, every derivative of L2 is the backward's
// contraction with one operand swapped for its cotangent (FlashCart, arXiv
// 2610.06409, section on symbolic VJPs: the VJP-of-VJP the edge convolution
// needs for force training):
//
//   gG = F(ax, w, Y) + F(x, aw, Y) + F(x, w, aY)                    (receivers)
//   gx = dx(aw, Y) + dx(w, aY),  gw = dw(ax, Y) + dw(x, aY),
//   gY = dY(ax, w) + dY(x, aw)                                     (senders)
//
// Two kernels, each in the layout and schedule of its first-order sibling:
// k_dd_recv sums into receivers in CSR order like the forward, with two
// per-edge coupling tables T(Y) and T(aY) in LDS; k_dd_send walks each
// sender's out-edges like the backward.  Both write every output once in a
// fixed order: results are bitwise reproducible.
//
// Variant 1 (per-path output slots) takes the same code: each path reads and
// writes its own block of G, and the sender kernel walks the backward's path
// groups.  Above 512 channels the sender kernel runs as two channel tiles that
// add their partial gY into a zeroed gY (two addends onto zero: order-free).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace ctp {
namespace conv {

constexpr int kDdRecvMaxThreads = 256;
constexpr int kDdSendMaxThreads = 512;

template <int D>
__device__ __forceinline__ void load_row(rsrc_t r, uint32_t voff, uint32_t c4, float (&v)[D]) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
        float t[1];
        bload<1>(r, voff, (uint32_t)d * c4, t);
        v[d] = t[0];
    }
}

template <int D>
__device__ __forceinline__ void load_row_stream(rsrc_t r, uint32_t voff, uint32_t c4, float (&v)[D]) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
        float t[1];
        bload<1, kStream>(r, voff, (uint32_t)d * c4, t);
        v[d] = t[0];
    }
}

template <int D>
__device__ __forceinline__ void store_row_stream(rsrc_t r, uint32_t voff, uint32_t c4, const float (&v)[D]) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const float t[1] = {v[d]};
        bstore<1, kStream>(r, voff, (uint32_t)d * c4, t);
    }
}

// ------------------------------------------------------------ gG: receiver-major
//
// Per edge and path p:  s1 = w_p ax + aw_p x,  s2 = w_p x  (x rows of the sender),
//   gG[l3 m3] += sum_m1 T_p(Y)[m1][m3] s1[m1] + T_p(aY)[m1][m3] s2[m1].

template <class S>
__global__ void __launch_bounds__(kDdRecvMaxThreads)
k_dd_recv(int C, const float* __restrict__ x, const float* __restrict__ ax, const float* __restrict__ Y,
          const float* __restrict__ aY, const float* __restrict__ w, const float* __restrict__ aw,
          const int* __restrict__ row_ptr, const int* __restrict__ senders, float* __restrict__ gG) {
    constexpr int D1 = S::D1, D2 = S::D2, D3 = S::DO, P = S::P, NT = S::NT, NTP = (NT + 3) & ~3;
    __shared__ __attribute__((aligned(16))) float sT[2][2][NTP];   // [buffer][T(Y), T(aY)]
    __shared__ float sY[2][2][16];
    __shared__ SlotDev sTab[NT];

    const int i = blockIdx.x;
    const int tid = threadIdx.x, nth = blockDim.x;
    const int c0 = blockIdx.y * nth + tid;
    const uint32_t voff = opaque_lane(c0 < C ? (uint32_t)c0 * 4u : kOffLane);

    float acc[D3];
#pragma unroll
    for (int d = 0; d < D3; ++d) acc[d] = 0.0f;

    const int e0 = row_ptr[i], e1 = row_ptr[i + 1];
    if (e0 < e1) {
        {
            const SlotDev* tab = slot_tab<S>();
            for (int t = tid; t < NT; t += nth) sTab[t] = tab[t];
        }
        float xv[D1], axv[D1], wv[P], awv[P];
        auto load_edge = [&](long e, uint32_t vo) __attribute__((always_inline)) {
            const long j = senders[e];
            const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
            load_row<D1>(make_row(x + j * D1 * C, (long)D1 * C), vo, c4, xv);
            load_row<D1>(make_row(ax + j * D1 * C, (long)D1 * C), vo, c4, axv);
            load_row_stream<P>(make_row(w + e * P * C, (long)P * C), vo, c4, wv);
            load_row_stream<P>(make_row(aw + e * P * C, (long)P * C), vo, c4, awv);
        };
        {
            const float y0 = sh_load<D2, false>(Y, e0, tid), a0 = sh_load<D2, false>(aY, e0, tid);
            load_edge(e0, voff);
            if (tid < D2) {
                sY[0][0][tid] = y0;
                sY[0][1][tid] = a0;
            }
        }
        __syncthreads();
        build_T_lds<S>(sT[0][0], sY[0][0], sTab, tid, nth);
        build_T_lds<S>(sT[0][1], sY[0][1], sTab, tid, nth);
        __syncthreads();
        for (int e = e0; e < e1; ++e) {
            const int buf = (e - e0) & 1;
            const bool has_next = e + 1 < e1;
            const float* T0 = sT[buf][0];
            const float* T1 = sT[buf][1];
            static_for<P>([&](auto pI) __attribute__((always_inline)) {
                constexpr int p = decltype(pI)::value;
                constexpr PathL q = S::paths[p];
                constexpr int n1 = 2 * q.l1 + 1, o1 = q.l1 * q.l1, o3 = S::out_off[p];
                constexpr int t0 = S::slot_begin[p], t1 = S::slot_begin[p + 1];
                float s1[n1], s2[n1];
#pragma unroll
                for (int a = 0; a < n1; ++a) {
                    s2[a] = wv[p] * xv[o1 + a];
                    s1[a] = __builtin_fmaf(awv[p], xv[o1 + a], wv[p] * axv[o1 + a]);
                }
                static_for<t1 - t0>([&](auto tI) __attribute__((always_inline)) {
                    constexpr int t = t0 + decltype(tI)::value;
                    constexpr TSlot s = S::slots[t];
                    acc[o3 + s.m3] = __builtin_fmaf(slot_value<t>(T0), s1[s.m1], acc[o3 + s.m3]);
                    acc[o3 + s.m3] = __builtin_fmaf(slot_value<t>(T1), s2[s.m1], acc[o3 + s.m3]);
                });
                if constexpr (S::P >= 20) __builtin_amdgcn_sched_barrier(0x100);
            });
            // the sums are pinned so the next edge's loads cannot be hoisted above
            // the arithmetic that still needs the registers they reuse
#pragma unroll
            for (int d = 0; d < D3; ++d) pin_f32(acc[d]);
            const long en = has_next ? e + 1 : e;
            const int tt = (int)opaque_lane((uint32_t)tid);
            const float yn = sh_load<D2, false>(Y, en, tt), an = sh_load<D2, false>(aY, en, tt);
            load_edge(en, has_next ? voff : kOffLane);
            __builtin_amdgcn_sched_barrier(0);
            if (has_next) {
                if (tt < D2) {
                    sY[buf ^ 1][0][tt] = yn;
                    sY[buf ^ 1][1][tt] = an;
                }
                __syncthreads();
                build_T_lds<S>(sT[buf ^ 1][0], sY[buf ^ 1][0], sTab, tt, nth);
                build_T_lds<S>(sT[buf ^ 1][1], sY[buf ^ 1][1], sTab, tt, nth);
                __syncthreads();
            }
        }
    }
    store_row_stream<D3>(make_row(gG + (long)i * D3 * C, (long)D3 * C), voff, opaque_u32((uint32_t)C * 4u), acc);
}

// ------------------------------------------------------------ gx, gw, gY: sender-major
//
// Per out-edge e = j -> i with g = G[i], for each (l1, l3) pair:
//   v_p = T_p(Y)^T g,  v'_p = T_p(aY)^T g
//   gw[e,p] = ax . v_p + x . v'_p,   gx[j] += aw_p v_p + w_p v'_p
//   gY[e, l2 m2] = sum_c sum_p w_p B_p(ax, g)[m2] + aw_p B_p(x, g)[m2]
//                = sum_c sum_p B_p(w_p ax + aw_p x, g)[m2]   (B is linear in a),
//   B_p(a, g)[m2] = sum_{m1,m3} C_p[m1][m2][m3] a[m1] g[m3].

// Three waves per SIMD for variant 0 (at lmax 3: 168 VGPRs with 52 bytes of
// spills per lane instead of 175 VGPRs and two waves; measured 6% faster);
// variant 1 would spill 220 bytes and keeps the compiler's choice.
template <class S>
__global__ void __launch_bounds__(kDdSendMaxThreads)
__attribute__((amdgpu_waves_per_eu(S::V == kVariantSlots ? 2 : 3, 8)))
k_dd_send(int C, const float* __restrict__ G, const float* __restrict__ x, const float* __restrict__ ax,
          const float* __restrict__ Y, const float* __restrict__ aY, const float* __restrict__ w,
          const float* __restrict__ aw, const int* __restrict__ send_ptr, const int* __restrict__ send_perm,
          const int* __restrict__ send_recv, float* __restrict__ gx, float* __restrict__ gw,
          float* __restrict__ gY, int gy_atomic) {
    constexpr int D1 = S::D1, D2 = S::D2, D3 = S::DO, P = S::P, NT = S::NT, NTP = (NT + 3) & ~3;
    __shared__ __attribute__((aligned(16))) float sT[2][2][NTP];
    __shared__ float sY[2][2][16];
    __shared__ float sRed[kDdSendMaxThreads / 64][16];
    __shared__ SlotDev sTab[NT];

    const int j = blockIdx.x;
    const int tid = threadIdx.x, nth = blockDim.x;
    const int nwaves = nth >> 6;
    const int c0 = blockIdx.y * nth + tid;
    const uint32_t voff = opaque_lane(c0 < C ? (uint32_t)c0 * 4u : kOffLane);

    float xv[D1], axv[D1], gxa[D1];
    {
        const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
        load_row_stream<D1>(make_row(x + (long)j * D1 * C, (long)D1 * C), voff, c4, xv);
        load_row_stream<D1>(make_row(ax + (long)j * D1 * C, (long)D1 * C), voff, c4, axv);
#pragma unroll
        for (int d = 0; d < D1; ++d) gxa[d] = 0.0f;
    }

    const int k0 = send_ptr[j], k1 = send_ptr[j + 1];
    if (k0 < k1) {
        {
            const SlotDev* tab = slot_tab<S>();
            for (int t = tid; t < NT; t += nth) sTab[t] = tab[t];
        }
        float gv[D3], wv[P], awv[P];
        auto load_edge = [&](long i, long e, uint32_t vo) __attribute__((always_inline)) {
            const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
            load_row<D3>(make_row(G + i * D3 * C, (long)D3 * C), vo, c4, gv);
            load_row_stream<P>(make_row(w + e * P * C, (long)P * C), vo, c4, wv);
            load_row_stream<P>(make_row(aw + e * P * C, (long)P * C), vo, c4, awv);
        };
        long e = send_perm[k0];
        {
            const float y0 = sh_load<D2, false>(Y, e, tid), a0 = sh_load<D2, false>(aY, e, tid);
            load_edge(send_recv[k0], e, voff);
            if (tid < D2) {
                sY[0][0][tid] = y0;
                sY[0][1][tid] = a0;
            }
        }
        __syncthreads();
        build_T_lds<S>(sT[0][0], sY[0][0], sTab, tid, nth);
        build_T_lds<S>(sT[0][1], sY[0][1], sTab, tid, nth);
        __syncthreads();

        for (int k = k0; k < k1; ++k) {
            const int buf = (k - k0) & 1;
            const bool has_next = k + 1 < k1;
            const float* T0 = sT[buf][0];
            const float* T1 = sT[buf][1];
            const rsrc_t gwr = make_row(gw + e * P * C, (long)P * C);
            float gya[16];
#pragma unroll
            for (int d = 0; d < 16; ++d) gya[d] = 0.0f;
            static_for<S::NG>([&](auto gI) __attribute__((always_inline)) {
                constexpr PathGroup pp = S::groups[decltype(gI)::value];
                constexpr int l1 = pp.l1;
                {
                    {
                        constexpr int n1 = 2 * l1 + 1;
                        constexpr int o1 = l1 * l1, o3 = pp.o3;   // o3: the group's block of G
                        // (a) v, v', gw and gx for the pair's paths
                        static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
                            constexpr int p = pp.p[decltype(kI)::value];
                            constexpr int t0 = S::slot_begin[p], t1 = S::slot_begin[p + 1];
                            float v[n1], v2[n1];
                            static_for<t1 - t0>([&](auto tI) __attribute__((always_inline)) {
                                constexpr int t = t0 + decltype(tI)::value;
                                constexpr TSlot s = S::slots[t];
                                const float ty = slot_value<t>(T0), ta = slot_value<t>(T1);
                                if constexpr (first_m1<S>(t)) {
                                    v[s.m1] = ty * gv[o3 + s.m3];
                                    v2[s.m1] = ta * gv[o3 + s.m3];
                                } else {
                                    v[s.m1] = __builtin_fmaf(ty, gv[o3 + s.m3], v[s.m1]);
                                    v2[s.m1] = __builtin_fmaf(ta, gv[o3 + s.m3], v2[s.m1]);
                                }
                            });
                            float dw0 = axv[o1] * v[0];
#pragma unroll
                            for (int a = 1; a < n1; ++a) dw0 = __builtin_fmaf(axv[o1 + a], v[a], dw0);
#pragma unroll
                            for (int a = 0; a < n1; ++a) dw0 = __builtin_fmaf(xv[o1 + a], v2[a], dw0);
                            const float dwv[1] = {dw0};
                            bstore<1, kStream>(gwr, voff, (uint32_t)p * opaque_u32((uint32_t)C * 4u), dwv);
#pragma unroll
                            for (int a = 0; a < n1; ++a) {
                                gxa[o1 + a] = __builtin_fmaf(awv[p], v[a], gxa[o1 + a]);
                                gxa[o1 + a] = __builtin_fmaf(wv[p], v2[a], gxa[o1 + a]);
                                pin_f32(gxa[o1 + a]);
                            }
                            if constexpr (S::P >= 20) __builtin_amdgcn_sched_barrier(0);
                        });
                        __builtin_amdgcn_sched_barrier(0);
                        // (b) gY per path: u_p = w_p ax + aw_p x, then B_p(u_p, g) accumulated
                        // straight into gY.  Weighting before the contraction halves the
                        // coupling work, and accumulating each non-zero into gY needs no
                        // per-path partial sums: at L=3 1,534 instead of 2,046 operations per
                        // (edge, channel) for gY.
                        static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
                            constexpr int p = pp.p[decltype(kI)::value];
                            constexpr int o2 = S::paths[p].l2 * S::paths[p].l2;
                            float u[n1];
#pragma unroll
                            for (int q = 0; q < n1; ++q) u[q] = __builtin_fmaf(awv[p], xv[o1 + q], wv[p] * axv[o1 + q]);
                            static_for<n1>([&](auto aI) __attribute__((always_inline)) {
                                constexpr int q = decltype(aI)::value;
                                constexpr int z0 = nz_m1_begin<S>(p, q), z1 = nz_m1_begin<S>(p, q + 1);
                                static_for<z1 - z0>([&](auto zI) __attribute__((always_inline)) {
                                    constexpr int n = z0 + decltype(zI)::value;
                                    constexpr CgNz nzv = S::nz[n];
                                    const float prod = u[q] * gv[o3 + nzv.m3];
                                    gya[o2 + nzv.m2] = __builtin_fmaf(nzv.c, prod, gya[o2 + nzv.m2]);
                                });
                            });
                            if constexpr (S::P >= 20) __builtin_amdgcn_sched_barrier(0);
                        });
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            });

            // next edge's rows into the registers just freed (zeros after the last)
#pragma unroll
            for (int d = 0; d < D2; ++d) pin_f32(gya[d]);
            const long e_cur = e;
            const int kn = has_next ? k + 1 : k;
            e = send_perm[kn];
            const int tt = (int)opaque_lane((uint32_t)tid);
            const int ln = tt & 63;
            const float yn = sh_load<D2, false>(Y, e, tt), an = sh_load<D2, false>(aY, e, tt);
            load_edge(send_recv[kn], e, has_next ? voff : kOffLane);
            __builtin_amdgcn_sched_barrier(0);

            // gY: lanes (fixed-order halving), then waves (LDS, fixed order)
            const float r = wave_sum16(gya, ln);
            if (sum16_holder(ln)) sRed[tt >> 6][sum16_index(ln)] = r;
            if (has_next && tt < D2) {
                sY[buf ^ 1][0][tt] = yn;
                sY[buf ^ 1][1][tt] = an;
            }
            __syncthreads();
            if (has_next) {
                build_T_lds<S>(sT[buf ^ 1][0], sY[buf ^ 1][0], sTab, tt, nth);
                build_T_lds<S>(sT[buf ^ 1][1], sY[buf ^ 1][1], sTab, tt, nth);
            }
            if (tt < D2) {
                float tot = sRed[0][tt];
                for (int q = 1; q < nwaves; ++q) tot += sRed[q][tt];
                if (gy_atomic) unsafeAtomicAdd(gY + e_cur * D2 + tt, tot);
                else gY[e_cur * D2 + tt] = tot;
            }
            __syncthreads();
        }
    }
    store_row_stream<D1>(make_row(gx + (long)j * D1 * C, (long)D1 * C), voff, opaque_u32((uint32_t)C * 4u), gxa);
}

template <class S>
hipError_t dd_launch(const DoubleArgs& a, hipStream_t st) {
    // receivers: one channel per lane, up to 4 waves per tile
    {
        const int need = (a.C + 63) / 64;
        const int waves = need < kDdRecvMaxThreads / 64 ? need : kDdRecvMaxThreads / 64;
        const int tiles = (need + waves - 1) / waves;
        hipLaunchKernelGGL((k_dd_recv<S>), dim3(a.n_nodes, tiles), dim3(64 * waves), 0, st, a.C, a.x, a.ax, a.y,
                           a.ay, a.w, a.aw, a.row_ptr, a.senders, a.g_grad);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    // senders: the channels of a sender in one workgroup per tile (fixed-order gY)
    const int tiles = (a.C + kDdSendMaxThreads - 1) / kDdSendMaxThreads;
    const int waves = ((a.C + tiles - 1) / tiles + 63) / 64;
    if (tiles > 1 && a.n_edges > 0)
        hipLaunchKernelGGL(k_fill0, dim3(1024), dim3(256), 0, st, a.g_y, (long)a.n_edges * S::D2);
    hipLaunchKernelGGL((k_dd_send<S>), dim3(a.n_nodes, tiles), dim3(64 * waves), 0, st, a.C, a.grad, a.x, a.ax, a.y,
                       a.ay, a.w, a.aw, a.send_ptr, a.send_perm, a.send_recv, a.g_x, a.g_w, a.g_y,
                       (int)(tiles > 1));
    return hipGetLastError();
}

}  // namespace conv
}  // namespace ctp
