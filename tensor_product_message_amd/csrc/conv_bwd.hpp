// Backward kernels of the fused equivariant convolution tensor product
// (gfx950): the exact VJP (FlashCart, arXiv 2610.06409, section 3, symbolic
// VJPs) of
//   out[i, l3 m3, c] = sum_{e = j->i} sum_p w[e,p,c] sum_{m1} T_{p,e}[m1][m3] x[j, l1 m1, c]
// for the upstream gradient G = dL/dout: dx, dw, and dY (or dvec = J^T dY
// with edge vectors).  S = Spec<L1, L2, L3, V> as in the forward.
//
// K3 (k_bwd_sender): one workgroup per sender and channel tile walks the
// sender's out-edges in (send_ptr, send_perm) order, stable in CSR id (the
// sender ordering FlashCart's section 4 cites for deterministic gradients):
//   v_p[m1]      = sum_m3 T_p[m1][m3] G[i, l3 m3]
//   dw[e,p]      = sum_m1 x[j, l1 m1] v_p[m1]
//   dx[j, l1 m1] += w_p v_p[m1]                      (registers; stored once)
//   B_p[m2]      = sum_{m1,m3} C_p[m1][m2][m3] x[j, l1 m1] G[i, l3 m3]
//   dY[e, l2 m2] = sum_c sum_p w_p B_p[m2]           (lanes, then waves, fixed order)
//
// K3m (k_bwd_recv): the same products with the roles of the two nodes
// exchanged, for outputs whose G rows are much wider than x's: one workgroup
// per receiver keeps G[i] in registers, stores dw[e], dY[e] and the edge's dx
// message msg[e] = sum_p w_p v_p to a workspace; a second pass sums each
// sender's messages in sender-sorted order.
//
// Channels: up to 512 per workgroup (8 waves, one channel per lane).  Above
// that, two channel tiles (grid.z) each sum dY over their own channels and add
// the partial into a zeroed dY with fp32 atomics: two addends onto zero give
// fl(a + b) in either order, so dY stays bitwise reproducible.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace ctp {
namespace conv {

constexpr int kBwdMaxThreads = 512;   // backward workgroups: channels of one tile
constexpr int kBwdWavesPerEU = 3;

// ------------------------------------------------------------ per-edge building blocks

// G row of receiver i (or x row of sender j) and the w row of edge e.
template <int D, int P>
__device__ __forceinline__ void load_node_edge_rows(float (&nv)[D], float (&wv)[P], const float* __restrict__ node,
                                                    const float* __restrict__ w, long n, long e, int C,
                                                    uint32_t voff) {
    const rsrc_t nr = make_row(node + n * D * C, (long)D * C);
    const rsrc_t wr = make_row(w + e * P * C, (long)P * C);
    const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
#pragma unroll
    for (int d = 0; d < D; ++d) {
        float t[1];
        bload<1>(nr, voff, (uint32_t)d * c4, t);
        nv[d] = t[0];
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float t[1];
        bload<1, kStream>(wr, voff, (uint32_t)p * c4, t);
        wv[p] = t[0];
    }
}

// Paths in the order edge_backward consumes them (group by group), and back.
template <class S>
constexpr int path_at_pos(int k) {
    for (int g = 0; g < S::NG; ++g) {
        if (k < S::groups[g].n) return S::groups[g].p[k];
        k -= S::groups[g].n;
    }
    return -1;
}
template <class S>
constexpr int pos_of_path(int p) {
    int k = 0;
    for (int g = 0; g < S::NG; ++g)
        for (int i = 0; i < S::groups[g].n; ++i, ++k)
            if (S::groups[g].p[i] == p) return k;
    return -1;
}
template <class S>
constexpr int group_pos0(int g) {
    int k = 0;
    for (int i = 0; i < g; ++i) k += S::groups[i].n;
    return k;
}

// Window of w registers of the sender-major backward: half the paths when
// there are enough of them (P even and at least 32), else all (see
// edge_backward).
template <class S>
constexpr int bwd_window() {
    return (S::P >= 32 && S::P % 2 == 0) ? S::P / 2 : S::P;
}

// Register of path p's w: with the whole row (R = P) index p, else the
// path's position in consumption order modulo R.
template <class S, int R>
constexpr int w_slot(int p) {
    return R == S::P ? p : pos_of_path<S>(p) % R;
}

// G row of receiver n alone.
template <int D>
__device__ __forceinline__ void load_node_row(float (&nv)[D], const float* __restrict__ node, long n, int C,
                                              uint32_t voff) {
    const rsrc_t nr = make_row(node + n * D * C, (long)D * C);
    const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
#pragma unroll
    for (int d = 0; d < D; ++d) {
        float t[1];
        bload<1>(nr, voff, (uint32_t)d * c4, t);
        nv[d] = t[0];
    }
}

// One edge of the backward, given T = T(Y_e) in LDS, the sender's row x, the
// receiver's row g of G and the edge's row w (one channel per lane):
//   v_p = T_p^T g,  dw[e,p] = x . v_p (stored through dwr),  dxa += w_p v_p,
//   dya[l2 m2] += sum_p w_p B_p[m2],  B_p[m2] = sum C_p[m1][m2][m3] x[m1] g[m3].
// Work is grouped by the paths that read one block of G: for each group, v_p,
// dw_p and dx for its paths, then B_p from the products x[l1 m1] g[l3 m3]
// formed m1 by m1 and shared by the group's paths.  Scheduling barriers after
// each path and group bound register lifetimes.
// w: with R = P the caller loads the whole row (wv[p] = w[e,p]) and cw, nw,
// nvoff are unused.  With R < P (R divides P) wv is a window: the path at
// consumption position k reads register k mod R, and after each group its
// registers receive the rows R positions ahead, from this edge's row cw or,
// past the last position, from the next edge's row nw (nvoff out of range
// after the last edge: the loads return 0).  Each load then has about half an
// edge of arithmetic to arrive instead of the dY reduction between edges.
template <class S, int R>
__device__ __forceinline__ void edge_backward(const float* T, const float (&xv)[S::D1], const float (&gv)[S::DO],
                                              float (&wv)[R], rsrc_t dwr, uint32_t voff, int C,
                                              float (&dxa)[S::D1], float (&dya)[16], rsrc_t cw, rsrc_t nw,
                                              uint32_t nvoff) {
    static_assert(S::P % R == 0, "the window must divide the path count");
    constexpr bool kBig = S::P >= 20;   // bound register lifetimes more tightly in the large cases
    static_for<S::NG>([&](auto gI) __attribute__((always_inline)) {
        constexpr int gidx = decltype(gI)::value;
        constexpr PathGroup pp = S::groups[gidx];
        constexpr int l1 = pp.l1, l3 = pp.l3;
        constexpr int n1 = 2 * l1 + 1, n3 = 2 * l3 + 1;
        constexpr int o1 = l1 * l1, o3 = pp.o3;   // o3: the group's block of G
        // (a) v_p = T_p^T g, dw_p = x . v_p, dx += w_p v_p
        static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
            constexpr int p = pp.p[decltype(kI)::value];
            constexpr int ws = w_slot<S, R>(p);   // constexpr: folded, never a runtime index
            constexpr int t0 = S::slot_begin[p], t1 = S::slot_begin[p + 1];
            float v[n1];
            static_for<t1 - t0>([&](auto tI) __attribute__((always_inline)) {
                constexpr int t = t0 + decltype(tI)::value;
                constexpr TSlot s = S::slots[t];
                const float tv = slot_value<t>(T);
                if constexpr (first_m1<S>(t))
                    v[s.m1] = tv * gv[o3 + s.m3];
                else
                    v[s.m1] = __builtin_fmaf(tv, gv[o3 + s.m3], v[s.m1]);
            });
            float dwv[1];
            dwv[0] = xv[o1] * v[0];
#pragma unroll
            for (int a = 1; a < n1; ++a) dwv[0] = __builtin_fmaf(xv[o1 + a], v[a], dwv[0]);
            bstore<1, kStream>(dwr, voff, (uint32_t)p * opaque_u32((uint32_t)C * 4u), dwv);
#pragma unroll
            for (int a = 0; a < n1; ++a) {
                dxa[o1 + a] = __builtin_fmaf(wv[ws], v[a], dxa[o1 + a]);
                pin_f32(dxa[o1 + a]);
            }
            if constexpr (kBig) __builtin_amdgcn_sched_barrier(0);
        });
        __builtin_amdgcn_sched_barrier(0);
        // (b) B_p[m2] = sum C_p[m1][m2][m3] x[m1] g[m3], m1 outermost
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
            if constexpr (kBig) __builtin_amdgcn_sched_barrier(0);
        });
        // (c) dY partial sums
        static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
            constexpr int kk = decltype(kI)::value;
            constexpr int p = pp.p[kk];
            constexpr int n2 = 2 * S::paths[p].l2 + 1, o2 = S::paths[p].l2 * S::paths[p].l2;
            constexpr int ws = w_slot<S, R>(p);
#pragma unroll
            for (int b = 0; b < n2; ++b) dya[o2 + b] = __builtin_fmaf(wv[ws], B[kk][b], dya[o2 + b]);
        });
        if constexpr (R < S::P) {
#pragma unroll
            for (int d = 0; d < 16; ++d) pin_f32(dya[d]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (R < S::P) {
            // the group's w registers are free: the rows R positions ahead
            const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
            static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
                constexpr int k = group_pos0<S>(gidx) + decltype(kI)::value;
                constexpr int q = k + R;
                constexpr int pq = path_at_pos<S>(q < S::P ? q : q - S::P);
                float t[1];
                if constexpr (q < S::P)
                    bload<1, kStream>(cw, voff, (uint32_t)pq * c4, t);
                else
                    bload<1, kStream>(nw, nvoff, (uint32_t)pq * c4, t);
                wv[k % R] = t[0];
            });
            __builtin_amdgcn_sched_barrier(0);
        }
    });
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

// After an edge: dY summed over the workgroup's channels (lanes by fixed-order
// halving, then waves through LDS in wave order) while T of the next edge is
// built into Tn from its harmonics ynext (staged in Yn); wave 0 stores dY of
// edge e_cur, or with VEC dvec = J(vec)^T dY.  With two channel tiles
// (dy_atomic) the tile's partial is added into a zeroed dY / dvec instead.
// tt is the thread index.
template <class S, bool VEC>
__device__ __forceinline__ void edge_dy_finish(const float (&dya)[16], float (*sRed)[16], float* Tn, float* Yn,
                                               const SlotDev* sTab, const ShCoef* sSh, bool has_next, float ynext,
                                               int tt, int nth, int nwaves, const float* __restrict__ yv, long e_cur,
                                               float* __restrict__ dyv, bool dy_atomic) {
    constexpr int D2 = S::D2;
    const int ln = tt & 63;
    // dY: lanes (fixed-order halving), then waves (LDS, fixed order)
    const float r = wave_sum16(dya, ln);
    if (sum16_holder(ln)) sRed[tt >> 6][sum16_index(ln)] = r;
    if (has_next && tt < D2) Yn[tt] = ynext;
    __syncthreads();
    if (has_next) build_T_lds<S>(Tn, Yn, sTab, tt, nth);
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
                const float v = (gl - rg * rl) * inv;
                if (dy_atomic) unsafeAtomicAdd(dyv + 3 * e_cur + ln, v);
                else dyv[3 * e_cur + ln] = v;
            }
        }
    } else {
        if (tt < D2) {
            if (dy_atomic) unsafeAtomicAdd(dyv + e_cur * D2 + tt, tot);
            else dyv[e_cur * D2 + tt] = tot;
        }
    }
}

// ------------------------------------------------------------ K3: sender-sorted backward

// With one G slot per path (variant 1) the G row alone is D_out registers per
// channel, so that variant may take two waves per SIMD instead of spilling.
// SPLIT (small grids): blockIdx.y picks one half of the sender's out-edges;
// dx is added with fp32 atomics into a zeroed dx (two addends: order-free).
// blockIdx.z is the channel tile.
template <class S, bool VEC, bool SPLIT>
__global__ void __launch_bounds__(kBwdMaxThreads)
__attribute__((amdgpu_waves_per_eu(S::V == kVariantSlots ? 2 : kBwdWavesPerEU, 8)))
k_bwd_sender(int C, const float* __restrict__ G, const float* __restrict__ x, const float* __restrict__ yv,
             const float* __restrict__ w, const int* __restrict__ send_ptr, const int* __restrict__ send_perm,
             const int* __restrict__ send_recv, float* __restrict__ dx, float* __restrict__ dw,
             float* __restrict__ dyv, int dy_atomic) {
    constexpr int D1 = S::D1, D2 = S::D2, D3 = S::DO, P = S::P, NT = S::NT, NTP = (NT + 3) & ~3;
    __shared__ __attribute__((aligned(16))) float sT[2][NTP];
    __shared__ float sY[2][16];
    __shared__ float sRed[kBwdMaxThreads / 64][16];
    __shared__ SlotDev sTab[NT];
    __shared__ ShCoef sSh[VEC ? 16 : 1];   // harmonic coefficients, read per edge from LDS

    const int j = blockIdx.x;
    const int tid = threadIdx.x, nth = blockDim.x;
    const int nwaves = nth >> 6;
    const int c0 = blockIdx.z * nth + tid;
    const uint32_t voff = opaque_lane(c0 < C ? (uint32_t)c0 * 4u : kOffLane);   // no channel: loads 0, stores dropped

    float xv[D1], dxa[D1];
    {
        const rsrc_t xr = make_row(x + (long)j * D1 * C, (long)D1 * C);
#pragma unroll
        for (int d = 0; d < D1; ++d) {
            float t[1];
            bload<1, kStream>(xr, voff, (uint32_t)(d * C * 4), t);
            xv[d] = t[0];
            dxa[d] = 0.0f;
        }
    }

    int k0 = send_ptr[j], k1 = send_ptr[j + 1];
    if constexpr (SPLIT) {
        const int mid = k0 + (k1 - k0 + 1) / 2;
        if (blockIdx.y == 0) k1 = mid; else k0 = mid;
    }
    if (k0 < k1) {
        {
            const SlotDev* tab = slot_tab<S>();
            for (int t = tid; t < NT; t += nth) sTab[t] = tab[t];
            if constexpr (VEC)
                if (tid < 16) sSh[tid] = sh_tab().k[tid];
        }
        constexpr int R = bwd_window<S>();
        float gv[D3], wv[R];
        long e = send_perm[k0];
        const float y0 = sh_load<D2, VEC>(yv, e, tid);
        if constexpr (R == P) {
            load_node_edge_rows<D3, P>(gv, wv, G, w, send_recv[k0], e, C, voff);
        } else {
            // G row and the first R positions of the w row
            load_node_row<D3>(gv, G, send_recv[k0], C, voff);
            const rsrc_t wr = make_row(w + e * P * C, (long)P * C);
            const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
            static_for<R>([&](auto kI) __attribute__((always_inline)) {
                constexpr int pk = path_at_pos<S>(decltype(kI)::value);
                float t[1];
                bload<1, kStream>(wr, voff, (uint32_t)pk * c4, t);
                wv[decltype(kI)::value] = t[0];
            });
        }
        if (tid < D2) sY[0][tid] = y0;
        __syncthreads();
        build_T_lds<S>(sT[0], sY[0], sTab, tid, nth);
        __syncthreads();

        // Per out-edge k: compute with T(k) and the rows already in registers
        // (with a w window, w rows of this and the next edge are loaded during
        // the arithmetic); then load the G row (and with R = P the w row) of
        // edge k+1 into the same registers, reduce dY, and build T(k+1) in the
        // other buffer while those loads are in flight.
        for (int k = k0; k < k1; ++k) {
            const int buf = (k - k0) & 1;
            const bool has_next = k + 1 < k1;
            const int kn = has_next ? k + 1 : k;
            float dya[16];
#pragma unroll
            for (int d = 0; d < 16; ++d) dya[d] = 0.0f;
            {
                const rsrc_t cw = make_row(w + e * P * C, (long)P * C);
                const rsrc_t nw = make_row(w + (long)send_perm[kn] * P * C, (long)P * C);
                edge_backward<S, R>(sT[buf], xv, gv, wv, make_row(dw + e * P * C, (long)P * C), voff, C, dxa, dya,
                                    cw, nw, has_next ? voff : kOffLane);
            }
            // rows of the next edge into the registers just freed (unconditional:
            // after the last edge the loads use an out-of-range offset and return 0).
            // The dY sums are pinned first so the loads cannot be hoisted into the
            // arithmetic above, where their registers would still be in use.
#pragma unroll
            for (int d = 0; d < D2; ++d) pin_f32(dya[d]);
            const long e_cur = e;
            e = send_perm[kn];
            // A fresh copy of the thread index each edge keeps the address
            // arithmetic below from being hoisted out of the loop, where it would
            // hold registers through the arithmetic above.
            const int tt = (int)opaque_lane((uint32_t)tid);
            const float ynext = next_y<D2, VEC>(yv, e, tt, sSh);
            if constexpr (R == P)
                load_node_edge_rows<D3, P>(gv, wv, G, w, send_recv[kn], e, C, has_next ? voff : kOffLane);
            else
                load_node_row<D3>(gv, G, send_recv[kn], C, has_next ? voff : kOffLane);
            __builtin_amdgcn_sched_barrier(0);
            edge_dy_finish<S, VEC>(dya, sRed, sT[buf ^ 1], sY[buf ^ 1], sTab, sSh, has_next, ynext, tt, nth, nwaves,
                                   yv, e_cur, dyv, dy_atomic != 0);
            __syncthreads();
        }
    }

    if constexpr (SPLIT) {
        if (k0 < k1 && c0 < C) {
            float* o = dx + (long)j * D1 * C + c0;
#pragma unroll
            for (int d = 0; d < D1; ++d) unsafeAtomicAdd(o + (long)d * C, dxa[d]);
        }
    } else {
        const rsrc_t dxr = make_row(dx + (long)j * D1 * C, (long)D1 * C);
#pragma unroll
        for (int d = 0; d < D1; ++d) {
            const float t[1] = {dxa[d]};
            bstore<1, kStream>(dxr, voff, (uint32_t)(d * C * 4), t);
        }
    }
}

// ------------------------------------------------------------ K3m: receiver-major backward with edge messages

// ATOMIC_DX: each edge's message is added into dx[sender] (zeroed first) with
// fp32 atomics instead of being stored: no workspace and no second pass, but
// the order of the additions into dx varies from run to run.
template <class S, bool VEC, bool ATOMIC_DX>
__global__ void __launch_bounds__(kBwdMaxThreads)
__attribute__((amdgpu_waves_per_eu(S::V == kVariantSlots ? 2 : kBwdWavesPerEU, 8)))
k_bwd_recv(int C, const float* __restrict__ G, const float* __restrict__ x, const float* __restrict__ yv,
           const float* __restrict__ w, const int* __restrict__ row_ptr, const int* __restrict__ senders,
           float* __restrict__ msg, float* __restrict__ dw, float* __restrict__ dyv, int dy_atomic) {
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
    const int c0 = blockIdx.y * nth + tid;
    const uint32_t voff = opaque_lane(c0 < C ? (uint32_t)c0 * 4u : kOffLane);   // no channel: loads 0, stores dropped

    float gv[D3];
    {
        const rsrc_t gr = make_row(G + (long)i * D3 * C, (long)D3 * C);
#pragma unroll
        for (int d = 0; d < D3; ++d) {
            float t[1];
            bload<1, kStream>(gr, voff, (uint32_t)(d * C * 4), t);
            gv[d] = t[0];
        }
    }
    {
        const SlotDev* tab = slot_tab<S>();
        for (int t = tid; t < NT; t += nth) sTab[t] = tab[t];
        if constexpr (VEC)
            if (tid < 16) sSh[tid] = sh_tab().k[tid];
    }
    float xv[D1], wv[P];
    long e = k0;
    const float y0 = sh_load<D2, VEC>(yv, e, tid);
    load_node_edge_rows<D1, P>(xv, wv, x, w, senders[k0], e, C, voff);
    if (tid < D2) sY[0][tid] = y0;
    __syncthreads();
    build_T_lds<S>(sT[0], sY[0], sTab, tid, nth);
    __syncthreads();

    // Per in-edge: products with T(e) and the rows in registers, the message
    // stored, then the next edge's rows loaded while dY is reduced and T(e+1)
    // built in the other buffer.
    for (int k = k0; k < k1; ++k) {
        const int buf = (k - k0) & 1;
        const bool has_next = k + 1 < k1;
        float mx[D1], dya[16];
#pragma unroll
        for (int d = 0; d < D1; ++d) mx[d] = 0.0f;
#pragma unroll
        for (int d = 0; d < 16; ++d) dya[d] = 0.0f;
        {
            const rsrc_t dwr = make_row(dw + e * P * C, (long)P * C);
            edge_backward<S, P>(sT[buf], xv, gv, wv, dwr, voff, C, mx, dya, dwr, dwr, kOffLane);   // whole w rows
        }
        if constexpr (ATOMIC_DX) {
            if (c0 < C) {
                float* o = msg + (long)senders[e] * D1 * C + c0;   // msg = dx here
#pragma unroll
                for (int d = 0; d < D1; ++d) unsafeAtomicAdd(o + (long)d * C, mx[d]);
            }
        } else {
            const rsrc_t mr = make_row(msg + e * D1 * C, (long)D1 * C);
#pragma unroll
            for (int d = 0; d < D1; ++d) {
                const float t[1] = {mx[d]};
                bstore<1, kStream>(mr, voff, (uint32_t)(d * C * 4), t);
            }
        }
#pragma unroll
        for (int d = 0; d < D2; ++d) pin_f32(dya[d]);
        const long e_cur = e;
        e = has_next ? k + 1 : k;
        const int tt = (int)opaque_lane((uint32_t)tid);
        const float ynext = next_y<D2, VEC>(yv, e, tt, sSh);
        load_node_edge_rows<D1, P>(xv, wv, x, w, senders[e], e, C, has_next ? voff : kOffLane);
        __builtin_amdgcn_sched_barrier(0);
        edge_dy_finish<S, VEC>(dya, sRed, sT[buf ^ 1], sY[buf ^ 1], sTab, sSh, has_next, ynext, tt, nth, nwaves,
                               yv, e_cur, dyv, dy_atomic != 0);
        __syncthreads();
    }
}

// ------------------------------------------------------------ launchers

// Channel tiles of the backward: at most 512 channels per workgroup, at most
// two tiles (C <= 1024).
struct BwdTiles {
    int waves, tiles;
};
inline BwdTiles bwd_tiles(int C) {
    const int tiles = (C + kBwdMaxThreads - 1) / kBwdMaxThreads;
    const int per_tile = (C + tiles - 1) / tiles;
    return BwdTiles{(per_tile + 63) / 64, tiles};
}

constexpr long kBwdSplitBelowWaves = 4L * 1024;

template <class S, bool SPLIT>
hipError_t bwd_sender_launch(const LaunchArgs& a, const BwdTiles& t, hipStream_t st) {
    const dim3 grid(a.n_nodes, SPLIT ? 2 : 1, t.tiles), block(64 * t.waves);
    if (SPLIT) hipLaunchKernelGGL(k_fill0, dim3(1024), dim3(256), 0, st, a.dx, (long)a.n_nodes * S::D1 * a.C);
    if (a.vec_mode)
        hipLaunchKernelGGL((k_bwd_sender<S, true, SPLIT>), grid, block, 0, st, a.C, a.grad, a.x, a.y, a.w, a.send_ptr,
                           a.send_perm, a.send_recv, a.dx, a.dw, a.dy, (int)(t.tiles > 1));
    else
        hipLaunchKernelGGL((k_bwd_sender<S, false, SPLIT>), grid, block, 0, st, a.C, a.grad, a.x, a.y, a.w,
                           a.send_ptr, a.send_perm, a.send_recv, a.dx, a.dw, a.dy, (int)(t.tiles > 1));
    return hipGetLastError();
}

// dY (or dvec) zeroed before two channel tiles add their partials.
inline void zero_dy_for_tiles(const LaunchArgs& a, int tiles, int D2, hipStream_t st) {
    if (tiles > 1 && a.n_edges > 0)
        hipLaunchKernelGGL(k_fill0, dim3(1024), dim3(256), 0, st, a.dy, (long)a.n_edges * (a.vec_mode ? 3 : D2));
}

template <class S>
hipError_t bwd_launch(const LaunchArgs& a, hipStream_t st) {
    const BwdTiles t = bwd_tiles(a.C);
    zero_dy_for_tiles(a, t.tiles, S::D2, st);
    if constexpr (S::V == kVariantSummed)
        if ((long)a.n_nodes * t.waves * t.tiles < kBwdSplitBelowWaves) return bwd_sender_launch<S, true>(a, t, st);
    return bwd_sender_launch<S, false>(a, t, st);
}

// Pass 1 of the message backward (pass 2, the per-sender sums, is launched by
// the caller): dw, dY and msg[E][D1][C].
template <class S, bool ATOMIC_DX>
hipError_t recv_launch(const LaunchArgs& a, float* msg, hipStream_t st) {
    const BwdTiles t = bwd_tiles(a.C);
    zero_dy_for_tiles(a, t.tiles, S::D2, st);
    if (ATOMIC_DX) hipLaunchKernelGGL(k_fill0, dim3(1024), dim3(256), 0, st, msg, (long)a.n_nodes * S::D1 * a.C);
    if (a.n_edges == 0) return hipGetLastError();
    const dim3 grid(a.n_nodes, t.tiles), block(64 * t.waves);
    if (a.vec_mode)
        hipLaunchKernelGGL((k_bwd_recv<S, true, ATOMIC_DX>), grid, block, 0, st, a.C, a.grad, a.x, a.y, a.w,
                           a.row_ptr, a.senders, msg, a.dw, a.dy, (int)(t.tiles > 1));
    else
        hipLaunchKernelGGL((k_bwd_recv<S, false, ATOMIC_DX>), grid, block, 0, st, a.C, a.grad, a.x, a.y, a.w,
                           a.row_ptr, a.senders, msg, a.dw, a.dy, (int)(t.tiles > 1));
    return hipGetLastError();
}

template <class S>
hipError_t bwd_recv_launch(const LaunchArgs& a, float* msg, hipStream_t st) {
    return recv_launch<S, false>(a, msg, st);
}

// algo 1: receiver-major, messages added into dx with atomics.
template <class S>
hipError_t bwd_atomic_launch(const LaunchArgs& a, hipStream_t st) {
    return recv_launch<S, true>(a, a.dx, st);
}

}  // namespace conv
}  // namespace ctp
