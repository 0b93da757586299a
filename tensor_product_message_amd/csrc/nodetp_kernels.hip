// Node-local channelwise tensor product (gfx950): the convolution's couplings
// applied at each node to two of its own features, with per-node weights
// (e3j, arXiv 2609.35099, abstract: tensor-product operations measured against
// HBM bandwidth; FlashCart, arXiv 2610.06409, section 4: node-local products
// beside the edge convolutions):
//
//   out[i, l3 m3, c] = sum_{p = (l1,l2,l3)} w[i,p,c]
//                      sum_{m1,m2} C_p[m1][m2][m3] x[i, l1 m1, c] y[i, l2 m2, c]
//
// Layout: x[N][D1][C], y[N][D2][C], w[N][P][C], out[N][D3][C], channel fastest.
// Every (node, channel) is independent: one lane per channel, one wave per
// (node, 64-channel block), each row read once through a buffer resource with
// non-temporal loads and stores (a pure stream; nothing is reused).  The
// coupling non-zeros are instruction constants of the unrolled path loops.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace ctp {
namespace {

constexpr int kNodeThreads = 256;   // 4 (node, channel block) items per workgroup

// True if non-zero n is the first of its path to touch m3 (resp. m1): the first
// product initialises a partial sum instead of accumulating.
template <class S>
constexpr bool nz_first_m3(int n) {
    for (int u = nz_begin<S>(S::nz[n].p); u < n; ++u)
        if (S::nz[u].m3 == S::nz[n].m3) return false;
    return true;
}
template <class S>
constexpr bool nz_first_m1(int n) {
    for (int u = nz_begin<S>(S::nz[n].p); u < n; ++u)
        if (S::nz[u].m1 == S::nz[n].m1) return false;
    return true;
}

// Paths sharing (l1, l2) form one run of the lexicographic path list.
struct PathRun {
    int p0, n;
};
template <class S>
constexpr PathRun paths_l1l2(int l1, int l2) {
    PathRun r{0, 0};
    for (int p = 0; p < S::P; ++p)
        if (S::paths[p].l1 == l1 && S::paths[p].l2 == l2) {
            if (r.n == 0) r.p0 = p;
            ++r.n;
        }
    return r;
}

// Item -> (node, lane offset); lanes past C read zeros and drop their stores.
struct Item {
    long node;
    uint32_t voff;
    bool valid;
};

__device__ __forceinline__ Item node_item(int n_nodes, int C) {
    const int nblk = (C + 63) >> 6;
    const long t = (long)blockIdx.x * (kNodeThreads / 64) + (threadIdx.x >> 6);
    Item it;
    it.node = t / nblk;
    const int c = (int)(t - it.node * nblk) * 64 + (int)(threadIdx.x & 63);
    it.valid = it.node < n_nodes;
    it.voff = opaque_lane(c < C ? (uint32_t)c * 4u : kOffLane);
    return it;
}

template <int D>
__device__ __forceinline__ void load_rows(const float* base, long node, int C, uint32_t voff, float (&v)[D]) {
    const rsrc_t r = make_row(base + node * D * C, (long)D * C);
    const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
#pragma unroll
    for (int d = 0; d < D; ++d) {
        float t[1];
        bload<1, kStream>(r, voff, (uint32_t)d * c4, t);
        v[d] = t[0];
    }
}

template <int D>
__device__ __forceinline__ void store_rows(float* base, long node, int C, uint32_t voff, const float (&v)[D]) {
    const rsrc_t r = make_row(base + node * D * C, (long)D * C);
    const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const float t[1] = {v[d]};
        bstore<1, kStream>(r, voff, (uint32_t)d * c4, t);
    }
}

// u_p[m3] = sum_{m1,m2} C_p x[l1 m1] y[l2 m2] for the paths of one (l1, l2)
// run, from products x[m1] * y[m2] formed m1 by m1 and shared by the run.
template <class S, int l1, int l2, class F>
__device__ __forceinline__ void couple_xy(const float (&x)[S::D1], const float (&y)[S::D2], F&& per_path) {
    constexpr PathRun run = paths_l1l2<S>(l1, l2);
    if constexpr (run.n > 0) {
        constexpr int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, o1 = l1 * l1, o2 = l2 * l2;
        float u[kMaxL + 1][2 * kMaxL + 1];
        static_for<n1>([&](auto aI) __attribute__((always_inline)) {
            constexpr int a = decltype(aI)::value;
            float pr[n2];
#pragma unroll
            for (int b = 0; b < n2; ++b) pr[b] = x[o1 + a] * y[o2 + b];
            static_for<run.n>([&](auto kI) __attribute__((always_inline)) {
                constexpr int k = decltype(kI)::value;
                constexpr int p = run.p0 + k;
                constexpr int z0 = nz_m1_begin<S>(p, a), z1 = nz_m1_begin<S>(p, a + 1);
                static_for<z1 - z0>([&](auto zI) __attribute__((always_inline)) {
                    constexpr int n = z0 + decltype(zI)::value;
                    constexpr CgNz q = S::nz[n];
                    if constexpr (nz_first_m3<S>(n))
                        u[k][q.m3] = q.c * pr[q.m2];
                    else
                        u[k][q.m3] = __builtin_fmaf(q.c, pr[q.m2], u[k][q.m3]);
                });
            });
        });
        static_for<run.n>([&](auto kI) __attribute__((always_inline)) {
            constexpr int k = decltype(kI)::value;
            per_path(std::integral_constant<int, run.p0 + k>{}, u[k]);
        });
    }
}

template <int L>
__global__ void __launch_bounds__(kNodeThreads)
k_node_fwd(int n_nodes, int C, const float* __restrict__ x, const float* __restrict__ y,
           const float* __restrict__ w, float* __restrict__ out) {
    using S = Spec<L, L, L>;
    const Item it = node_item(n_nodes, C);
    if (!it.valid) return;
    float xv[S::D1], yv[S::D2], wv[S::P], acc[S::D3];
    load_rows<S::D1>(x, it.node, C, it.voff, xv);
    load_rows<S::D2>(y, it.node, C, it.voff, yv);
    load_rows<S::P>(w, it.node, C, it.voff, wv);
#pragma unroll
    for (int d = 0; d < S::D3; ++d) acc[d] = 0.0f;
    static_for<L + 1>([&](auto l1I) __attribute__((always_inline)) {
        static_for<L + 1>([&](auto l2I) __attribute__((always_inline)) {
            couple_xy<S, decltype(l1I)::value, decltype(l2I)::value>(
                xv, yv, [&](auto pI, const float (&u)[2 * kMaxL + 1]) __attribute__((always_inline)) {
                    constexpr int p = decltype(pI)::value;
                    constexpr int l3 = S::paths[p].l3, o3 = l3 * l3;
#pragma unroll
                    for (int k = 0; k < 2 * l3 + 1; ++k) acc[o3 + k] = __builtin_fmaf(wv[p], u[k], acc[o3 + k]);
                });
        });
    });
    store_rows<S::D3>(out, it.node, C, it.voff, acc);
}

// Backward for upstream gradient g = dL/dout:
//   dw[i,p]     = sum_m3 g[l3 m3] u_p[m3]              (u_p as in the forward)
//   dx[i,l1 m1] += w_p sum_{m2,m3} C_p y[l2 m2] g[l3 m3]
//   dy[i,l2 m2] += w_p sum_{m1,m3} C_p x[l1 m1] g[l3 m3]
// Each sum is formed from products shared by the paths that pair the same two
// blocks: x*y per (l1, l2), y*g per (l2, l3), x*g per (l1, l3).
template <int L>
__global__ void __launch_bounds__(kNodeThreads)
k_node_bwd(int n_nodes, int C, const float* __restrict__ G, const float* __restrict__ x,
           const float* __restrict__ y, const float* __restrict__ w, float* __restrict__ dx,
           float* __restrict__ dy, float* __restrict__ dw) {
    using S = Spec<L, L, L>;
    const Item it = node_item(n_nodes, C);
    if (!it.valid) return;
    float xv[S::D1], yv[S::D2], wv[S::P], gv[S::D3];
    load_rows<S::D1>(x, it.node, C, it.voff, xv);
    load_rows<S::D2>(y, it.node, C, it.voff, yv);
    load_rows<S::D3>(G, it.node, C, it.voff, gv);
    load_rows<S::P>(w, it.node, C, it.voff, wv);

    // dw from the forward's per-path sums
    float dwv[S::P];
    static_for<L + 1>([&](auto l1I) __attribute__((always_inline)) {
        static_for<L + 1>([&](auto l2I) __attribute__((always_inline)) {
            couple_xy<S, decltype(l1I)::value, decltype(l2I)::value>(
                xv, yv, [&](auto pI, const float (&u)[2 * kMaxL + 1]) __attribute__((always_inline)) {
                    constexpr int p = decltype(pI)::value;
                    constexpr int l3 = S::paths[p].l3, o3 = l3 * l3;
                    float s = gv[o3] * u[0];
#pragma unroll
                    for (int k = 1; k < 2 * l3 + 1; ++k) s = __builtin_fmaf(gv[o3 + k], u[k], s);
                    dwv[p] = s;
                });
        });
    });
    store_rows<S::P>(dw, it.node, C, it.voff, dwv);

    // dy: products x[m1] g[m3] per (l1, l3), non-zeros of each path taken m1 by m1
    float dyv[S::D2];
#pragma unroll
    for (int d = 0; d < S::D2; ++d) dyv[d] = 0.0f;
    static_for<L + 1>([&](auto l1I) __attribute__((always_inline)) {
        constexpr int l1 = decltype(l1I)::value;
        static_for<L + 1>([&](auto l3I) __attribute__((always_inline)) {
            constexpr int l3 = decltype(l3I)::value;
            constexpr PairPaths pp = pair_paths<S>(l1, l3);
            if constexpr (pp.n > 0) {
                constexpr int n1 = 2 * l1 + 1, n3 = 2 * l3 + 1, o1 = l1 * l1, o3 = l3 * l3;
                float B[kMaxL + 1][2 * kMaxL + 1];
                static_for<n1>([&](auto aI) __attribute__((always_inline)) {
                    constexpr int a = decltype(aI)::value;
                    float pr[n3];
#pragma unroll
                    for (int b = 0; b < n3; ++b) pr[b] = xv[o1 + a] * gv[o3 + b];
                    static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
                        constexpr int k = decltype(kI)::value;
                        constexpr int p = pp.p[k];
                        constexpr int z0 = nz_m1_begin<S>(p, a), z1 = nz_m1_begin<S>(p, a + 1);
                        static_for<z1 - z0>([&](auto zI) __attribute__((always_inline)) {
                            constexpr int n = z0 + decltype(zI)::value;
                            constexpr CgNz q = S::nz[n];
                            if constexpr (nz_first_m2<S>(n))
                                B[k][q.m2] = q.c * pr[q.m3];
                            else
                                B[k][q.m2] = __builtin_fmaf(q.c, pr[q.m3], B[k][q.m2]);
                        });
                    });
                });
                static_for<pp.n>([&](auto kI) __attribute__((always_inline)) {
                    constexpr int k = decltype(kI)::value;
                    constexpr int p = pp.p[k];
                    constexpr int l2 = S::paths[p].l2, o2 = l2 * l2;
#pragma unroll
                    for (int b = 0; b < 2 * l2 + 1; ++b) dyv[o2 + b] = __builtin_fmaf(wv[p], B[k][b], dyv[o2 + b]);
                });
            }
        });
    });
    store_rows<S::D2>(dy, it.node, C, it.voff, dyv);

    // dx: products y[m2] g[m3] per (l2, l3); each path's non-zeros scanned per m2
    float dxv[S::D1];
#pragma unroll
    for (int d = 0; d < S::D1; ++d) dxv[d] = 0.0f;
    static_for<L + 1>([&](auto l2I) __attribute__((always_inline)) {
        constexpr int l2 = decltype(l2I)::value;
        static_for<L + 1>([&](auto l3I) __attribute__((always_inline)) {
            constexpr int l3 = decltype(l3I)::value;
            constexpr int n2 = 2 * l2 + 1, n3 = 2 * l3 + 1, o2 = l2 * l2, o3 = l3 * l3;
            static_for<S::P>([&](auto pI) __attribute__((always_inline)) {
                constexpr int p = decltype(pI)::value;
                if constexpr (S::paths[p].l2 == l2 && S::paths[p].l3 == l3) {
                    constexpr int l1 = S::paths[p].l1, o1 = l1 * l1;
                    constexpr int z0 = nz_begin<S>(p), z1 = nz_begin<S>(p + 1);
                    float A[2 * kMaxL + 1];
                    static_for<n2>([&](auto bI) __attribute__((always_inline)) {
                        constexpr int b = decltype(bI)::value;
                        float pr[n3];
#pragma unroll
                        for (int k = 0; k < n3; ++k) pr[k] = yv[o2 + b] * gv[o3 + k];
                        static_for<z1 - z0>([&](auto zI) __attribute__((always_inline)) {
                            constexpr int n = z0 + decltype(zI)::value;
                            constexpr CgNz q = S::nz[n];
                            if constexpr (q.m2 == b) {
                                if constexpr (nz_first_m1<S>(n))
                                    A[q.m1] = q.c * pr[q.m3];
                                else
                                    A[q.m1] = __builtin_fmaf(q.c, pr[q.m3], A[q.m1]);
                            }
                        });
                    });
#pragma unroll
                    for (int a = 0; a < 2 * l1 + 1; ++a) dxv[o1 + a] = __builtin_fmaf(wv[p], A[a], dxv[o1 + a]);
                }
            });
        });
    });
    store_rows<S::D1>(dx, it.node, C, it.voff, dxv);
}

}  // namespace

hipError_t launch_node_fwd(int L, int n_nodes, int C, const float* x, const float* y, const float* w, float* out,
                           hipStream_t st) {
    const long items = (long)n_nodes * ((C + 63) / 64);
    const dim3 grid((unsigned)((items + kNodeThreads / 64 - 1) / (kNodeThreads / 64))), block(kNodeThreads);
    switch (L) {
        case 0: hipLaunchKernelGGL(k_node_fwd<0>, grid, block, 0, st, n_nodes, C, x, y, w, out); break;
        case 1: hipLaunchKernelGGL(k_node_fwd<1>, grid, block, 0, st, n_nodes, C, x, y, w, out); break;
        case 2: hipLaunchKernelGGL(k_node_fwd<2>, grid, block, 0, st, n_nodes, C, x, y, w, out); break;
        case 3: hipLaunchKernelGGL(k_node_fwd<3>, grid, block, 0, st, n_nodes, C, x, y, w, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_node_bwd(int L, int n_nodes, int C, const float* G, const float* x, const float* y,
                           const float* w, float* dx, float* dy, float* dw, hipStream_t st) {
    const long items = (long)n_nodes * ((C + 63) / 64);
    const dim3 grid((unsigned)((items + kNodeThreads / 64 - 1) / (kNodeThreads / 64))), block(kNodeThreads);
    switch (L) {
        case 0: hipLaunchKernelGGL(k_node_bwd<0>, grid, block, 0, st, n_nodes, C, G, x, y, w, dx, dy, dw); break;
        case 1: hipLaunchKernelGGL(k_node_bwd<1>, grid, block, 0, st, n_nodes, C, G, x, y, w, dx, dy, dw); break;
        case 2: hipLaunchKernelGGL(k_node_bwd<2>, grid, block, 0, st, n_nodes, C, G, x, y, w, dx, dy, dw); break;
        case 3: hipLaunchKernelGGL(k_node_bwd<3>, grid, block, 0, st, n_nodes, C, G, x, y, w, dx, dy, dw); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ctp
