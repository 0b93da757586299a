// Triple-independent kernels and the run-time dispatch of the convolution
// tensor product (gfx950).
//
// The convolution kernels themselves are compiled once per degree triple
// (convtp_triple.hip); this file selects Triple<l_in, l_sh, l_out> for a call,
// and holds the kernels that do not depend on the degrees of x and out: the
// per-sender sums of the message backward's second pass and the standalone
// harmonics (vec -> Y, dY -> dvec and the second-order terms for the VJP of
// the backward).
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace ctp {

static __constant__ ShTab kShTab = make_sh_tab();
__device__ __forceinline__ const ShTab& sh_tab() { return kShTab; }

namespace {

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

// ------------------------------------------------------------ dispatch over degree triples

// Calls f.template operator()<l_in, l_sh, l_out>() for the run-time degrees.
template <int K = 0, class F>
hipError_t by_triple(int key, F&& f) {
    if constexpr (K == 64) {
        return hipErrorInvalidValue;
    } else {
        if (key == K) return f.template operator()<K / 16, (K / 4) % 4, K % 4>();
        return by_triple<K + 1>(key, f);
    }
}

int triple_key(int l1, int l2, int l3) {
    if (l1 < 0 || l1 > kMaxL || l2 < 0 || l2 > kMaxL || l3 < 0 || l3 > kMaxL) return -1;
    return l1 * 16 + l2 * 4 + l3;
}

}  // namespace

hipError_t launch_fwd(const LaunchArgs& a, hipStream_t st) {
    if (a.n_nodes == 0) return hipSuccess;
    const int key = triple_key(a.l_in, a.l_sh, a.l_out);
    if (a.algo == 2)
        return by_triple(key, [&]<int A, int B, int C>() { return Triple<A, B, C>::fwd_frame(a, st); });
    return by_triple(key, [&]<int A, int B, int C>() { return Triple<A, B, C>::fwd(a, st); });
}

hipError_t launch_bwd(const LaunchArgs& a, hipStream_t st) {
    if (a.n_nodes == 0) return hipSuccess;
    if (a.algo == 2)
        return by_triple(triple_key(a.l_in, a.l_sh, a.l_out),
                         [&]<int A, int B, int C>() { return Triple<A, B, C>::bwd_frame(a, st); });
    if (a.algo == 1)
        return by_triple(triple_key(a.l_in, a.l_sh, a.l_out),
                         [&]<int A, int B, int C>() { return Triple<A, B, C>::bwd_atomic(a, st); });
    return by_triple(triple_key(a.l_in, a.l_sh, a.l_out),
                     [&]<int A, int B, int C>() { return Triple<A, B, C>::bwd(a, st); });
}

hipError_t launch_bwd_msg(const LaunchArgs& a, float* msg, hipStream_t st) {
    if (a.n_nodes == 0) return hipSuccess;
    const hipError_t e = by_triple(triple_key(a.l_in, a.l_sh, a.l_out),
                                   [&]<int A, int B, int C>() { return Triple<A, B, C>::bwd_recv(a, msg, st); });
    if (e != hipSuccess) return e;
    // dx rows of senders without out-edges come out zero
    const long row = (long)dim_of(a.l_in) * a.C;
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

hipError_t launch_bwd_dy(const LaunchArgs& a, hipStream_t st) {
    if (a.n_nodes == 0 || a.n_edges == 0) return hipSuccess;
    return by_triple(triple_key(a.l_in, a.l_sh, a.l_out),
                     [&]<int A, int B, int C>() { return Triple<A, B, C>::bwd_dy(a, st); });
}

hipError_t launch_double_bwd(const DoubleArgs& a, hipStream_t st) {
    if (a.n_nodes == 0) return hipSuccess;
    return by_triple(triple_key(a.l_in, a.l_sh, a.l_out),
                     [&]<int A, int B, int C>() { return Triple<A, B, C>::double_bwd(a, st); });
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
