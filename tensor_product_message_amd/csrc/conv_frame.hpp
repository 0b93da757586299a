// Edge-aligned-frame forward of the convolution tensor product (gfx950), for
// edge vectors (E2Former-V2, arXiv 2601.16622, abstract: equivariant products
// sparsified by working in each edge's own frame, SO(2) style).
//
// For edge e with unit direction r, any rotation R with R r = z-hat gives,
// with D^l = D^l(R) (Y_l(R v) = D^l Y_l(v)) and the coupling's equivariance
// C_p(D1 a, D2 b) = D3 C_p(a, b):
//
//   C_p(x, Y(r)) = C_p(x, D^T Y(z-hat)) = D3^T C_p(D1 x, Y(z-hat)),
//
// and Y_l2(z-hat) is non-zero only at m2 = 0 (value sqrt((2 l2 + 1) / 4pi)).
// So per edge and channel: x' = D x (84 FMA at l = 3), the m2 = 0 slice of
// every path's coupling (111 non-zeros at l = 3) scaled by w, summed per l3 in
// the frame, and one rotation back into the receiver's sum (84 FMA): about
// 400 FMA instead of the direct form's 665, and 84 broadcast LDS values per
// edge (D) instead of 541 (T).  The result equals the direct forward up to
// rounding.
//
// D^l comes from the harmonics themselves: with seven fixed directions v_j,
// M_l[a][j] = Y_la(v_j) has full row rank, so D^l = [Y_l(R v_j)]_j P_l with the
// constant right inverse P_l = M_l^T (M_l M_l^T)^-1 (compile-time tables).
// R is the shortest rotation taking r to z-hat (or to -z-hat followed by a
// half turn about x when r_z < 0).  A zero edge vector has Y = (1/sqrt(4pi),
// 0, ...): D = identity and the l2 >= 1 paths get weight 0.
//
// One workgroup per receiver and channel tile (up to four waves), one channel
// per lane, edges in CSR order with the same rotating prefetch as the direct
// forward; D of the next edge is built into the other LDS buffer after each
// edge.  SPLIT (small grids) halves each edge list as in the direct forward.
// With unequal degrees x is rotated up to l_in, the result back up to l_out,
// and the rotations are built up to the larger of the two.
#pragma once

#include <hip/hip_runtime.h>

#include "conv_bwd.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace ctp {
namespace conv {

constexpr int kFrameThreads = 256;
constexpr int kDirs = 7;                       // fixed directions v_j
constexpr int kDOff[4] = {0, 0, 9, 34};        // D^l blocks (l >= 1) in the flat D table
constexpr int kDEntries = 9 + 25 + 49;         // 83
constexpr int kDPad = 84;

// ------------------------------------------------------------ compile-time tables

// Seven unit-ish directions (normalised below) whose harmonics have full rank
// at l = 1, 2, 3 (condition numbers 2.2, 2.6, 2.8).
constexpr double kDirRaw[kDirs][3] = {
    {-0.8834895491600037, 0.03064717911183834, -0.46744731068611145},
    {-0.6929545402526855, 0.7203747034072876, 0.02956932224333286},
    {0.7007521390914917, 0.6210730671882629, 0.3510195314884186},
    {0.9977782368659973, 0.04325412213802338, 0.05067275837063789},
    {0.18411050736904144, -0.961883544921875, -0.20219644904136658},
    {0.23605982959270477, -0.8178870677947998, 0.5247251391410828},
    {-0.05702731758356094, -0.682953953742981, -0.7282319664955139},
};

// Real harmonic Y_{l,m} of a unit vector in double: the same recipe as the
// device tables (A_m(x, y) * N_lm * d^|m|/dz^|m| P_l(z)).
constexpr double sh_d(int l, int m, double x, double y, double z) {
    double Pl[4][4] = {};
    Pl[0][0] = 1.0;
    Pl[1][1] = 1.0;
    for (int n = 1; n < 3; ++n)
        for (int d = 0; d < 4; ++d) {
            double v = -n * Pl[n - 1][d];
            if (d > 0) v += (2 * n + 1) * Pl[n][d - 1];
            Pl[n + 1][d] = v / (n + 1);
        }
    const int a = m < 0 ? -m : m;
    double poly[4] = {Pl[l][0], Pl[l][1], Pl[l][2], Pl[l][3]};
    for (int r = 0; r < a; ++r)
        for (int d = 0; d < 4; ++d) poly[d] = (d + 1 < 4) ? (d + 1) * poly[d + 1] : 0.0;
    const double pi = 3.14159265358979323846;
    double N = csqrt((2 * l + 1) / (4 * pi) * cfact(l - a) / cfact(l + a));
    if (m != 0) N *= csqrt(2.0);
    const double q = ((poly[3] * z + poly[2]) * z + poly[1]) * z + poly[0];
    double re = 1.0, im = 0.0;
    for (int k = 0; k < a; ++k) {
        const double nr = re * x - im * y, ni = re * y + im * x;
        re = nr;
        im = ni;
    }
    return (m < 0 ? im : re) * N * q;
}

struct FrameTab {
    float v[kDirs][3];                 // normalised directions
    float p[kDirs][kDEntries];         // P_l[j][b] at p[j][kDOff[l] + b]
};

// P_l = M_l^T (M_l M_l^T)^-1, M_l[a][j] = Y_{l, a-l}(v_j); stored per l as
// p[j][kDOff[l] + b], b < 2l+1 (the first 2l+1 slots of each block).
constexpr FrameTab make_frame_tab() {
    FrameTab t{};
    double v[kDirs][3] = {};
    for (int j = 0; j < kDirs; ++j) {
        const double n = csqrt(kDirRaw[j][0] * kDirRaw[j][0] + kDirRaw[j][1] * kDirRaw[j][1] +
                               kDirRaw[j][2] * kDirRaw[j][2]);
        for (int c = 0; c < 3; ++c) {
            v[j][c] = kDirRaw[j][c] / n;
            t.v[j][c] = static_cast<float>(v[j][c]);
        }
    }
    for (int l = 1; l <= 3; ++l) {
        const int n = 2 * l + 1;
        double M[7][kDirs] = {};
        for (int a = 0; a < n; ++a)
            for (int j = 0; j < kDirs; ++j) M[a][j] = sh_d(l, a - l, v[j][0], v[j][1], v[j][2]);
        // G = M M^T, then its inverse by Gauss-Jordan with partial pivoting
        double G[7][14] = {};
        for (int a = 0; a < n; ++a) {
            for (int b = 0; b < n; ++b) {
                double s = 0.0;
                for (int j = 0; j < kDirs; ++j) s += M[a][j] * M[b][j];
                G[a][b] = s;
            }
            G[a][n + a] = 1.0;
        }
        for (int c = 0; c < n; ++c) {
            int piv = c;
            for (int r = c + 1; r < n; ++r)
                if (cabs(G[r][c]) > cabs(G[piv][c])) piv = r;
            for (int k = 0; k < 2 * n; ++k) {
                const double tmp = G[c][k];
                G[c][k] = G[piv][k];
                G[piv][k] = tmp;
            }
            const double inv = 1.0 / G[c][c];
            for (int k = 0; k < 2 * n; ++k) G[c][k] *= inv;
            for (int r = 0; r < n; ++r)
                if (r != c) {
                    const double f = G[r][c];
                    for (int k = 0; k < 2 * n; ++k) G[r][k] -= f * G[c][k];
                }
        }
        for (int j = 0; j < kDirs; ++j)
            for (int b = 0; b < n; ++b) {
                double s = 0.0;
                for (int a = 0; a < n; ++a) s += M[a][j] * G[a][n + b];
                t.p[j][kDOff[l] + b] = static_cast<float>(s);
            }
    }
    return t;
}

static __constant__ FrameTab kFrameTab = make_frame_tab();

// Y_{l2,0}(z-hat) = sqrt((2 l2 + 1) / 4pi).
constexpr float y_pole(int l2) {
    const double pi = 3.14159265358979323846;
    return static_cast<float>(csqrt((2 * l2 + 1) / (4 * pi)));
}

// One channel per lane: single-dword buffer accesses.
__device__ __forceinline__ float ld1(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kCached));
}
__device__ __forceinline__ float ld1_stream(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStream));
}
__device__ __forceinline__ void st1_stream(rsrc_t r, uint32_t voff, uint32_t soff, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, voff, soff, kStream);
}

// ------------------------------------------------------------ per-edge rotation D in LDS

// The rotation taking the direction of v to z-hat (rows of R); false for a
// zero vector.
__device__ __forceinline__ bool frame_rotation(float vx, float vy, float vz, float (&R)[3][3]) {
    const float n2 = vx * vx + vy * vy + vz * vz;
    if (n2 == 0.0f) return false;
    const float inv = 1.0f / sqrtf(n2);
    float x = vx * inv, y = vy * inv, z = vz * inv;
    const bool south = z < 0.0f;
    if (south) {   // take -r to z-hat, then a half turn about x (diag(1, -1, -1))
        x = -x;
        y = -y;
        z = -z;
    }
    const float k = 1.0f / (1.0f + z);   // z >= 0
    R[0][0] = 1.0f - x * x * k;
    R[0][1] = -x * y * k;
    R[0][2] = -x;
    R[1][0] = -x * y * k;
    R[1][1] = 1.0f - y * y * k;
    R[1][2] = -y;
    R[2][0] = x;
    R[2][1] = y;
    R[2][2] = 1.0f - (x * x + y * y) * k;
    if (south) {   // the half turn diag(1, -1, -1) after the map of -r to z-hat: R r = H (-z-hat) = z-hat
        for (int c = 0; c < 3; ++c) {
            R[1][c] = -R[1][c];
            R[2][c] = -R[2][c];
        }
    }
    return true;
}

// Builds D^1..D^L of edge vector vp into sD (kDPad floats) in two lane-parallel
// phases through sYR (directions, harmonic coefficients and P_l from their
// LDS copies: no global loads on the per-edge path); returns (uniformly)
// whether the vector is non-zero.  Leaves the workgroup synchronised.  (Moving
// the first phase ahead of the previous edge's arithmetic measured no faster.)
template <int L>
__device__ __forceinline__ bool build_frame(const float* __restrict__ vp, float* sD, float (*sYR)[16],
                                            const float (*sP)[kDEntries], const float (*sV)[3], const ShCoef* sSh,
                                            int tid, int nth) {
    constexpr int D = (L + 1) * (L + 1);
    float R[3][3];
    const bool nonzero = frame_rotation(vp[0], vp[1], vp[2], R);
    if (!nonzero) {   // no rotation: D = identity
        for (int t = tid; t < kDOff[L] + (2 * L + 1) * (2 * L + 1) && L > 0; t += nth) {
            const int l = t < 9 ? 1 : (t < 34 ? 2 : 3), n = 2 * l + 1, r = t - kDOff[l];
            sD[t] = (r / n == r % n) ? 1.0f : 0.0f;
        }
    } else {
        for (int t = tid; t < kDirs * D; t += nth) {
            const int j = t / D, k = t - j * D;
            const float* v = sV[j];
            const float ux = R[0][0] * v[0] + R[0][1] * v[1] + R[0][2] * v[2];
            const float uy = R[1][0] * v[0] + R[1][1] * v[1] + R[1][2] * v[2];
            const float uz = R[2][0] * v[0] + R[2][1] * v[1] + R[2][2] * v[2];
            sYR[j][k] = sh_component_c(k, sSh[k], ux, uy, uz);
        }
        __syncthreads();
        for (int t = tid; t < kDOff[L] + (2 * L + 1) * (2 * L + 1) && L > 0; t += nth) {
            const int l = t < 9 ? 1 : (t < 34 ? 2 : 3), n = 2 * l + 1, r = t - kDOff[l];
            const int a = r / n, b = r - a * n;
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < kDirs; ++j) s = __builtin_fmaf(sYR[j][l * l + a], sP[j][kDOff[l] + b], s);
            sD[t] = s;
        }
    }
    __syncthreads();
    return nonzero;
}

// ------------------------------------------------------------ forward kernel

constexpr int dflat(int l, int a, int b) {
    return kDOff[l] + a * (2 * l + 1) + b;
}

// One edge in its frame: x' = D x, m' = sum_p w_p * slice_p(x'), acc += D^T m';
// the rows of the next edge are loaded into x and w as they are freed.
template <class S>
__device__ __forceinline__ void edge_frame(float (&acc)[S::D3], float (&xv)[S::D1], float (&wv)[S::P],
                                           const float* sD, float f, rsrc_t nx, rsrc_t nw, uint32_t nvoff,
                                           int C) {
    constexpr int D = S::D1, D3 = S::D3;
    float xr[D];
    xr[0] = xv[0];
    static_for<S::L1>([&](auto lI) __attribute__((always_inline)) {
        constexpr int l = decltype(lI)::value + 1, n = 2 * l + 1, o = l * l;
        static_for<n>([&](auto aI) __attribute__((always_inline)) {
            constexpr int a = decltype(aI)::value;
            float s = slot_value<dflat(l, a, 0)>(sD) * xv[o];
            static_for<n - 1>([&](auto bI) __attribute__((always_inline)) {
                constexpr int b = decltype(bI)::value + 1;
                s = __builtin_fmaf(slot_value<dflat(l, a, b)>(sD), xv[o + b], s);
            });
            xr[o + a] = s;
        });
    });
    // x is consumed: the next sender's row goes into its registers
    {
        const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
#pragma unroll
        for (int d = 0; d < D; ++d) xv[d] = ld1(nx, nvoff, (uint32_t)d * c4);
    }
    float mr[D3];
#pragma unroll
    for (int d = 0; d < D3; ++d) mr[d] = 0.0f;
    static_for<S::P>([&](auto pI) __attribute__((always_inline)) {
        constexpr int p = decltype(pI)::value;
        constexpr PathL q = S::paths[p];
        constexpr int o1 = q.l1 * q.l1, o3 = q.l3 * q.l3;
        constexpr float yz = y_pole(q.l2);
        constexpr int n0 = nz_begin<S>(p), n1 = nz_begin<S>(p + 1);
        // f = 0 drops the l2 >= 1 paths for a zero edge vector (Y = Y_00 only)
        const float wp = q.l2 == 0 ? wv[p] : wv[p] * f;
        static_for<n1 - n0>([&](auto zI) __attribute__((always_inline)) {
            constexpr CgNz z = S::nz[n0 + decltype(zI)::value];
            if constexpr (z.m2 == q.l2) {   // the m2 = 0 component of block l2
                const float t = wp * xr[o1 + z.m1];
                mr[o3 + z.m3] = __builtin_fmaf(z.c * yz, t, mr[o3 + z.m3]);
            }
        });
        const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
        wv[p] = ld1_stream(nw, nvoff, (uint32_t)p * c4);
        __builtin_amdgcn_sched_barrier(0x100);
    });
    // re-read D from LDS for the way back rather than keep the 84 values of the
    // first rotation live in registers through the path loop
    asm volatile("" ::: "memory");
    acc[0] += mr[0];
    static_for<S::L3>([&](auto lI) __attribute__((always_inline)) {
        constexpr int l = decltype(lI)::value + 1, n = 2 * l + 1, o = l * l;
        static_for<n>([&](auto aI) __attribute__((always_inline)) {
            constexpr int a = decltype(aI)::value;
            static_for<n>([&](auto bI) __attribute__((always_inline)) {
                constexpr int b = decltype(bI)::value;
                acc[o + b] = __builtin_fmaf(slot_value<dflat(l, a, b)>(sD), mr[o + a], acc[o + b]);
            });
        });
    });
#pragma unroll
    for (int d = 0; d < D3; ++d) pin_f32(acc[d]);
}

template <class S, bool SPLIT>
__global__ void __launch_bounds__(kFrameThreads)
k_fwd_frame(int C, const float* __restrict__ x, const float* __restrict__ vec, const float* __restrict__ w,
            const int* __restrict__ row_ptr, const int* __restrict__ senders, float* __restrict__ out) {
    constexpr int D = S::D1, D3 = S::D3, P = S::P;
    constexpr int LD = S::L1 > S::L3 ? S::L1 : S::L3;   // rotations needed up to this degree
    __shared__ __attribute__((aligned(16))) float sD[2][kDPad];
    __shared__ float sYR[kDirs][16];
    __shared__ float sP[kDirs][kDEntries];
    __shared__ float sV[kDirs][3];
    __shared__ ShCoef sSh[16];

    const int i = blockIdx.x;
    const int tid = threadIdx.x, nth = blockDim.x;
    const int c0 = blockIdx.y * nth + tid;
    const uint32_t voff = opaque_lane(c0 < C ? (uint32_t)c0 * 4u : kOffLane);

    float acc[D3];
#pragma unroll
    for (int d = 0; d < D3; ++d) acc[d] = 0.0f;

    int e0 = row_ptr[i], e1 = row_ptr[i + 1];
    if constexpr (SPLIT) {
        const int mid = e0 + (e1 - e0 + 1) / 2;
        if (blockIdx.z == 0) e1 = mid; else e0 = mid;
    }
    if (e0 < e1) {
        float xv[D], wv[P];
        {
            const long j = senders[e0];
            const rsrc_t xr = make_row(x + j * D * C, (long)D * C);
            const rsrc_t wr = make_row(w + (long)e0 * P * C, (long)P * C);
            const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
#pragma unroll
            for (int d = 0; d < D; ++d) xv[d] = ld1(xr, voff, (uint32_t)d * c4);
#pragma unroll
            for (int p = 0; p < P; ++p)
                wv[p] = ld1_stream(wr, voff, (uint32_t)p * c4);
        }
        // per-edge constants into LDS once: P_l, the directions, the harmonic coefficients
        for (int t = tid; t < kDirs * kDEntries; t += nth) sP[t / kDEntries][t % kDEntries] = (&kFrameTab.p[0][0])[t];
        if (tid < kDirs * 3) sV[tid / 3][tid % 3] = kFrameTab.v[tid / 3][tid % 3];
        if (tid < 16) sSh[tid] = sh_tab().k[tid];
        __syncthreads();
        bool nonzero = build_frame<LD>(vec + 3L * e0, sD[0], sYR, sP, sV, sSh, tid, nth);
        for (int e = e0; e < e1; ++e) {
            const int buf = (e - e0) & 1;
            const bool has_next = e + 1 < e1;
            const long en = has_next ? e + 1 : e;
            const long jn = senders[en];
            const rsrc_t nx = make_row(x + jn * D * C, (long)D * C);
            const rsrc_t nw = make_row(w + en * P * C, (long)P * C);
            const uint32_t nvoff = has_next ? voff : kOffLane;
            edge_frame<S>(acc, xv, wv, sD[buf], nonzero ? 1.0f : 0.0f, nx, nw, nvoff, C);
            if (has_next) nonzero = build_frame<LD>(vec + 3 * en, sD[buf ^ 1], sYR, sP, sV, sSh, tid, nth);
        }
    }
    if constexpr (SPLIT) {
        if (e0 < e1 && c0 < C) {
            float* o = out + (long)i * D3 * C + c0;
#pragma unroll
            for (int d = 0; d < D3; ++d) unsafeAtomicAdd(o + (long)d * C, acc[d]);
        }
    } else {
        const rsrc_t orow = make_row(out + (long)i * D3 * C, (long)D3 * C);
#pragma unroll
        for (int d = 0; d < D3; ++d)
            st1_stream(orow, voff, (uint32_t)(d * C * 4), acc[d]);
    }
}

constexpr long kFrameSplitBelowWaves = 4L * 1024;

template <class S>
hipError_t frame_launch(const LaunchArgs& a, hipStream_t st) {
    const int waves_needed = (a.C + 63) / 64;
    const int waves = waves_needed < kFrameThreads / 64 ? waves_needed : kFrameThreads / 64;
    const int tiles = (waves_needed + waves - 1) / waves;
    const bool split = (long)a.n_nodes * tiles * waves < kFrameSplitBelowWaves;
    const dim3 block(64 * waves);
    if (split) {
        hipLaunchKernelGGL(k_fill0, dim3(1024), dim3(256), 0, st, a.out, (long)a.n_nodes * S::D3 * a.C);
        hipLaunchKernelGGL((k_fwd_frame<S, true>), dim3(a.n_nodes, tiles, 2), block, 0, st, a.C, a.x, a.y, a.w,
                           a.row_ptr, a.senders, a.out);
    } else {
        hipLaunchKernelGGL((k_fwd_frame<S, false>), dim3(a.n_nodes, tiles), block, 0, st, a.C, a.x, a.y, a.w,
                           a.row_ptr, a.senders, a.out);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------ backward in each edge's frame (edge vectors)
//
// The exact VJP of the frame forward above (equal to the direct backward up
// to rounding).  With D = D(R) of edge e (R r = z-hat), x' = D1 x[j] and
// g' = D3 G[i] (the gradient of the frame product m', since m = D3^T m'):
//   v'_p[m1] = y_pole(l2) sum_m3 C_p[m1][0][m3] g'[m3]      (m2 = 0 slice)
//   dw[e,p]  = x' . v'_p,   dx'[m1] += w_p v'_p[m1],   dx[j] += D1^T dx'
//   dY'[l2, m2] = sum_c sum_p w_p sum C_p[m1][m2][m3] x'[m1] g'[m3]
// dY' = D2 dY is the harmonic gradient in the frame.  Only its m2 = +-1
// components have a gradient across the edge direction at z-hat (the m2 = 0
// ones are radial there, all others vanish), so the edge-vector gradient is
//   dvec = R^T (sum_l c_l dY'[l, +1], sum_l c_l dY'[l, -1], 0) / |v|,
// c_l = dY_{l,1}/dx (z-hat) = dY_{l,-1}/dy (z-hat) = sqrt((2l+1) l (l+1) / (8 pi)),
// and only those 2 L2 components are formed and summed over channels.  Per
// (edge, channel) at L = 3: 84 + 84 FMAs to rotate x and G, 111 for v', 124 +
// 124 for dw and dx', 388 for the m2 = +-1 products and 84 to rotate dx back,
// about 1,000 against the direct backward's 1,876.  A zero edge vector takes
// D = identity, weight 0 on the l2 >= 1 paths (its Y is Y_00 alone) and dvec = 0.

// c_l above, l >= 1
constexpr float pole_grad(int l) {
    const double pi = 3.14159265358979323846;
    return static_cast<float>(csqrt((2 * l + 1) * l * (l + 1) / (8.0 * pi)));
}

// The m2 = 0 slice of path p (non-zeros of C_p with m2 at the block centre):
// whether non-zero n is the first of the slice with its m1, and whether the
// slice reaches m1 at all.
template <class S>
constexpr bool slice0_first_m1(int p, int n) {
    for (int u = nz_begin<S>(p); u < n; ++u)
        if (S::nz[u].m2 == S::paths[p].l2 && S::nz[u].m1 == S::nz[n].m1) return false;
    return true;
}
template <class S>
constexpr bool slice0_reaches(int p, int m1) {
    for (int u = nz_begin<S>(p); u < nz_begin<S>(p + 1); ++u)
        if (S::nz[u].m2 == S::paths[p].l2 && S::nz[u].m1 == m1) return true;
    return false;
}
template <class S>
constexpr int slice0_first_reached(int p) {
    for (int a = 0; a < 2 * S::paths[p].l1 + 1; ++a)
        if (slice0_reaches<S>(p, a)) return a;
    return -1;
}

// First non-zero of path p's slice m2 (-1 if none), and whether some path of
// group g reaches the product x'[m1] g'[m3] through an m2 = +-1 slice.
template <class S>
constexpr int slice_first_nz(int p, int m2) {
    for (int u = nz_begin<S>(p); u < nz_begin<S>(p + 1); ++u)
        if (S::nz[u].m2 == m2) return u;
    return -1;
}
template <class S>
constexpr bool group_pm1_reaches(PathGroup g, int m1, int m3) {
    for (int k = 0; k < g.n; ++k) {
        const int p = g.p[k], l2 = S::paths[p].l2;
        if (l2 == 0) continue;
        for (int u = nz_begin<S>(p); u < nz_begin<S>(p + 1); ++u)
            if ((S::nz[u].m2 == l2 - 1 || S::nz[u].m2 == l2 + 1) && S::nz[u].m1 == m1 && S::nz[u].m3 == m3)
                return true;
    }
    return false;
}

// One edge in its frame, one channel per lane; D of the edge in LDS, f = 0 for
// a zero vector (1 otherwise).  dya[2 (l2 - 1) + s] collects dY'[l2, m2 = -1
// (s = 0) or +1 (s = 1)] for l2 >= 1.
template <class S>
__device__ __forceinline__ void edge_frame_backward(const float* sD, float f, const float (&xv)[S::D1],
                                                    const float (&gv)[S::D3], const float (&wv)[S::P], rsrc_t dwr,
                                                    uint32_t voff, int C, float (&dxa)[S::D1], float (&dya)[6]) {
    // g' = D3 g (the l = 0 component is unrotated)
    float gr[S::D3];
    gr[0] = gv[0];
    static_for<S::L3>([&](auto lI) __attribute__((always_inline)) {
        constexpr int l = decltype(lI)::value + 1, n = 2 * l + 1, o = l * l;
        static_for<n>([&](auto aI) __attribute__((always_inline)) {
            constexpr int a = decltype(aI)::value;
            float s = slot_value<dflat(l, a, 0)>(sD) * gv[o];
            static_for<n - 1>([&](auto bI) __attribute__((always_inline)) {
                constexpr int b = decltype(bI)::value + 1;
                s = __builtin_fmaf(slot_value<dflat(l, a, b)>(sD), gv[o + b], s);
            });
            gr[o + a] = s;
        });
    });
    // l1 by l1: x'_l1 = D1 x_l1; then the path groups (l1, l3) of that l1, each
    // with the products x'[m1] g'[m3] its m2 = +-1 slices need formed once;
    // then dx_l1 += D1^T dx'_l1
    static_for<S::L1 + 1>([&](auto l1I) __attribute__((always_inline)) {
        constexpr int l1 = decltype(l1I)::value, n1 = 2 * l1 + 1, o1 = l1 * l1;
        float xr[n1], dxr[n1];
        if constexpr (l1 == 0) {
            xr[0] = xv[0];
        } else {
            static_for<n1>([&](auto aI) __attribute__((always_inline)) {
                constexpr int a = decltype(aI)::value;
                float s = slot_value<dflat(l1, a, 0)>(sD) * xv[o1];
                static_for<n1 - 1>([&](auto bI) __attribute__((always_inline)) {
                    constexpr int b = decltype(bI)::value + 1;
                    s = __builtin_fmaf(slot_value<dflat(l1, a, b)>(sD), xv[o1 + b], s);
                });
                xr[a] = s;
            });
        }
#pragma unroll
        for (int a = 0; a < n1; ++a) dxr[a] = 0.0f;
        static_for<S::NG>([&](auto gI) __attribute__((always_inline)) {
            constexpr PathGroup pg = S::groups[decltype(gI)::value];
            if constexpr (pg.l1 == l1) {
                constexpr int l3 = pg.l3, n3 = 2 * l3 + 1, o3 = l3 * l3;
                // x'[m1] g'[m3] for the pairs the group's +-1 slices reach
                float pr[n1][n3];
                static_for<n1 * n3>([&](auto kI) __attribute__((always_inline)) {
                    constexpr int a = decltype(kI)::value / n3, b = decltype(kI)::value % n3;
                    if constexpr (group_pm1_reaches<S>(pg, a, b)) pr[a][b] = xr[a] * gr[o3 + b];
                });
                static_for<pg.n>([&](auto kI) __attribute__((always_inline)) {
                    constexpr int p = pg.p[decltype(kI)::value];
                    constexpr PathL q = S::paths[p];
                    constexpr float yz = y_pole(q.l2);
                    constexpr int z0 = nz_begin<S>(p), z1 = nz_begin<S>(p + 1);
                    // v'_p over the m2 = 0 slice
                    float v[n1];
                    static_for<z1 - z0>([&](auto zI) __attribute__((always_inline)) {
                        constexpr int n = z0 + decltype(zI)::value;
                        constexpr CgNz z = S::nz[n];
                        if constexpr (z.m2 == q.l2) {
                            constexpr float c = z.c * yz;
                            if constexpr (slice0_first_m1<S>(p, n))
                                v[z.m1] = c * gr[o3 + z.m3];
                            else
                                v[z.m1] = __builtin_fmaf(c, gr[o3 + z.m3], v[z.m1]);
                        }
                    });
                    constexpr int a0 = slice0_first_reached<S>(p);
                    static_assert(a0 >= 0, "every path's m2 = 0 slice has a non-zero");
                    float dwv = xr[a0] * v[a0];
                    static_for<n1>([&](auto aI) __attribute__((always_inline)) {
                        constexpr int a = decltype(aI)::value;
                        if constexpr (a > a0 && slice0_reaches<S>(p, a)) dwv = __builtin_fmaf(xr[a], v[a], dwv);
                    });
                    float wf = wv[p];
                    if constexpr (q.l2 > 0) {   // weight 0 for a zero edge vector
                        dwv *= f;
                        wf *= f;
                    }
                    const float dwo[1] = {dwv};
                    bstore<1, kStream>(dwr, voff, (uint32_t)p * opaque_u32((uint32_t)C * 4u), dwo);
                    static_for<n1>([&](auto aI) __attribute__((always_inline)) {
                        constexpr int a = decltype(aI)::value;
                        if constexpr (slice0_reaches<S>(p, a)) dxr[a] = __builtin_fmaf(wf, v[a], dxr[a]);
                    });
                    // dY'[l2, -1] and dY'[l2, +1]
                    if constexpr (q.l2 > 0) {
                        float B[2];
                        static_for<2>([&](auto sI) __attribute__((always_inline)) {
                            constexpr int sgn = decltype(sI)::value, m2 = q.l2 - 1 + 2 * sgn;
                            constexpr int nf = slice_first_nz<S>(p, m2);
                            static_assert(nf >= 0, "the m2 = +-1 slices of an l2 >= 1 path have non-zeros");
                            B[sgn] = S::nz[nf].c * pr[S::nz[nf].m1][S::nz[nf].m3];
                            static_for<z1 - z0>([&](auto zI) __attribute__((always_inline)) {
                                constexpr int n = z0 + decltype(zI)::value;
                                constexpr CgNz z = S::nz[n];
                                if constexpr (n > nf && z.m2 == m2) B[sgn] = __builtin_fmaf(z.c, pr[z.m1][z.m3], B[sgn]);
                            });
                        });
                        dya[2 * (q.l2 - 1)] = __builtin_fmaf(wv[p], B[0], dya[2 * (q.l2 - 1)]);
                        dya[2 * (q.l2 - 1) + 1] = __builtin_fmaf(wv[p], B[1], dya[2 * (q.l2 - 1) + 1]);
                    }
                    if constexpr (S::P >= 20) __builtin_amdgcn_sched_barrier(0);
                });
            }
        });
        // dx_l1 += D1^T dx'_l1
        if constexpr (l1 == 0) {
            dxa[0] += dxr[0];
        } else {
            static_for<n1>([&](auto bI) __attribute__((always_inline)) {
                constexpr int b = decltype(bI)::value;
                static_for<n1>([&](auto aI) __attribute__((always_inline)) {
                    constexpr int a = decltype(aI)::value;
                    dxa[o1 + b] = __builtin_fmaf(slot_value<dflat(l1, a, b)>(sD), dxr[a], dxa[o1 + b]);
                });
            });
        }
#pragma unroll
        for (int a = 0; a < n1; ++a) pin_f32(dxa[o1 + a]);
    });
}

template <class S, bool SPLIT>
__global__ void __launch_bounds__(kBwdMaxThreads) __attribute__((amdgpu_waves_per_eu(kBwdWavesPerEU, 8)))
k_bwd_frame(int C, const float* __restrict__ G, const float* __restrict__ x, const float* __restrict__ vec,
            const float* __restrict__ w, const int* __restrict__ send_ptr, const int* __restrict__ send_perm,
            const int* __restrict__ send_recv, float* __restrict__ dx, float* __restrict__ dw,
            float* __restrict__ dvec, int dy_atomic) {
    constexpr int D1 = S::D1, D3 = S::D3, P = S::P;
    constexpr int LD = S::L1 > S::L3 ? S::L1 : S::L3;   // rotations needed up to this degree
    __shared__ __attribute__((aligned(16))) float sD[2][kDPad];
    __shared__ float sYR[kDirs][16];
    __shared__ float sP[kDirs][kDEntries];
    __shared__ float sV[kDirs][3];
    __shared__ ShCoef sSh[16];
    __shared__ float sRed[kBwdMaxThreads / 64][16];

    const int j = blockIdx.x;
    const int tid = threadIdx.x, nth = blockDim.x, nwaves = nth >> 6;
    const int c0 = blockIdx.z * nth + tid;
    const uint32_t voff = opaque_lane(c0 < C ? (uint32_t)c0 * 4u : kOffLane);

    float xv[D1], dxa[D1];
    {
        const rsrc_t xr = make_row(x + (long)j * D1 * C, (long)D1 * C);
#pragma unroll
        for (int d = 0; d < D1; ++d) {
            xv[d] = ld1_stream(xr, voff, (uint32_t)(d * C * 4));
            dxa[d] = 0.0f;
        }
    }
    int k0 = send_ptr[j], k1 = send_ptr[j + 1];
    if constexpr (SPLIT) {
        const int mid = k0 + (k1 - k0 + 1) / 2;
        if (blockIdx.y == 0) k1 = mid; else k0 = mid;
    }
    if (k0 < k1) {
        for (int t = tid; t < kDirs * kDEntries; t += nth) sP[t / kDEntries][t % kDEntries] = (&kFrameTab.p[0][0])[t];
        if (tid < kDirs * 3) sV[tid / 3][tid % 3] = kFrameTab.v[tid / 3][tid % 3];
        if (tid < 16) sSh[tid] = sh_tab().k[tid];
        __syncthreads();
        long e = send_perm[k0];
        float gv[D3], wv[P];
        {
            const rsrc_t gr = make_row(G + (long)send_recv[k0] * D3 * C, (long)D3 * C);
            const rsrc_t wr = make_row(w + e * P * C, (long)P * C);
            const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
#pragma unroll
            for (int d = 0; d < D3; ++d) gv[d] = ld1(gr, voff, (uint32_t)d * c4);
#pragma unroll
            for (int p = 0; p < P; ++p) wv[p] = ld1_stream(wr, voff, (uint32_t)p * c4);
        }
        bool nonzero = build_frame<LD>(vec + 3 * e, sD[0], sYR, sP, sV, sSh, tid, nth);
        for (int k = k0; k < k1; ++k) {
            const int buf = (k - k0) & 1;
            const bool has_next = k + 1 < k1;
            float dya[6] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
            edge_frame_backward<S>(sD[buf], nonzero ? 1.0f : 0.0f, xv, gv, wv, make_row(dw + e * P * C, (long)P * C),
                                   voff, C, dxa, dya);
#pragma unroll
            for (int d = 0; d < 6; ++d) pin_f32(dya[d]);
            // rows of the next edge into the registers just freed (zeros after the last)
            const long e_cur = e;
            const bool nz_cur = nonzero;
            const int kn = has_next ? k + 1 : k;
            e = send_perm[kn];
            {
                const uint32_t nvoff = has_next ? voff : kOffLane;
                const rsrc_t gr = make_row(G + (long)send_recv[kn] * D3 * C, (long)D3 * C);
                const rsrc_t wr = make_row(w + e * P * C, (long)P * C);
                const uint32_t c4 = opaque_u32((uint32_t)C * 4u);
#pragma unroll
                for (int d = 0; d < D3; ++d) gv[d] = ld1(gr, nvoff, (uint32_t)d * c4);
#pragma unroll
                for (int p = 0; p < P; ++p) wv[p] = ld1_stream(wr, nvoff, (uint32_t)p * c4);
            }
            __builtin_amdgcn_sched_barrier(0);
            // dY'[l2, +-1] over the channels: lanes (fixed-order halving), then waves
            const int tt = (int)opaque_lane((uint32_t)tid), ln = tt & 63;
            float r16[16];
#pragma unroll
            for (int d = 0; d < 16; ++d) r16[d] = d < 6 ? dya[d] : 0.0f;
            const float r = wave_sum16(r16, ln);
            if (sum16_holder(ln)) sRed[tt >> 6][sum16_index(ln)] = r;
            __syncthreads();
            if (tt < 3) {
                float tot[6];
#pragma unroll
                for (int d = 0; d < 6; ++d) {
                    tot[d] = sRed[0][d];
                    for (int q = 1; q < nwaves; ++q) tot[d] += sRed[q][d];
                }
                float gx = 0.0f, gy = 0.0f;
#pragma unroll
                for (int l = 1; l <= 3; ++l)
                    if (l <= S::L2) {
                        gy = __builtin_fmaf(pole_grad(l), tot[2 * (l - 1)], gy);       // m2 = -1
                        gx = __builtin_fmaf(pole_grad(l), tot[2 * (l - 1) + 1], gx);   // m2 = +1
                    }
                const float* vp = vec + 3 * e_cur;
                float R[3][3];
                frame_rotation(vp[0], vp[1], vp[2], R);
                const float n2 = vp[0] * vp[0] + vp[1] * vp[1] + vp[2] * vp[2];
                const float inv = nz_cur ? 1.0f / sqrtf(n2) : 0.0f;
                const float rl = tt == 0 ? R[0][0] * gx + R[1][0] * gy
                                         : (tt == 1 ? R[0][1] * gx + R[1][1] * gy : R[0][2] * gx + R[1][2] * gy);
                const float val = nz_cur ? rl * inv : 0.0f;
                if (dy_atomic) unsafeAtomicAdd(dvec + 3 * e_cur + tt, val);
                else dvec[3 * e_cur + tt] = val;
            }
            // the frame of the next edge (synchronises the workgroup, also for sRed)
            if (has_next) nonzero = build_frame<LD>(vec + 3 * e, sD[buf ^ 1], sYR, sP, sV, sSh, tid, nth);
            else __syncthreads();
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
        for (int d = 0; d < D1; ++d) st1_stream(dxr, voff, (uint32_t)(d * C * 4), dxa[d]);
    }
}

template <class S>
hipError_t frame_bwd_launch(const LaunchArgs& a, hipStream_t st) {
    const BwdTiles t = bwd_tiles(a.C);
    if (t.tiles > 1 && a.n_edges > 0)
        hipLaunchKernelGGL(k_fill0, dim3(1024), dim3(256), 0, st, a.dy, (long)a.n_edges * 3);
    const bool split = (long)a.n_nodes * t.waves * t.tiles < kBwdSplitBelowWaves;
    const dim3 block(64 * t.waves);
    if (split) {
        hipLaunchKernelGGL(k_fill0, dim3(1024), dim3(256), 0, st, a.dx, (long)a.n_nodes * S::D1 * a.C);
        hipLaunchKernelGGL((k_bwd_frame<S, true>), dim3(a.n_nodes, 2, t.tiles), block, 0, st, a.C, a.grad, a.x, a.y,
                           a.w, a.send_ptr, a.send_perm, a.send_recv, a.dx, a.dw, a.dy, (int)(t.tiles > 1));
    } else {
        hipLaunchKernelGGL((k_bwd_frame<S, false>), dim3(a.n_nodes, 1, t.tiles), block, 0, st, a.C, a.grad, a.x,
                           a.y, a.w, a.send_ptr, a.send_perm, a.send_recv, a.dx, a.dw, a.dy, (int)(t.tiles > 1));
    }
    return hipGetLastError();
}

}  // namespace conv
}  // namespace ctp
