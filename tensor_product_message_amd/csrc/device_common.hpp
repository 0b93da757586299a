// Device helpers shared by the conv tensor-product kernels: compile-time loops,
// wavefront reductions, the per-edge coupling-slot tables and the real
// spherical harmonics of an edge direction.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "tables.hpp"

namespace ctp {

// ------------------------------------------------------------ compile-time loops

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}

template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------ zero fill

// Zero fill of n floats (a kernel, not a memset, so that calls can be captured
// in a HIP graph); one copy per translation unit that launches it.
[[maybe_unused]] static __global__ void k_fill0(float* __restrict__ p, long n) {
    long k = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long stride = (long)gridDim.x * blockDim.x;
    for (; k < n; k += stride) p[k] = 0.0f;
}

// ------------------------------------------------------------ per-slot flags

// True if slot t is the first slot of its path that touches m3 (resp. m1):
// the first product initialises a partial sum instead of accumulating.
template <class S>
constexpr bool first_m3(int t) {
    for (int u = S::slot_begin[S::slots[t].p]; u < t; ++u)
        if (S::slots[u].m3 == S::slots[t].m3) return false;
    return true;
}
template <class S>
constexpr bool first_m1(int t) {
    for (int u = S::slot_begin[S::slots[t].p]; u < t; ++u)
        if (S::slots[u].m1 == S::slots[t].m1) return false;
    return true;
}

// First coupling non-zero of each path (and NNZ at the end).
template <class S>
constexpr int nz_begin(int p) {
    for (int n = 0; n < S::NNZ; ++n)
        if (S::nz[n].p >= p) return n;
    return S::NNZ;
}
template <class S>
constexpr bool nz_first_m2(int n) {
    for (int u = nz_begin<S>(S::nz[n].p); u < n; ++u)
        if (S::nz[u].m2 == S::nz[n].m2) return false;
    return true;
}

// First non-zero of path p with m1 >= a (non-zeros are sorted by m1, m2, m3).
template <class S>
constexpr int nz_m1_begin(int p, int a) {
    for (int n = nz_begin<S>(p); n < nz_begin<S>(p + 1); ++n)
        if (S::nz[n].m1 >= a) return n;
    return nz_begin<S>(p + 1);
}

// Paths sharing (l1, l3), in path order (at most kMaxL + 1 of them).
struct PairPaths {
    int n;
    int p[kMaxL + 1];
};
template <class S>
constexpr PairPaths pair_paths(int l1, int l3) {
    PairPaths r{0, {0, 0, 0, 0}};
    for (int p = 0; p < S::P; ++p)
        if (S::paths[p].l1 == l1 && S::paths[p].l3 == l3) r.p[r.n++] = p;
    return r;
}

// ------------------------------------------------------------ slot tables in device memory

// Lane-parallel build of T_p[m1][m3] = c1 * Y[y1] + c2 * Y[y2]; y1 | (y2 << 8).
struct SlotDev {
    int32_t yy;
    float c1, c2;
};

// One table per problem spec S (a Spec<L1, L2, L3, V>).
template <class S>
struct SlotTab {
    SlotDev s[S::NT];
};

template <class S>
constexpr SlotTab<S> make_slot_tab() {
    SlotTab<S> r{};
    for (int t = 0; t < S::NT; ++t)
        r.s[t] = SlotDev{S::slots[t].y1 | (S::slots[t].y2 << 8), S::slots[t].c1, S::slots[t].c2};
    return r;
}

// Device copy of S's slot table (defined next to the kernels that use it).
template <class S>
__device__ __forceinline__ const SlotDev* slot_tab();

// ------------------------------------------------------------ real spherical harmonics

// Component k = l*l + l + m of the real harmonics (orthonormal, no
// Condon-Shortley phase) of a unit vector (x, y, z):
//   Y_k = A_m(x, y) * Q_k(z),  A_m = Re (x+iy)^m (m>0), 1 (m=0), Im (x+iy)^|m| (m<0),
//   Q_k = N_lm * d^|m|/dz^|m| P_l(z), N_lm = sqrt((2l+1)/(4pi) (l-|m|)!/(l+|m|)!) (* sqrt2 if m != 0).
// Legendre polynomials come from Bonnet's recurrence; Q_k is stored as
// ascending power coefficients (degree <= 3) together with its derivative.
struct ShCoef {
    int32_t a;       // |m|
    int32_t sine;    // 1 if m < 0
    float q[4];      // Q_k(z) coefficients
    float dq[4];     // Q_k'(z) coefficients
};

struct ShTab {
    ShCoef k[16];
};

constexpr ShTab make_sh_tab() {
    // Legendre P_l in the power basis, l <= 3
    double Pl[4][4] = {};
    Pl[0][0] = 1.0;
    Pl[1][1] = 1.0;
    for (int n = 1; n < 3; ++n)
        for (int d = 0; d < 4; ++d) {
            double v = -n * Pl[n - 1][d];
            if (d > 0) v += (2 * n + 1) * Pl[n][d - 1];
            Pl[n + 1][d] = v / (n + 1);
        }
    ShTab t{};
    const double pi = 3.14159265358979323846;
    for (int l = 0; l <= 3; ++l)
        for (int m = -l; m <= l; ++m) {
            int a = m < 0 ? -m : m;
            double poly[4] = {Pl[l][0], Pl[l][1], Pl[l][2], Pl[l][3]};
            for (int r = 0; r < a; ++r)           // differentiate a times
                for (int d = 0; d < 4; ++d) poly[d] = (d + 1 < 4) ? (d + 1) * poly[d + 1] : 0.0;
            double N = csqrt((2 * l + 1) / (4 * pi) * cfact(l - a) / cfact(l + a));
            if (m != 0) N *= csqrt(2.0);
            ShCoef& c = t.k[l * l + l + m];
            c.a = a;
            c.sine = m < 0 ? 1 : 0;
            for (int d = 0; d < 4; ++d) c.q[d] = static_cast<float>(N * poly[d]);
            for (int d = 0; d < 4; ++d) c.dq[d] = static_cast<float>((d + 1 < 4) ? (d + 1) * N * poly[d + 1] : 0.0);
        }
    return t;
}

__device__ __forceinline__ const ShTab& sh_tab();

// Re and Im of (x + iy)^a, a = 0..3, selected with scalar selects (no
// dynamically indexed local arrays, which the compiler would move to LDS).
__device__ __forceinline__ void xy_power(float x, float y, int a, float& re, float& im) {
    const float c2 = x * x - y * y, s2 = 2.0f * x * y;
    const float c3 = c2 * x - s2 * y, s3 = c2 * y + s2 * x;
    re = a == 0 ? 1.0f : (a == 1 ? x : (a == 2 ? c2 : c3));
    im = a == 0 ? 0.0f : (a == 1 ? y : (a == 2 ? s2 : s3));
}

__device__ __forceinline__ float horner4(const float* q, float z) {
    return ((q[3] * z + q[2]) * z + q[1]) * z + q[0];
}

// Y_k of the direction of v with k's coefficients c; |v| = 0 gives
// Y_0 = 1/sqrt(4pi) and 0 otherwise.
__device__ __forceinline__ float sh_component_c(int k, const ShCoef& c, float vx, float vy, float vz) {
    const float n2 = vx * vx + vy * vy + vz * vz;
    if (n2 == 0.0f) return k == 0 ? 0.28209479177387814f : 0.0f;
    const float inv = 1.0f / sqrtf(n2);
    const float x = vx * inv, y = vy * inv, z = vz * inv;
    float re, im;
    xy_power(x, y, c.a, re, im);
    return (c.sine ? im : re) * horner4(c.q, z);
}

__device__ __forceinline__ float sh_component(int k, float vx, float vy, float vz) {
    return sh_component_c(k, sh_tab().k[k], vx, vy, vz);
}

// dY_k / dr (gradient of the polynomial form at the unit vector r).
__device__ __forceinline__ void sh_component_grad_c(const ShCoef& c, float x, float y, float z, float g[3]) {
    const float Q = horner4(c.q, z), dQ = horner4(c.dq, z);
    const int a = c.a;
    const float fa = static_cast<float>(a);
    float re, im, rm, imm;
    xy_power(x, y, a, re, im);
    xy_power(x, y, a > 0 ? a - 1 : 0, rm, imm);
    float A, dAx, dAy;
    if (c.sine) {          // Im (x+iy)^a:  d/dx = a Im w^(a-1),  d/dy = a Re w^(a-1)
        A = im;
        dAx = fa * imm;
        dAy = fa * rm;
    } else {               // Re (x+iy)^a:  d/dx = a Re w^(a-1),  d/dy = -a Im w^(a-1)
        A = re;
        dAx = fa * rm;
        dAy = -fa * imm;
    }
    g[0] = dAx * Q;
    g[1] = dAy * Q;
    g[2] = A * dQ;
}

__device__ __forceinline__ void sh_component_grad(int k, float x, float y, float z, float g[3]) {
    sh_component_grad_c(sh_tab().k[k], x, y, z, g);
}

// Gradient g and Hessian h = (xx, xy, yy, xz, yz, zz) in r of the polynomial
// form of Y_k (r a free vector).  With w = x + iy and A = Re w^a (Im w^a):
// A_x = a Re w^(a-1) (a Im), A_y = -a Im w^(a-1) (a Re), A_xx = a(a-1) Re w^(a-2)
// (a(a-1) Im), A_xy = -a(a-1) Im w^(a-2) (a(a-1) Re), A_yy = -A_xx.
__device__ __forceinline__ void sh_component_hess(int k, float x, float y, float z, float g[3], float h[6]) {
    const ShCoef& c = sh_tab().k[k];
    const float Q = horner4(c.q, z), dQ = horner4(c.dq, z);
    const float d2Q = c.dq[1] + 2.0f * c.dq[2] * z + 3.0f * c.dq[3] * z * z;
    const int a = c.a;
    const float fa = static_cast<float>(a), fb = static_cast<float>(a * (a - 1));
    float re, im, r1, i1, r2, i2;
    xy_power(x, y, a, re, im);
    xy_power(x, y, a > 0 ? a - 1 : 0, r1, i1);
    xy_power(x, y, a > 1 ? a - 2 : 0, r2, i2);
    float A, Ax, Ay, Axx, Axy;
    if (c.sine) {
        A = im;
        Ax = fa * i1;
        Ay = fa * r1;
        Axx = fb * i2;
        Axy = fb * r2;
    } else {
        A = re;
        Ax = fa * r1;
        Ay = -fa * i1;
        Axx = fb * r2;
        Axy = -fb * i2;
    }
    g[0] = Ax * Q;
    g[1] = Ay * Q;
    g[2] = A * dQ;
    h[0] = Axx * Q;
    h[1] = Axy * Q;
    h[2] = -Axx * Q;
    h[3] = Ax * dQ;
    h[4] = Ay * dQ;
    h[5] = A * d2Q;
}

// ------------------------------------------------------------ wavefront reductions (wave64, DPP)

template <int Ctrl, int RowMask = 0xf>
__device__ __forceinline__ float dpp_t(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, RowMask, 0xf, false));
}

// Sum over the 64 lanes, in a fixed order; the total is valid in lane 63.
__device__ __forceinline__ float wave_sum_to_last(float v) {
    v += dpp_t<0xB1>(v);          // quad_perm [1,0,3,2]
    v += dpp_t<0x4E>(v);          // quad_perm [2,3,0,1]
    v += dpp_t<0x124>(v);         // row_ror:4
    v += dpp_t<0x128>(v);         // row_ror:8  -> every lane holds its row sum
    v += dpp_t<0x142, 0xa>(v);    // row_bcast:15 into rows 1 and 3
    v += dpp_t<0x143, 0xc>(v);    // row_bcast:31 into rows 2 and 3
    return v;
}

__device__ __forceinline__ float lane_value(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sums of 16 per-lane values over the 64 lanes, in a fixed order, by
// recursive halving: at each exchange a lane sends the half of its values that
// its partner keeps and adds what the partner sends back, so 16 sums cost 35
// instructions instead of 16 full reductions.  Exchanges, in order: lane bit 5
// (v_permlane32_swap), bit 4 (v_permlane16_swap), bit 3 (row_ror:8), bit 0
// (quad_perm [1,0,3,2]); then bits 1 and 2 are summed in place (quad_perm
// [2,3,0,1], then row_ror:12, which hands lane l the value of lane l + 4 in
// its row).  The sum of value d ends in lane sum16_lane(d); lanes with bit 1
// or bit 2 set hold partial or duplicate values.
__host__ __device__ constexpr int sum16_lane(int d) { return (d & 1) | ((d >> 1) << 3); }
__device__ __forceinline__ int sum16_index(int lane) { return (lane & 1) | ((lane >> 3) << 1); }
__device__ __forceinline__ bool sum16_holder(int lane) { return (lane & 6) == 0; }

__device__ __forceinline__ float wave_sum16(const float (&v)[16], int lane) {
    float u[8], t[4], s[2];
#pragma unroll
    for (int k = 0; k < 8; ++k) {   // lanes 0-31 keep value k, lanes 32-63 value k + 8
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 8]), false,
                                                        false);
        u[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {   // even rows keep k, odd rows k + 4
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(u[k]), __float_as_uint(u[k + 4]), false,
                                                        false);
        t[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const bool b3 = (lane & 8) != 0, b0 = (lane & 1) != 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {   // lane bit 3 clear keeps k, set keeps k + 2
        const float keep = b3 ? t[k + 2] : t[k];
        const float send = b3 ? t[k] : t[k + 2];
        s[k] = keep + dpp_t<0x128>(send);
    }
    const float keep = b0 ? s[1] : s[0];
    const float send = b0 ? s[0] : s[1];
    float r = keep + dpp_t<0xB1>(send);
    r += dpp_t<0x4E>(r);
    r += dpp_t<0x12C>(r);
    return r;
}

// ------------------------------------------------------------ buffer rows
//
// Every feature/weight row is addressed through a buffer resource built from
// a wave-uniform base (SGPRs), one per-lane byte offset (a single VGPR) and a
// per-path/component offset in an SGPR.  Lanes with no channel get an offset
// beyond the row: their loads return 0 and their stores are dropped by the
// buffer range check.

using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kSrdWord3 = 0x00020000;      // gfx9 raw buffer, 32-bit dwords
constexpr uint32_t kOffLane = 0x80000000u;       // out-of-range lane offset

__device__ __forceinline__ rsrc_t make_row(const float* base, long n_floats) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)(n_floats * 4),
                                             (int)kSrdWord3);
}

// A uniform value the compiler must treat as redefined here: offsets built
// from it are formed next to their use instead of being hoisted out of the
// edge loop (dozens of hoisted per-path offsets exhaust the SGPRs).
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v) {
    asm volatile("" : "+s"(v));
    return v;
}

// Per-lane byte offset made opaque, so "+4 per channel" folds into the
// instruction's immediate offset and adjacent channels merge into one
// dwordx2 access (a select hidden behind the offset would block that).
__device__ __forceinline__ uint32_t opaque_lane(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Pins a register value at this point of the program: the update that
// produced it cannot be sunk past later stores (keeps per-path temporaries
// short-lived instead of deferring every accumulation to the loop latch).
__device__ __forceinline__ void pin_f32(float& v) { asm volatile("" : "+v"(v)); }

// A lane owns CPL consecutive channels c0 .. c0 + CPL - 1 (c0 = CPL * lane
// within the wave's block): one access instruction covers the wave's 64 * CPL
// consecutive floats (256 or 512 contiguous bytes), one dword or dwordx2 per
// lane.
// Cache policy of a buffer access: kStream (non-temporal) marks the edge
// streams touched exactly once (w, dw, out, dx).
constexpr int kCached = 0;
constexpr int kStream = 2;

template <int CPL, int Aux = kCached>
__device__ __forceinline__ void bload(rsrc_t r, uint32_t voff, uint32_t soff, float (&v)[CPL]) {
    static_assert(CPL == 1 || CPL == 2, "one or two channels per lane");
    // Two adjacent dword loads, which the backend merges into one dwordx2.  (This
    // compiler narrows __builtin_amdgcn_raw_buffer_load_b64 to a single dword
    // when its two halves are used apart, so that builtin is not used.)
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        v[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff + 4u * c, soff, Aux));
}

template <int CPL, int Aux = kCached>
__device__ __forceinline__ void bstore(rsrc_t r, uint32_t voff, uint32_t soff, const float (&v)[CPL]) {
    static_assert(CPL == 1 || CPL == 2, "one or two channels per lane");
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v[c]), r, voff + 4u * c, soff, Aux);
}

// ------------------------------------------------------------ per-edge coupling T in LDS

// Entry t of a per-edge T in LDS, read as part of its aligned group of four
// (T is 16-byte aligned and padded to a multiple of 4 entries): every read is
// then a 16-byte load at an immediate offset from one address register, and
// neighbouring entries share it.
template <int t>
__device__ __forceinline__ float slot_value(const float* T) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4 q = reinterpret_cast<const f4*>(T)[t >> 2];
    return q[t & 3];
}

// Component tid of Y for edge e (lanes >= D2 return 0).
template <int D2, bool VEC>
__device__ __forceinline__ float sh_value(const float* __restrict__ yv, long e, int tid) {
    float r = 0.0f;
    if (tid < D2) {
        if constexpr (VEC) {
            const float* v = yv + 3 * e;
            r = sh_component(tid, v[0], v[1], v[2]);
        } else {
            r = yv[e * D2 + tid];
        }
    }
    return r;
}

// The same through a buffer row in Y mode: lanes >= D2 read past the row and get 0.
template <int D2, bool VEC>
__device__ __forceinline__ float sh_load(const float* __restrict__ yv, long e, int tid) {
    if constexpr (VEC) {
        return sh_value<D2, true>(yv, e, tid);
    } else {
        const rsrc_t yr = make_row(yv + e * D2, D2);
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(yr, (uint32_t)tid * 4u, 0, 0));
    }
}

template <class S>
__device__ __forceinline__ void build_T_lds(float* sT, const float* sY, const SlotDev* tab, int tid, int nth) {
    for (int t = tid; t < S::NT; t += nth) {
        const SlotDev s = tab[t];
        sT[t] = s.c1 * sY[s.yy & 0xff] + s.c2 * sY[s.yy >> 8];
    }
}

}  // namespace ctp
