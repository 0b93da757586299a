// Compile-time path lists and real coupling tables for the conv tensor product.
//
// Everything here is constexpr: the kernels unroll over these tables with
// compile-time indices, so register arrays stay in registers and every
// coupling coefficient becomes an instruction constant.
//
// Coupling (FlashCart, arXiv 2610.06409, section on spherical and Cartesian
// products: one equivariant bilinear map per triangle-allowed path, unique up
// to normalisation):
//   * complex CG from the Wigner 3j symbol (Racah's explicit sum for the 3j
//     symbol, then <j1 m1 j2 m2|J M> = (-1)^(j1-j2+M) sqrt(2J+1) (j1 j2 J; m1 m2 -M));
//   * real basis: for m > 0 the real component is ((-1)^m c_m + c_-m)/sqrt2,
//     for m < 0 it is i(c_-|m| - (-1)^|m| c_|m|)/sqrt2, m = 0 unchanged;
//   * real tensor z[m1,m2,m3] = sum U1 U2 conj(U3) CG, keeping Re z for even
//     l1+l2+l3 and Im z for odd (the other part is zero).  Orthonormal:
//     sum_{m1,m2} C[m1,m2,m3] C[m1,m2,m3'] = delta.
// Paths: all (l1,l2,l3) with l1<=L1, l2<=L2, l3<=L3, |l1-l2|<=l3<=l1+l2,
// lexicographic, all paths with the same l3 summed into one output block.
// Component index d(l,m) = l*l + l + m.
#pragma once

#include <array>
#include <cstdint>

namespace ctp {

constexpr int kMaxL = 3;

constexpr int dim_of(int L) { return (L + 1) * (L + 1); }

constexpr bool triangle(int a, int b, int c) {
    return (a - b <= c && b - a <= c) && c <= a + b;
}

// Path variants.  0: every triangle-allowed path, paths sharing l3 summed
// into one output block.  1 (MACE's convolution): only natural-parity paths
// (l1 + l2 + l3 even), each with an output slot of its own.
constexpr int kVariantSummed = 0;
constexpr int kVariantSlots = 1;

constexpr bool path_ok(int a, int b, int c, int V) {
    return triangle(a, b, c) && (V == kVariantSummed || (a + b + c) % 2 == 0);
}

constexpr int num_paths(int L1, int L2, int L3, int V = kVariantSummed) {
    int n = 0;
    for (int a = 0; a <= L1; ++a)
        for (int b = 0; b <= L2; ++b)
            for (int c = 0; c <= L3; ++c)
                if (path_ok(a, b, c, V)) ++n;
    return n;
}

// Output components per channel: (L3+1)^2 summed, sum of 2 l3 + 1 over the
// paths with slots.
constexpr int out_dim(int L1, int L2, int L3, int V) {
    if (V == kVariantSummed) return dim_of(L3);
    int n = 0;
    for (int a = 0; a <= L1; ++a)
        for (int b = 0; b <= L2; ++b)
            for (int c = 0; c <= L3; ++c)
                if (path_ok(a, b, c, V)) n += 2 * c + 1;
    return n;
}

// ------------------------------------------------------------ scalar helpers

constexpr double cfact(int n) {
    double r = 1.0;
    for (int i = 2; i <= n; ++i) r *= i;
    return r;
}

constexpr double csqrt(double v) {
    if (v <= 0.0) return 0.0;
    double x = v > 1.0 ? v : 1.0;
    for (int it = 0; it < 200; ++it) {
        double nx = 0.5 * (x + v / x);
        if (nx == x) break;
        x = nx;
    }
    return x;
}

constexpr double cabs(double v) { return v < 0 ? -v : v; }

constexpr double sgn_pow(int k) { return (k % 2 == 0) ? 1.0 : -1.0; }  // (-1)^k, k may be < 0

struct Cplx {
    double re, im;
};
constexpr Cplx cmul(Cplx a, Cplx b) { return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }
constexpr Cplx cconj(Cplx a) { return {a.re, -a.im}; }

// Wigner 3j symbol (j1 j2 j3; m1 m2 m3), Racah's explicit sum.
constexpr double wigner3j(int j1, int j2, int j3, int m1, int m2, int m3) {
    if (m1 + m2 + m3 != 0) return 0.0;
    if (!triangle(j1, j2, j3)) return 0.0;
    if (cabs(m1) > j1 || cabs(m2) > j2 || cabs(m3) > j3) return 0.0;
    double delta = cfact(j1 + j2 - j3) * cfact(j1 - j2 + j3) * cfact(-j1 + j2 + j3) / cfact(j1 + j2 + j3 + 1);
    double pre = csqrt(delta * cfact(j1 + m1) * cfact(j1 - m1) * cfact(j2 + m2) * cfact(j2 - m2) *
                       cfact(j3 + m3) * cfact(j3 - m3));
    double s = 0.0;
    for (int k = 0; k <= j1 + j2 + j3; ++k) {
        int a = j3 - j2 + k + m1, b = j3 - j1 + k - m2, c = j1 + j2 - j3 - k, d = j1 - k - m1, e = j2 - k + m2;
        if (a < 0 || b < 0 || c < 0 || d < 0 || e < 0) continue;
        s += sgn_pow(k) / (cfact(k) * cfact(a) * cfact(b) * cfact(c) * cfact(d) * cfact(e));
    }
    return sgn_pow(j1 - j2 - m3) * pre * s;
}

constexpr double clebsch(int j1, int m1, int j2, int m2, int J, int M) {
    return sgn_pow(j1 - j2 + M) * csqrt(2.0 * J + 1.0) * wigner3j(j1, j2, J, m1, m2, -M);
}

// Entry U^l[m][mu] of the real-basis map (complex component mu -> real m).
constexpr Cplx ubasis(int m, int mu) {
    const double h = 0.70710678118654752440;
    if (m == 0) return (mu == 0) ? Cplx{1.0, 0.0} : Cplx{0.0, 0.0};
    if (m > 0) {
        if (mu == m) return {sgn_pow(m) * h, 0.0};
        if (mu == -m) return {h, 0.0};
        return {0.0, 0.0};
    }
    int a = -m;
    if (mu == a) return {0.0, -sgn_pow(a) * h};
    if (mu == -a) return {0.0, h};
    return {0.0, 0.0};
}

// Real coupling coefficient C_(l1,l2,l3)[m1][m2][m3], m's signed.
constexpr double real_coupling(int l1, int l2, int l3, int m1, int m2, int m3) {
    Cplx z{0.0, 0.0};
    for (int s1 = -1; s1 <= 1; s1 += 2)
        for (int s2 = -1; s2 <= 1; s2 += 2) {
            if (m1 == 0 && s1 > 0) continue;   // mu = 0 counted once
            if (m2 == 0 && s2 > 0) continue;
            int mu1 = s1 * m1, mu2 = s2 * m2, mu3 = mu1 + mu2;
            if (cabs(mu3) > l3) continue;
            Cplx u3 = ubasis(m3, mu3);
            if (u3.re == 0.0 && u3.im == 0.0) continue;
            double c = clebsch(l1, mu1, l2, mu2, l3, mu3);
            Cplx t = cmul(cmul(ubasis(m1, mu1), ubasis(m2, mu2)), cconj(u3));
            z.re += t.re * c;
            z.im += t.im * c;
        }
    double v = ((l1 + l2 + l3) % 2 == 0) ? z.re : z.im;
    return cabs(v) < 1e-12 ? 0.0 : v;
}

// ------------------------------------------------------------ per-problem tables

struct PathL {
    int l1, l2, l3;
};

// One structural non-zero of the per-edge coupling matrix
// T_p[m1][m3] = sum_m2 C_p[m1][m2][m3] Y[l2 m2]; at most two m2 terms.
struct TSlot {
    int p, m1, m3;      // path, 0-based m1 in 0..2l1, m3 in 0..2l3
    int y1, y2;         // flat Y component indices (y2 = y1 if unused)
    float c1, c2;       // coefficients (c2 = 0 if unused)
};

// One non-zero of a coupling tensor.
struct CgNz {
    int p, m1, m2, m3;  // 0-based within the path's blocks
    float c;
};

// A set of paths that read the same block of G in the backward: for summed
// outputs all paths with the same (l1, l3) (block l3), for slots one path.
struct PathGroup {
    int l1, l3, o3, n;
    int p[kMaxL + 1];
};

template <int L1_, int L2_, int L3_, int V_ = kVariantSummed>
struct Spec {
    static constexpr int L1 = L1_, L2 = L2_, L3 = L3_, V = V_;
    static constexpr int D1 = dim_of(L1), D2 = dim_of(L2), D3 = dim_of(L3);
    static constexpr int P = num_paths(L1, L2, L3, V);
    static constexpr int DO = out_dim(L1, L2, L3, V);   // output (and G) components

    static constexpr std::array<PathL, P> make_paths() {
        std::array<PathL, P> r{};
        int n = 0;
        for (int a = 0; a <= L1; ++a)
            for (int b = 0; b <= L2; ++b)
                for (int c = 0; c <= L3; ++c)
                    if (path_ok(a, b, c, V)) r[n++] = PathL{a, b, c};
        return r;
    }
    static constexpr std::array<PathL, P> paths = make_paths();

    // First output component of each path's contribution.
    static constexpr std::array<int, P> make_out_off() {
        std::array<int, P> r{};
        int o = 0;
        for (int p = 0; p < P; ++p) {
            r[p] = V == kVariantSummed ? paths[p].l3 * paths[p].l3 : o;
            o += 2 * paths[p].l3 + 1;
        }
        return r;
    }
    static constexpr std::array<int, P> out_off = make_out_off();

    static constexpr int count_groups() {
        if (V != kVariantSummed) return P;
        int n = 0;
        for (int a = 0; a <= L1; ++a)
            for (int c = 0; c <= L3; ++c) {
                bool any = false;
                for (int p = 0; p < P; ++p)
                    if (paths[p].l1 == a && paths[p].l3 == c) any = true;
                if (any) ++n;
            }
        return n;
    }
    static constexpr int NG = count_groups();

    // Groups in the order the backward walks them: (l1, l3) with l1 outer for
    // summed outputs, path order for slots.
    static constexpr std::array<PathGroup, NG> make_groups() {
        std::array<PathGroup, NG> r{};
        int n = 0;
        if (V != kVariantSummed) {
            for (int p = 0; p < P; ++p) r[n++] = PathGroup{paths[p].l1, paths[p].l3, out_off[p], 1, {p, 0, 0, 0}};
            return r;
        }
        for (int a = 0; a <= L1; ++a)
            for (int c = 0; c <= L3; ++c) {
                PathGroup g{a, c, c * c, 0, {0, 0, 0, 0}};
                for (int p = 0; p < P; ++p)
                    if (paths[p].l1 == a && paths[p].l3 == c) g.p[g.n++] = p;
                if (g.n > 0) r[n++] = g;
            }
        return r;
    }
    static constexpr std::array<PathGroup, NG> groups = make_groups();

    static constexpr int count_nz() {
        int n = 0;
        for (int p = 0; p < P; ++p) {
            auto q = paths[p];
            for (int a = 0; a < 2 * q.l1 + 1; ++a)
                for (int b = 0; b < 2 * q.l2 + 1; ++b)
                    for (int c = 0; c < 2 * q.l3 + 1; ++c)
                        if (real_coupling(q.l1, q.l2, q.l3, a - q.l1, b - q.l2, c - q.l3) != 0.0) ++n;
        }
        return n;
    }
    static constexpr int NNZ = count_nz();

    static constexpr std::array<CgNz, NNZ> make_nz() {
        std::array<CgNz, NNZ> r{};
        int n = 0;
        for (int p = 0; p < P; ++p) {
            auto q = paths[p];
            for (int a = 0; a < 2 * q.l1 + 1; ++a)
                for (int b = 0; b < 2 * q.l2 + 1; ++b)
                    for (int c = 0; c < 2 * q.l3 + 1; ++c) {
                        double v = real_coupling(q.l1, q.l2, q.l3, a - q.l1, b - q.l2, c - q.l3);
                        if (v != 0.0) r[n++] = CgNz{p, a, b, c, static_cast<float>(v)};
                    }
        }
        return r;
    }
    static constexpr std::array<CgNz, NNZ> nz = make_nz();

    static constexpr int count_slots() {
        int n = 0;
        for (int p = 0; p < P; ++p) {
            auto q = paths[p];
            for (int a = 0; a < 2 * q.l1 + 1; ++a)
                for (int c = 0; c < 2 * q.l3 + 1; ++c) {
                    bool any = false;
                    for (int b = 0; b < 2 * q.l2 + 1; ++b)
                        if (real_coupling(q.l1, q.l2, q.l3, a - q.l1, b - q.l2, c - q.l3) != 0.0) any = true;
                    if (any) ++n;
                }
        }
        return n;
    }
    static constexpr int NT = count_slots();

    // Slots ordered by path, then m1, then m3.
    static constexpr std::array<TSlot, NT> make_slots() {
        std::array<TSlot, NT> r{};
        int n = 0;
        for (int p = 0; p < P; ++p) {
            auto q = paths[p];
            for (int a = 0; a < 2 * q.l1 + 1; ++a)
                for (int c = 0; c < 2 * q.l3 + 1; ++c) {
                    int k = 0;
                    TSlot s{p, a, c, 0, 0, 0.0f, 0.0f};
                    for (int b = 0; b < 2 * q.l2 + 1; ++b) {
                        double v = real_coupling(q.l1, q.l2, q.l3, a - q.l1, b - q.l2, c - q.l3);
                        if (v == 0.0) continue;
                        int y = q.l2 * q.l2 + b;
                        if (k == 0) { s.y1 = y; s.y2 = y; s.c1 = static_cast<float>(v); }
                        else { s.y2 = y; s.c2 = static_cast<float>(v); }
                        ++k;
                    }
                    if (k > 0) r[n++] = s;
                }
        }
        return r;
    }
    static constexpr std::array<TSlot, NT> slots = make_slots();

    // First slot of each path (and NT at the end).
    static constexpr std::array<int, P + 1> make_slot_begin() {
        std::array<int, P + 1> r{};
        int p = 0;
        for (int t = 0; t < NT; ++t)
            while (p <= slots[t].p) r[p++] = t;
        while (p <= P) r[p++] = NT;
        return r;
    }
    static constexpr std::array<int, P + 1> slot_begin = make_slot_begin();

    static constexpr int max_terms() {
        int m = 0;
        for (int t = 0; t < NT; ++t) {
            int k = (slots[t].c2 != 0.0f) ? 2 : 1;
            if (k > m) m = k;
        }
        return m;
    }
};

// Host-side lookups for the C ABI (runtime degrees).
int host_num_paths(int l1, int l2, int l3, int variant = kVariantSummed);
int host_out_dim(int l1, int l2, int l3, int variant);
int host_paths(int l_in, int l_sh, int l_out, int32_t* l123, int variant = kVariantSummed);
int host_coupling(int l1, int l2, int l3, double* out);

}  // namespace ctp
