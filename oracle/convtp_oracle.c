/*
 * Naive fp64 edge loop of the equivariant convolution tensor product.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU baseline; never by the product path.  It shares no code
 * with the HIP library.
 *
 * Definition (e3j, arXiv 2609.35099, abstract and Table 1 caption: the
 * message-passing convolution that e3nn computes by materialising messages):
 *
 *   msg_e[l3 m3, c] = sum_{p=(l1,l2,l3)} w[e,p,c]
 *                     sum_{m1,m2} C_p[m1,m2,m3] x[s_e, l1 m1, c] Y[e, l2 m2]
 *   out[i] = sum_{e into i} msg_e
 *
 * and its vector-Jacobian products (FlashCart, arXiv 2610.06409, symbolic
 * VJP section) for an upstream gradient G = dL/dout:
 *
 *   dx[j, l1 m1, c] = sum_{e out of j} sum_p w[e,p,c] sum_{m2,m3} C_p Y[e,l2 m2] G[r_e, l3 m3, c]
 *   dw[e, p, c]     = sum_{m1,m2,m3} C_p x[s_e, l1 m1, c] Y[e, l2 m2] G[r_e, l3 m3, c]
 *   dY[e, l2 m2]    = sum_c sum_p w[e,p,c] sum_{m1,m3} C_p x[s_e, l1 m1, c] G[r_e, l3 m3, c]
 *
 * Inputs x, w, G are fp32 (as the GPU sees them) and are read as fp32 and
 * widened; all arithmetic and accumulation is fp64.  Y is passed in fp64 so a
 * caller can give either the fp32 values the GPU reads or exact harmonics.
 * The coupling tensors come in from the caller as dense fp64 blocks, path p
 * at cg + cg_off[p], laid out [2l1+1][2l2+1][2l3+1].
 *
 * Component index d(l, m) = l*l + l + m; arrays are x[N][D1][C],
 * Y[E][D2], w[E][P][C], out/G[N][D3][C].  Path p's output block starts at
 * component o3[p]: l3*l3 when paths sharing l3 are summed, or the path's own
 * slot when each path keeps its output (MACE's convolution).  Every function evaluates only the
 * rows (receivers, senders or edges) it is asked for, so large workloads can
 * be checked on samples.
 */
#include <stdlib.h>
#include <string.h>
#include <stdint.h>
#include <omp.h>

#define IDX3(a, b, c, nb, nc) (((size_t)(a) * (nb) + (b)) * (nc) + (c))

/* out[r][D3][C] for receiver rows[r] */
int oracle_fwd(int C, int D1, int D2, int D3, int P, const int *l123, const int *o3,
               const double *cg, const int64_t *cg_off,
               const float *x, const double *Y, const float *w,
               const int *row_ptr, const int *senders,
               int n_rows, const int *rows, double *out, int n_threads)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(+ : bad)
    for (int r = 0; r < n_rows; ++r) {
        double *msg = (double *)malloc(sizeof(double) * (size_t)D3 * C);
        double *o = out + (size_t)r * D3 * C;
        memset(o, 0, sizeof(double) * (size_t)D3 * C);
        if (!msg) { bad += 1; continue; }
        int i = rows[r];
        for (int e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            int j = senders[e];
            memset(msg, 0, sizeof(double) * (size_t)D3 * C);
            for (int p = 0; p < P; ++p) {
                int l1 = l123[3 * p], l2 = l123[3 * p + 1], l3 = l123[3 * p + 2];
                int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
                const double *cp = cg + cg_off[p];
                const float *wp = w + IDX3(e, p, 0, P, C);
                for (int a = 0; a < n1; ++a)
                    for (int b = 0; b < n2; ++b)
                        for (int k = 0; k < n3; ++k) {
                            double coef = cp[(a * n2 + b) * n3 + k];
                            if (coef == 0.0) continue;
                            double t = coef * Y[(size_t)e * D2 + l2 * l2 + b];
                            const float *xs = x + IDX3(j, l1 * l1 + a, 0, D1, C);
                            double *m = msg + (size_t)(o3[p] + k) * C;
                            for (int c = 0; c < C; ++c)
                                m[c] += (double)wp[c] * t * (double)xs[c];
                        }
            }
            for (size_t q = 0; q < (size_t)D3 * C; ++q) o[q] += msg[q];
        }
        free(msg);
    }
    return bad;
}

/* dx[r][D1][C] for sender rows[r], walking its out-edges via the transpose */
int oracle_bwd_dx(int C, int D1, int D2, int D3, int P, const int *l123, const int *o3,
                  const double *cg, const int64_t *cg_off,
                  const double *Y, const float *w, const float *G,
                  const int *send_ptr, const int *send_perm, const int *send_recv,
                  int n_rows, const int *rows, double *dx, int n_threads)
{
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int r = 0; r < n_rows; ++r) {
        double *o = dx + (size_t)r * D1 * C;
        memset(o, 0, sizeof(double) * (size_t)D1 * C);
        int j = rows[r];
        for (int k = send_ptr[j]; k < send_ptr[j + 1]; ++k) {
            int e = send_perm[k], i = send_recv[k];
            for (int p = 0; p < P; ++p) {
                int l1 = l123[3 * p], l2 = l123[3 * p + 1], l3 = l123[3 * p + 2];
                int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
                const double *cp = cg + cg_off[p];
                const float *wp = w + IDX3(e, p, 0, P, C);
                for (int a = 0; a < n1; ++a)
                    for (int b = 0; b < n2; ++b)
                        for (int q = 0; q < n3; ++q) {
                            double coef = cp[(a * n2 + b) * n3 + q];
                            if (coef == 0.0) continue;
                            double t = coef * Y[(size_t)e * D2 + l2 * l2 + b];
                            const float *g = G + IDX3(i, o3[p] + q, 0, D3, C);
                            double *d = o + (size_t)(l1 * l1 + a) * C;
                            for (int c = 0; c < C; ++c)
                                d[c] += (double)wp[c] * t * (double)g[c];
                        }
            }
        }
    }
    return 0;
}

/* dw[r][P][C] and dY[r][D2] for edge rows[r]; recv[e] is the edge's receiver */
int oracle_bwd_edge(int C, int D1, int D2, int D3, int P, const int *l123, const int *o3,
                    const double *cg, const int64_t *cg_off,
                    const float *x, const double *Y, const float *w, const float *G,
                    const int *senders, const int *recv,
                    int n_rows, const int *rows, double *dw, double *dY, int n_threads)
{
#pragma omp parallel for schedule(dynamic, 16) num_threads(n_threads)
    for (int r = 0; r < n_rows; ++r) {
        int e = rows[r];
        int j = senders[e], i = recv[e];
        double *ow = dw + (size_t)r * P * C;
        double *oy = dY + (size_t)r * D2;
        memset(ow, 0, sizeof(double) * (size_t)P * C);
        memset(oy, 0, sizeof(double) * (size_t)D2);
        for (int p = 0; p < P; ++p) {
            int l1 = l123[3 * p], l2 = l123[3 * p + 1], l3 = l123[3 * p + 2];
            int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
            const double *cp = cg + cg_off[p];
            const float *wp = w + IDX3(e, p, 0, P, C);
            for (int a = 0; a < n1; ++a)
                for (int b = 0; b < n2; ++b)
                    for (int q = 0; q < n3; ++q) {
                        double coef = cp[(a * n2 + b) * n3 + q];
                        if (coef == 0.0) continue;
                        double yv = Y[(size_t)e * D2 + l2 * l2 + b];
                        const float *xs = x + IDX3(j, l1 * l1 + a, 0, D1, C);
                        const float *g = G + IDX3(i, o3[p] + q, 0, D3, C);
                        double sy = 0.0;
                        for (int c = 0; c < C; ++c) {
                            double xg = (double)xs[c] * (double)g[c];
                            ow[(size_t)p * C + c] += coef * yv * xg;
                            sy += (double)wp[c] * xg;
                        }
                        oy[l2 * l2 + b] += coef * sy;
                    }
        }
    }
    return 0;
}

int oracle_max_threads(void) { return omp_get_max_threads(); }
