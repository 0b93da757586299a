/* A plain C99 consumer of the conv TP C ABI (include/convtp.h).
 *
 * TEST INFRASTRUCTURE: reads a problem and its inputs from a binary file,
 * allocates device memory with the HIP runtime, runs conv_tp_build_transpose,
 * conv_tp_fwd and conv_tp_bwd (or conv_tp_bwd_msg) with the given algo on
 * the null stream, and
 * writes the outputs to a binary file.  tests/test_gpu_c_abi.py compares them
 * with the oracle.
 *
 *   roundtrip IN OUT
 *
 * IN : int32 head[8] = {N, E, C, L, y_mode, variant, use_msg, algo}, then
 *      x[N][D][C] f32, y[E][S] f32 (S = D or 3), w[E][P][C] f32,
 *      G[N][D_out][C] f32, row_ptr[N+1] i32, senders[E] i32
 * OUT: out[N][D_out][C], dx[N][D][C], dw[E][P][C], dy[E][S] (f32), then
 *      send_ptr[N+1], send_perm[E], send_recv[E] (i32)
 * P and D_out come from conv_tp_layout.  Exit status 0 on success; on a
 * library error the message of conv_tp_last_error goes to stderr.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "convtp.h"

static void die(const char *what) {
    fprintf(stderr, "roundtrip: %s\n", what);
    exit(1);
}

static void ck(int32_t status, const char *what) {
    if (status != CTP_OK) {
        fprintf(stderr, "roundtrip: %s -> status %d: %s\n", what, (int)status, conv_tp_last_error());
        exit(1);
    }
}

static void hck(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        fprintf(stderr, "roundtrip: %s: %s\n", what, hipGetErrorString(e));
        exit(1);
    }
}

/* host buffer of n elements of size sz read from f */
static void *read_array(FILE *f, size_t n, size_t sz) {
    void *p = malloc(n * sz > 0 ? n * sz : 1);
    if (p == NULL) die("out of host memory");
    if (n > 0 && fread(p, sz, n, f) != n) die("short input file");
    return p;
}

/* device copy of a host array (NULL for an empty one) */
static void *to_device(const void *h, size_t bytes) {
    void *d = NULL;
    if (bytes == 0) return NULL;
    hck(hipMalloc(&d, bytes), "hipMalloc");
    hck(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice), "hipMemcpy to device");
    return d;
}

static void *device_zeros(size_t bytes) {
    void *d = NULL;
    if (bytes == 0) return NULL;
    hck(hipMalloc(&d, bytes), "hipMalloc");
    hck(hipMemset(d, 0, bytes), "hipMemset");
    return d;
}

static void write_back(FILE *f, const void *d, size_t bytes) {
    void *h;
    if (bytes == 0) return;
    h = malloc(bytes);
    if (h == NULL) die("out of host memory");
    hck(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost), "hipMemcpy to host");
    if (fwrite(h, 1, bytes, f) != bytes) die("short write");
    free(h);
}

int main(int argc, char **argv) {
    FILE *fi, *fo;
    int32_t head[8], P = 0, DO = 0;
    size_t N, E, C, D, S;
    conv_tp_problem prob;
    float *x, *y, *w, *G;
    int32_t *row_ptr, *senders;
    void *dx_in, *dy_in, *dw_in, *dG, *drp, *ds, *dsp, *dpe, *dsr, *dout, *ddx, *ddw, *ddy, *dws = NULL;
    int64_t ws_bytes = 0;

    if (argc != 3) die("usage: roundtrip IN OUT");
    fi = fopen(argv[1], "rb");
    if (fi == NULL) die("cannot open input");
    if (fread(head, sizeof(int32_t), 8, fi) != 8) die("short header");
    N = (size_t)head[0];
    E = (size_t)head[1];
    C = (size_t)head[2];
    D = (size_t)(head[3] + 1) * (size_t)(head[3] + 1);
    S = head[4] ? 3 : D;
    ck(conv_tp_layout(head[5], head[3], head[3], head[3], &P, &DO, NULL), "conv_tp_layout");

    x = read_array(fi, N * D * C, sizeof(float));
    y = read_array(fi, E * S, sizeof(float));
    w = read_array(fi, E * (size_t)P * C, sizeof(float));
    G = read_array(fi, N * (size_t)DO * C, sizeof(float));
    row_ptr = read_array(fi, N + 1, sizeof(int32_t));
    senders = read_array(fi, E, sizeof(int32_t));
    fclose(fi);

    prob.n_nodes = head[0];
    prob.n_edges = head[1];
    prob.channels = head[2];
    prob.l_in = prob.l_sh = prob.l_out = head[3];
    prob.y_mode = head[4];
    prob.algo = head[7];
    prob.variant = head[5];

    dx_in = to_device(x, N * D * C * sizeof(float));
    dy_in = to_device(y, E * S * sizeof(float));
    dw_in = to_device(w, E * (size_t)P * C * sizeof(float));
    dG = to_device(G, N * (size_t)DO * C * sizeof(float));
    drp = to_device(row_ptr, (N + 1) * sizeof(int32_t));
    ds = to_device(senders, E * sizeof(int32_t));
    dsp = device_zeros((N + 1) * sizeof(int32_t));
    dpe = device_zeros(E * sizeof(int32_t));
    dsr = device_zeros(E * sizeof(int32_t));
    dout = device_zeros(N * (size_t)DO * C * sizeof(float));
    ddx = device_zeros(N * D * C * sizeof(float));
    ddw = device_zeros(E * (size_t)P * C * sizeof(float));
    ddy = device_zeros(E * S * sizeof(float));

    ck(conv_tp_build_transpose(head[0], head[1], drp, ds, dsp, dpe, dsr, NULL), "conv_tp_build_transpose");
    ck(conv_tp_fwd(&prob, dx_in, dy_in, dw_in, drp, ds, dout, NULL), "conv_tp_fwd");
    if (head[6]) {
        ck(conv_tp_bwd_msg_workspace(&prob, &ws_bytes), "conv_tp_bwd_msg_workspace");
        dws = device_zeros((size_t)ws_bytes);
        ck(conv_tp_bwd_msg(&prob, dG, dx_in, dy_in, dw_in, drp, ds, dsp, dpe, dsr, ddx, ddw, ddy, dws, ws_bytes,
                           NULL),
           "conv_tp_bwd_msg");
    } else {
        ck(conv_tp_bwd(&prob, dG, dx_in, dy_in, dw_in, drp, ds, dsp, dpe, dsr, ddx, ddw, ddy, NULL), "conv_tp_bwd");
    }
    hck(hipDeviceSynchronize(), "hipDeviceSynchronize");

    fo = fopen(argv[2], "wb");
    if (fo == NULL) die("cannot open output");
    write_back(fo, dout, N * (size_t)DO * C * sizeof(float));
    write_back(fo, ddx, N * D * C * sizeof(float));
    write_back(fo, ddw, E * (size_t)P * C * sizeof(float));
    write_back(fo, ddy, E * S * sizeof(float));
    write_back(fo, dsp, (N + 1) * sizeof(int32_t));
    write_back(fo, dpe, E * sizeof(int32_t));
    write_back(fo, dsr, E * sizeof(int32_t));
    fclose(fo);

    hipFree(dx_in); hipFree(dy_in); hipFree(dw_in); hipFree(dG); hipFree(drp); hipFree(ds);
    hipFree(dsp); hipFree(dpe); hipFree(dsr); hipFree(dout); hipFree(ddx); hipFree(ddw); hipFree(ddy);
    hipFree(dws);
    free(x); free(y); free(w); free(G); free(row_ptr); free(senders);
    return 0;
}
