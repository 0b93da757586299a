// Internal launch interface between the C ABI front and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ctp {

struct LaunchArgs {
    int L;                 // l_in = l_sh = l_out
    int n_nodes, n_edges, C;
    int algo;              // 0: CSR deterministic, 1: edge-parallel atomic, 2: edge frame (forward only)
    int vec_mode;          // 0: Y[E][D] given, 1: vec[E][3] given
    int variant;           // 0: all paths, same-l3 sums; 1: natural-parity paths, one output slot each
    const float* x;        // [N][D][C]
    const float* y;        // Y[E][D] or vec[E][3]
    const float* w;        // [E][P][C]
    const float* grad;     // [N][D][C] (backward)
    const int32_t* row_ptr;
    const int32_t* senders;
    const int32_t* send_ptr;
    const int32_t* send_perm;
    const int32_t* send_recv;
    float* out;            // forward output
    float* dx;             // [N][D][C]
    float* dw;             // [E][P][C]
    float* dy;             // dY[E][D] or dvec[E][3]
};

// VJP of the VJP (Y given): cotangents ax, aw, ay of (dx, dw, dY).
struct DoubleArgs {
    int L;
    int n_nodes, n_edges, C;
    const float *x, *ax;    // [N][D][C]
    const float *y, *ay;    // [E][D]
    const float *w, *aw;    // [E][P][C]
    const float* grad;      // G [N][D][C]
    const int32_t *row_ptr, *senders, *send_ptr, *send_perm, *send_recv;
    float* g_x;             // [N][D][C]
    float* g_w;             // [E][P][C]
    float* g_y;             // [E][D]
    float* g_grad;          // [N][D][C]
};

hipError_t launch_fwd(const LaunchArgs& a, hipStream_t st);
hipError_t launch_double_bwd(const DoubleArgs& a, hipStream_t st);
bool dd_supports_channels(int C);
// Forward in each edge's own frame (edge vectors, summed variant).
hipError_t launch_fwd_frame(const LaunchArgs& a, hipStream_t st);
// Harmonic gradient dY alone (Y given): receiver-major, G row once per receiver.
hipError_t launch_bwd_dy(const LaunchArgs& a, hipStream_t st);
bool dy_supports_channels(int C);
hipError_t launch_bwd(const LaunchArgs& a, hipStream_t st);
// Backward through an edge-message workspace msg[E][D][C]: receiver-major
// products, then per-sender sums of the messages.
hipError_t launch_bwd_msg(const LaunchArgs& a, float* msg, hipStream_t st);
bool bwd_supports_channels(int C);
hipError_t launch_sh(int L, long n_edges, const float* vec, float* Y, hipStream_t st);
hipError_t launch_sh_bwd(int L, long n_edges, const float* vec, const float* dY, float* dvec, hipStream_t st);
hipError_t launch_sh_jvp(int L, long n_edges, const float* vec, const float* a, float* aY, hipStream_t st);
hipError_t launch_sh_bwd_bwd(int L, long n_edges, const float* vec, const float* dY, const float* a, const float* gY,
                             float* gvec, hipStream_t st);

hipError_t launch_transpose(int n_nodes, int n_edges, const int32_t* row_ptr, const int32_t* senders,
                            int32_t* send_ptr, int32_t* send_perm, int32_t* send_recv, hipStream_t st);
hipError_t launch_node_fwd(int L, int n_nodes, int C, const float* x, const float* y, const float* w, float* out,
                           hipStream_t st);
hipError_t launch_node_bwd(int L, int n_nodes, int C, const float* G, const float* x, const float* y,
                           const float* w, float* dx, float* dy, float* dw, hipStream_t st);
hipError_t launch_stream_probe(int kind, const float* src, float* dst, long n_floats, hipStream_t st);
hipError_t launch_check_graph(int n_nodes, int n_edges, const int32_t* row_ptr, const int32_t* senders,
                              unsigned long long* d_bad, hipStream_t st);

}  // namespace ctp
