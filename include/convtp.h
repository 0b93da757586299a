/*
 * convtp.h - C ABI of the fused equivariant convolution tensor product
 *            (MI355X / gfx950).
 *
 * The operation is the message-passing convolution of MACE-style interatomic
 * potentials that the e3j paper (arXiv 2609.35099) accelerates: abstract
 * (the forward of message-passing convolutions), Table 1 (convolution
 * throughput by channel count) and Table 2 (only the convolution block of
 * MACE runs on the dedicated kernels).  For every edge e = j -> i:
 *
 *   out[i, l3 m3, c] = sum_e sum_{p = (l1,l2,l3)} w[e, p, c]
 *                      sum_{m1,m2} C_p[m1][m2][m3] x[j, l1 m1, c] Y[e, l2 m2]
 *
 * with Y the real spherical harmonics of the edge direction and C_p the real
 * Clebsch-Gordan coupling of path p.  Messages are never written to memory.
 * The paths are all (l1,l2,l3) with l1 <= l_in, l2 <= l_sh, l3 <= l_out and
 * |l1-l2| <= l3 <= l1+l2 (the admissible couplings of FlashCart, arXiv
 * 2610.06409, section on spherical vs Cartesian products), in lexicographic
 * order, and all paths with the same l3 are summed into one output block.
 * The backward pass is the exact vector-Jacobian product (FlashCart, section
 * on symbolic VJPs).
 *
 * Conventions.  Component index d(l, m) = l*l + l + m, m = -l..l; the l = 1
 * block is proportional to (y, z, x).  Y is orthonormal on the sphere without
 * the Condon-Shortley phase; C_p is orthonormal (sum over m1,m2 of
 * C[m1,m2,m3] C[m1,m2,m3'] = delta) and, for odd l1+l2+l3, is the imaginary
 * part of the complex CG transformed to the real basis (so path (1,1,1) maps
 * Cartesian a, b to -(a x b)/sqrt 2).  A zero edge vector gives
 * Y_00 = 1/sqrt(4 pi), every other Y = 0 and a zero vector gradient.
 *
 * Layout (all arrays contiguous, channel index fastest):
 *   x[N][D_in][C], out[N][D_out][C], grad_out[N][D_out][C], dx[N][D_in][C]
 *   (D_out = (l_out+1)^2 for variant 0; for variant 1 see conv_tp_problem)
 *   w[E][P][C], dw[E][P][C]
 *   Y[E][D_sh] (y_mode 0) or vec[E][3] (y_mode 1); dY / dvec alike
 *   row_ptr[N+1], senders[E]: CSR by receiver (edges of receiver i are
 *   row_ptr[i] .. row_ptr[i+1]-1); every edge array is in this CSR order.
 *   send_ptr[N+1], send_perm[E], send_recv[E]: the same edges grouped by
 *   sender, stable in CSR edge id (from conv_tp_build_transpose).
 *   D_l = (l+1)^2, P = conv_tp_num_paths(...).
 *   N and E are int32, but element offsets are formed in 64 bits, so any
 *   array may hold more than 2^31 elements (w and dw of E*P*C elements).
 *
 * Memory and ownership.  Array pointers are DEVICE pointers unless marked
 * host.  The caller allocates and owns every buffer; the library never
 * allocates, frees or retains caller memory.  It owns only a few bytes of
 * per-device state for conv_tp_check_graph and the fixed scratch array of
 * conv_tp_bwd_msg_noalloc (256 MiB of device memory on each GPU the library
 * is loaded on, held until the process ends).  Outputs are overwritten, never
 * accumulated into; rows with no edges get exact zeros.  Inputs and outputs
 * must not overlap.
 *
 * Streams.  `stream` is a hipStream_t (0 = the null stream).  Every call
 * except conv_tp_check_graph enqueues its kernels and returns without
 * synchronising; kernel faults surface at the caller's next synchronisation.
 *
 * Errors.  Every argument check runs on the host before any HIP call, so an
 * invalid call never touches the device.  Device contents (index ranges,
 * monotone row pointers) are NOT checked on the hot path: out-of-range
 * indices are undefined behaviour; conv_tp_check_graph validates a graph.
 * On a non-zero status, conv_tp_last_error() returns a message (per thread).
 *
 * Degrees.  l_in, l_sh and l_out are independent, each 0..3 (64 triples;
 * MACE's first layer, for instance, has scalar inputs: l_in = 0).  Paths with
 * no admissible l3 <= l_out or l2 <= l_sh do not exist; output blocks that no
 * path reaches are exact zeros.
 *
 * Determinism.  algo 0 (CSR forward) and the backward sum in a fixed order
 * and are bitwise reproducible.  On grids of fewer than 4096 waves each
 * node's edge list is split between two workgroups whose two partial sums are
 * added with fp32 atomics onto a zeroed output; two addends onto zero give
 * the same result in either order, so this keeps the guarantee.  The same
 * holds for the channel sums (dY, dvec, g_y) above 512 channels, which two
 * channel tiles of at most 512 channels each add into a zeroed output.  algo
 * 1 (atomics: edge-parallel forward, receiver-major backward) is not
 * reproducible.
 */
#ifndef CONVTP_H
#define CONVTP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    CTP_OK = 0,
    CTP_EINVAL = 1,        /* null pointer, negative size, bad enum value */
    CTP_EUNSUPPORTED = 2,  /* degree outside 0..3, channels above 1024, algo 1 outside conv_tp_fwd/bwd, algo 2
                              with Y given, variant 1 or in an entry point other than conv_tp_fwd and
                              conv_tp_bwd, edge vectors where only Y is taken */
    CTP_EALIGN = 3,        /* a feature/weight array not 16-byte aligned, an index array not 4-byte aligned */
    CTP_EHIP = 4,          /* HIP launch or runtime error (message from hipGetErrorString) */
    CTP_EGRAPH = 5         /* graph arguments inconsistent (e.g. edges without nodes) */
};

typedef struct conv_tp_problem {
    int32_t n_nodes;   /* N >= 0 */
    int32_t n_edges;   /* E >= 0 */
    int32_t channels;  /* C, 1..1024 */
    int32_t l_in;      /* max degree of x, 0..3 */
    int32_t l_sh;      /* max degree of Y, 0..3 */
    int32_t l_out;     /* max degree of out, 0..3 (independent of l_in and l_sh) */
    int32_t y_mode;    /* 0: Y[E][D_sh] given; 1: vec[E][3] given, Y evaluated in-kernel */
    int32_t algo;      /* 0: CSR segmented sum, deterministic; 1: fp32 atomics (not reproducible);
                          2: in each edge's own frame (conv_tp_fwd and conv_tp_bwd; y_mode 1, variant 0) */
    int32_t variant;   /* 0: every triangle path, same-l3 paths summed into one block of D_out = (l_out+1)^2;
                          1: MACE's convolution - natural-parity paths only (l1+l2+l3 even; e3j Table 3's
                          MACE model, FlashCart's admissible-coupling section), each path with an output
                          slot of its own: out[N][D_out][C] with D_out = sum over paths of 2 l3 + 1, slots
                          in path order.  grad_out has the same layout as out.  See conv_tp_layout. */
} conv_tp_problem;

/* Number of paths P of variant 0 for the degrees, or -1 (with a message) if a
 * degree is outside 0..3.  Pure host function. */
int32_t conv_tp_num_paths(int32_t l_in, int32_t l_sh, int32_t l_out);

/* Path list of variant 0: l123 (host, [P][3]) receives (l1, l2, l3) of every
 * path in the order of w's second index.  Pure host function. */
int32_t conv_tp_paths(int32_t l_in, int32_t l_sh, int32_t l_out, int32_t *l123);

/* Path list and output width of a variant: *n_paths = P, *out_dim = D_out
 * (components per channel of out and grad_out), and, if l123 (host,
 * [P][3]) is not null, the paths in the order of w's second index.  Pure host
 * function; CTP_EINVAL for an unknown variant or a null count pointer,
 * CTP_EUNSUPPORTED for a degree outside 0..3. */
int32_t conv_tp_layout(int32_t variant, int32_t l_in, int32_t l_sh, int32_t l_out, int32_t *n_paths,
                       int32_t *out_dim, int32_t *l123);

/* The library's real coupling tensor of path (l1, l2, l3) in double
 * precision: out (host, [2l1+1][2l2+1][2l3+1]).  The kernels use these
 * values rounded to fp32.  Pure host function; CTP_EINVAL if the triangle
 * rule fails, CTP_EUNSUPPORTED for a degree above 3. */
int32_t conv_tp_coupling(int32_t l1, int32_t l2, int32_t l3, double *out);

/* Forward: out = conv(x, Y or vec, w) over the CSR graph.
 * algo 0: one workgroup per receiver sums its edges in CSR order.
 * algo 1: one workgroup per edge adds its message with fp32 atomics into
 * out, which the call first zeroes.
 * algo 2 (edge vectors only, variant 0): as algo 0, but each edge's product is
 * taken in the edge's own frame (E2Former-V2's abstract: SO(2)-style
 * sparsification): x is rotated so that the edge points along z, where the
 * harmonics are non-zero only at m = 0, coupled through the m2 = 0 slice of
 * every path, and the result rotated back.  The same result as algo 0 up to
 * rounding (deterministic, fixed order), with about 40% fewer FMAs per edge
 * and channel at l = 3.  CTP_EUNSUPPORTED with Y given or variant 1. */
int32_t conv_tp_fwd(const conv_tp_problem *prob, const float *x, const float *y_or_vec, const float *w,
                    const int32_t *row_ptr, const int32_t *senders, float *out, void *stream);

/* Backward for upstream gradient grad_out = dL/dout (the exact VJP of the
 * forward, FlashCart's section on symbolic VJPs): writes dx, dw and dY
 * (y_mode 0) or dvec = (dY/dvec)^T dY (y_mode 1).  One workgroup per sender
 * and channel tile walks the sender's out-edges through (send_ptr, send_perm,
 * send_recv), one channel per lane; dY is summed over the tile's channels in a
 * fixed order (up to 512 channels in one tile; two tiles above that, see
 * Determinism).  C up to 1024.
 * algo 0: direct.  algo 2 (edge vectors, variant 0): in each edge's frame, as
 * the algo 2 forward: x and grad_out are rotated so that the edge points along
 * z, coupled through the m2 = 0 slice of every path, dx rotated back, and of
 * the harmonic gradient only the m2 = +-1 components (the ones with a gradient
 * across the edge direction there) are formed for dvec.  The same result up
 * to rounding, about 45% fewer FMAs per edge and channel at l = 3.  algo 1:
 * one workgroup per receiver walks its in-edges (grad_out row read once, as
 * in conv_tp_bwd_msg) and adds each edge's dx contribution into dx[sender]
 * with fp32 atomics (dx zeroed first): no workspace and no second pass, but
 * dx is not bitwise reproducible (dw and dY are); the transpose arrays are
 * still required. */
int32_t conv_tp_bwd(const conv_tp_problem *prob, const float *grad_out, const float *x, const float *y_or_vec,
                    const float *w, const int32_t *row_ptr, const int32_t *senders, const int32_t *send_ptr,
                    const int32_t *send_perm, const int32_t *send_recv, float *dx, float *dw, float *dy_or_dvec,
                    void *stream);

/* The harmonic gradient alone: dY[e, l2 m2] = sum_c sum_p w[e,p,c]
 * sum_{m1,m3} C_p[m1][m2][m3] x[j, l1 m1, c] grad_out[i, l3 m3, c] (the dY of
 * conv_tp_bwd, FlashCart's symbolic-VJP section), without dx and dw.  It does
 * not depend on Y, so Y is not an argument.  dy (device, [E][D_sh]) is
 * overwritten; one workgroup per receiver keeps grad_out's row in registers
 * and sums over channels in a fixed order: bitwise equal to conv_tp_bwd's dY.
 * For recomputing dY where dx and dw are not needed (the edge-vector VJP of
 * the VJP).  y_mode must be 0 and algo 0 (CTP_EUNSUPPORTED otherwise); both
 * variants, C up to 1024. */
int32_t conv_tp_bwd_dy(const conv_tp_problem *prob, const float *grad_out, const float *x, const float *w,
                       const int32_t *row_ptr, const int32_t *senders, float *dy, void *stream);

/* Bytes of device workspace conv_tp_bwd_msg needs: E * D_in * C * 4 with
 * D_in = (l_in+1)^2.  Pure host function; errors as conv_tp_bwd's problem
 * checks, CTP_EINVAL for a null bytes pointer. */
int32_t conv_tp_bwd_msg_workspace(const conv_tp_problem *prob, int64_t *bytes);

/* The same backward (same arguments, outputs and math as conv_tp_bwd: the
 * exact VJP of FlashCart's section on symbolic VJPs; e3j's abstract reports
 * its kernels for the backward pass too) in two passes through a caller-owned
 * device workspace
 * msg[E][D_in][C] (CSR edge order, 16-byte aligned, at least
 * conv_tp_bwd_msg_workspace bytes, else CTP_EINVAL; contents on entry are
 * ignored and overwritten).  Pass 1, one workgroup per receiver i: G[i] is
 * read once, and for each in-edge e = j -> i in CSR order the kernel stores
 * dw[e], dY[e] (or dvec[e]) and the edge's message
 * msg[e] = sum_p w[e,p] (T_p(Y_e)^T G[i])_p, the edge's share of dx[j].
 * Pass 2: dx[j] = sum over j's out-edges in (send_ptr, send_perm) order of
 * msg[e].  For variant 1 the G row is much wider than x's (99 against 16
 * components at l = 3), so reading G once per receiver instead of once per
 * edge moves fewer bytes; for variant 0 conv_tp_bwd moves fewer.  dw and dY
 * are bitwise those of conv_tp_bwd; dx differs only in the order of its fp32
 * additions (per edge, then over edges) and is reproducible.  algo 0; C up to
 * 1024.  Calls that share a workspace must not overlap. */
int32_t conv_tp_bwd_msg(const conv_tp_problem *prob, const float *grad_out, const float *x, const float *y_or_vec,
                        const float *w, const int32_t *row_ptr, const int32_t *senders, const int32_t *send_ptr,
                        const int32_t *send_perm, const int32_t *send_recv, float *dx, float *dw,
                        float *dy_or_dvec, float *workspace, int64_t workspace_bytes, void *stream);

/* conv_tp_bwd_msg for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, outputs and kernels without the workspace arguments.
 * The edge messages go to a fixed scratch array of 256 MiB (268435456 bytes)
 * that the library holds on each device it runs on until the process ends; the
 * call itself allocates nothing.  Problems whose messages need more,
 * E * (l_in+1)^2 * C * 4 bytes > 268435456 (conv_tp_bwd_msg_workspace), are
 * rejected with CTP_EUNSUPPORTED before any HIP call.  The first call on a
 * device looks up that device's scratch address (hipGetSymbolAddress).
 * Calls on one device share the scratch, so calls that overlap on one device
 * (different streams or threads without ordering) race and give undefined
 * results; calls on one stream are ordered and safe. */
int32_t conv_tp_bwd_msg_noalloc(const conv_tp_problem *prob, const float *grad_out, const float *x,
                                const float *y_or_vec, const float *w, const int32_t *row_ptr,
                                const int32_t *senders, const int32_t *send_ptr, const int32_t *send_perm,
                                const int32_t *send_recv, float *dx, float *dw, float *dy_or_dvec, void *stream);

/* VJP of the backward (the "VJP-of-VJP" of FlashCart's section on symbolic
 * VJPs, needed to train on forces), Y given.  With cotangents a_x, a_w, a_y of
 * conv_tp_bwd's outputs (dx, dw, dY) and L2 = <a_x, dx> + <a_w, dw> + <a_y, dY>,
 * it writes g_x = dL2/dx [N][D_in][C], g_w = dL2/dw [E][P][C],
 * g_y = dL2/dY [E][D_sh] and g_grad = dL2/dgrad_out [N][D_out][C]:
 *   g_grad = F(a_x, w, Y) + F(x, a_w, Y) + F(x, w, a_y)   (F = conv_tp_fwd)
 *   g_x = dx with (w, Y) -> (a_w, Y) plus (w, a_y); g_w = dw with x -> a_x plus
 *   Y -> a_y; g_y = dY with x -> a_x plus w -> a_w.
 * Layouts and graph arrays as for conv_tp_bwd (a_x like x, a_w like w, a_y
 * like Y, g_grad like grad_out); both variants.  y_mode must be 0 and algo 0
 * (CTP_EUNSUPPORTED otherwise); C up to 1024.  Every output is written once in
 * a fixed order (bitwise reproducible; above 512 channels g_y as in
 * Determinism).  For edge vectors see conv_tp_sh_jvp / conv_tp_sh_bwd_bwd. */
int32_t conv_tp_bwd_bwd(const conv_tp_problem *prob, const float *grad_out, const float *x, const float *y,
                        const float *w, const float *a_x, const float *a_w, const float *a_y, const int32_t *row_ptr,
                        const int32_t *senders, const int32_t *send_ptr, const int32_t *send_perm,
                        const int32_t *send_recv, float *g_x, float *g_w, float *g_y, float *g_grad, void *stream);

/* Real spherical harmonics of edge vectors: Y[E][(l_sh+1)^2] from vec[E][3]. */
int32_t conv_tp_sh(int32_t n_edges, int32_t l_sh, const float *vec, float *Y, void *stream);

/* Vector gradient of the harmonics: dvec[e] = (dY/dvec)(vec_e)^T dY[e]. */
int32_t conv_tp_sh_bwd(int32_t n_edges, int32_t l_sh, const float *vec, const float *dY, float *dvec,
                       void *stream);

/* Second-order terms of the harmonics, for the VJP of the backward with edge
 * vectors (force training).  With Y = Y(vec), J = dY/dvec [E][D_sh][3]:
 *   conv_tp_sh_jvp:     a_y[e] = J(vec_e) a_vec[e]                    ([E][D_sh])
 *   conv_tp_sh_bwd_bwd: g_vec[e] = J^T g_y[e] + d/dvec <J a_vec[e], dY[e]>  ([E][3])
 * With cotangents (a_x, a_w, a_vec) of the edge-vector backward's (dx, dw,
 * dvec), its VJP is: a_y = conv_tp_sh_jvp(vec, a_vec); (g_x, g_w, g_y, g_grad)
 * = conv_tp_bwd_bwd with Y = conv_tp_sh(vec) and that a_y; g_vec =
 * conv_tp_sh_bwd_bwd(vec, dY, a_vec, g_y), where dY is the first backward's
 * harmonic gradient (conv_tp_bwd with Y given).  A zero vector gives zeros.
 * All arrays device, 4-byte aligned. */
int32_t conv_tp_sh_jvp(int32_t n_edges, int32_t l_sh, const float *vec, const float *a_vec, float *a_y,
                       void *stream);
int32_t conv_tp_sh_bwd_bwd(int32_t n_edges, int32_t l_sh, const float *vec, const float *dY, const float *a_vec,
                           const float *g_y, float *g_vec, void *stream);

/* The same VJP of the edge-vector backward in one call (FlashCart, section
 * on symbolic VJPs: the second-order pass of force training), the steps
 * above on `stream` in order: Y = conv_tp_sh(vec), a_y = conv_tp_sh_jvp(vec,
 * a_vec), dY = conv_tp_bwd_dy (only if dY is NULL), (g_x, g_w, g_y, g_grad) =
 * conv_tp_bwd_bwd, g_vec = conv_tp_sh_bwd_bwd(vec, dY, a_vec, g_y).
 * dY [E][D_sh] is the first backward's harmonic gradient (conv_tp_bwd with Y
 * = conv_tp_sh(vec) given) when the caller kept it, which saves its
 * recomputation; NULL computes it.  prob: y_mode 1, algo 0, either variant.
 * Inputs and outputs as for conv_tp_bwd_bwd with vec[E][3], a_vec[E][3] and
 * g_vec[E][3] in place of Y, a_y, g_y.  workspace: device, 16-byte aligned,
 * at least conv_tp_bwd_bwd_vec_workspace bytes (Y, a_y and g_y, plus dY when
 * not given, [E][D_sh] fp32 each), caller-owned, contents undefined after
 * the call; CTP_EINVAL if smaller.  Bitwise reproducible as
 * conv_tp_bwd_bwd. */
int32_t conv_tp_bwd_bwd_vec(const conv_tp_problem *prob, const float *grad_out, const float *x, const float *vec,
                            const float *w, const float *a_x, const float *a_w, const float *a_vec, const float *dY,
                            const int32_t *row_ptr, const int32_t *senders, const int32_t *send_ptr,
                            const int32_t *send_perm, const int32_t *send_recv, float *g_x, float *g_w, float *g_vec,
                            float *g_grad, float *workspace, int64_t workspace_bytes, void *stream);
/* Workspace bytes conv_tp_bwd_bwd_vec needs; dy_given: whether dY is passed. */
int32_t conv_tp_bwd_bwd_vec_workspace(const conv_tp_problem *prob, int32_t dy_given, int64_t *bytes);

/* Sender-sorted transpose of a CSR-by-receiver graph (the ordering of edges
 * by sender that FlashCart's section 4 names for deterministic gradients of
 * shared inputs): send_ptr[N+1], send_perm[E] (CSR edge ids, ascending within
 * each sender) and send_recv[E] (receiver of each).  Integer work, bit-exact
 * and deterministic.  The graph must be valid (conv_tp_check_graph); for an
 * invalid one the result is undefined but nothing outside the three output
 * arrays is written. */
int32_t conv_tp_build_transpose(int32_t n_nodes, int32_t n_edges, const int32_t *row_ptr, const int32_t *senders,
                                int32_t *send_ptr, int32_t *send_perm, int32_t *send_recv, void *stream);

/* Debug check of a CSR graph: *n_bad (host) receives the number of defects
 * (row_ptr[0] != 0, each decreasing step of row_ptr, row_ptr[N] != E, each
 * sender outside [0, N)).  Synchronises `stream`. */
int32_t conv_tp_check_graph(int32_t n_nodes, int32_t n_edges, const int32_t *row_ptr, const int32_t *senders,
                            int64_t *n_bad, void *stream);

/* ---------------------------------------------------------------------------
 * Node-local channelwise tensor product: the same paths and couplings applied
 * at each node to two of its own features, with per-node weights (e3j
 * abstract: tensor-product operations measured against HBM bandwidth;
 * FlashCart section 4: node-local products beside the edge convolutions):
 *
 *   out[i, l3 m3, c] = sum_{p = (l1,l2,l3)} w[i,p,c]
 *                      sum_{m1,m2} C_p[m1][m2][m3] x[i, l1 m1, c] y[i, l2 m2, c]
 *
 * Paths as for the convolution (lexicographic triangle paths, same-l3 paths
 * summed).  Layout: x[N][D][C], y[N][D][C], w[N][P][C], out[N][D][C], channel
 * fastest, all device pointers, 16-byte aligned, caller-owned, outputs
 * overwritten.  l_x = l_y = l_out in 0..3 (CTP_EUNSUPPORTED otherwise), C >= 1.
 * Every (node, channel) is independent, so results do not depend on the
 * launch shape and are bitwise reproducible. */
typedef struct conv_tp_node_problem {
    int32_t n_nodes;   /* N >= 0 */
    int32_t channels;  /* C >= 1 */
    int32_t l_x;       /* max degree of x, 0..3 */
    int32_t l_y;       /* max degree of y, 0..3 */
    int32_t l_out;     /* max degree of out, 0..3 */
} conv_tp_node_problem;

int32_t conv_tp_node_fwd(const conv_tp_node_problem *prob, const float *x, const float *y, const float *w,
                         float *out, void *stream);

/* Exact VJP for upstream gradient grad_out[N][D][C]: dx, dy (as x, y) and
 * dw[N][P][C]. */
int32_t conv_tp_node_bwd(const conv_tp_node_problem *prob, const float *grad_out, const float *x, const float *y,
                         const float *w, float *dx, float *dy, float *dw, void *stream);

/* Measurement helper, not part of the operation: plain HBM streams shaped
 * like the kernels' edge streams (16-byte non-temporal accesses, grid-stride
 * loop).  kind 0 reads src[n_floats] (dst receives at most one float, only
 * for a non-finite input), 1 writes dst[n_floats], 2 copies src to dst;
 * kinds 3, 4 and 5 are the same streams with 4-byte accesses per lane (the
 * width of the kernels' one-channel-per-lane row accesses).  They
 * measure the bandwidth this device sustains for each traffic mix, against
 * which the kernels' fractions of the data-sheet HBM peak are read (e3j
 * abstract: throughput quoted as a fraction of maximum HBM bandwidth).
 * n_floats must be a multiple of 4; src and dst 16-byte aligned device
 * pointers.  Enqueued on `stream`. */
int32_t conv_tp_stream_probe(int32_t kind, const float *src, float *dst, int64_t n_floats, void *stream);

/* Measurement helper, not part of the operation: an fp32 FMA kernel without
 * packed instructions (the build of every kernel here excludes them), eight
 * independent chains per lane, enough workgroups for eight waves per SIMD on
 * every CU.  *fmas (host) receives the number of FMAs one launch performs;
 * timing the launch gives the FMA rate the vector ALUs sustain, against
 * which arithmetic-bound kernels are read.  dst (device, >= 1 float, 4-byte
 * aligned) receives a value only for a non-finite result.  iterations >= 0. */
int32_t conv_tp_valu_probe(int64_t iterations, float *dst, int64_t *fmas, void *stream);

/* Message for the last non-zero status on this thread ("" if none). */
const char *conv_tp_last_error(void);

/* ABI version (major * 100 + minor): 101 added conv_tp_problem.variant, 102
 * conv_tp_bwd_msg, 103 algo 2 (edge-frame forward), 104 conv_tp_bwd_dy, 105
 * independent degrees, up to 1024 channels in every backward and variant 1
 * in conv_tp_bwd_bwd, 106 conv_tp_bwd_msg_noalloc, 107 conv_tp_valu_probe and algo 2 in
 * conv_tp_bwd, 108 conv_tp_bwd_bwd_vec, 109 algo 1 in conv_tp_bwd, 110 4-byte stream
 * probes. */
int32_t conv_tp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CONVTP_H */
