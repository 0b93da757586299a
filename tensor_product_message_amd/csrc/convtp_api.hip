// C ABI front: argument validation (host only, before any HIP call), error
// reporting, path/coupling queries and kernel dispatch.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>
#include <unordered_map>

#include "../../include/convtp.h"
#include "kernels.hpp"
#include "tables.hpp"

namespace {

thread_local std::string g_last_error;

// node-local products: a row of D * C floats must stay addressable by a
// 32-bit byte offset
constexpr int kNodeMaxChannels = 1 << 20;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return CTP_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(CTP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// A pointer is required when its array has elements; alignment is checked
// whenever it is non-null.
int need(const void* p, int64_t count, uintptr_t align, const char* name) {
    if (count > 0 && p == nullptr) return fail(CTP_EINVAL, "%s is null but has %lld elements", name, (long long)count);
    if (p != nullptr && !aligned(p, align))
        return fail(CTP_EALIGN, "%s is not %u-byte aligned", name, (unsigned)align);
    return CTP_OK;
}

int check_degree(int l, const char* name) {
    if (l < 0 || l > ctp::kMaxL) return fail(CTP_EUNSUPPORTED, "%s = %d outside 0..%d", name, l, ctp::kMaxL);
    return CTP_OK;
}

struct Shape {
    int64_t N, E, C, D1, D2, D3, P, S;
};

int check_problem(const conv_tp_problem* pr, Shape* s) {
    if (pr == nullptr) return fail(CTP_EINVAL, "problem is null");
    if (pr->n_nodes < 0 || pr->n_edges < 0) return fail(CTP_EINVAL, "negative node or edge count");
    if (pr->channels < 1) return fail(CTP_EINVAL, "channels = %d must be >= 1", pr->channels);
    if (pr->channels > ctp::kMaxChannels)
        return fail(CTP_EUNSUPPORTED, "channels = %d above %d", pr->channels, ctp::kMaxChannels);
    if (int r = check_degree(pr->l_in, "l_in")) return r;
    if (int r = check_degree(pr->l_sh, "l_sh")) return r;
    if (int r = check_degree(pr->l_out, "l_out")) return r;
    if (pr->y_mode != 0 && pr->y_mode != 1) return fail(CTP_EINVAL, "y_mode = %d not 0 or 1", pr->y_mode);
    if (pr->algo < 0 || pr->algo > 2) return fail(CTP_EINVAL, "algo = %d not 0, 1 or 2", pr->algo);
    if (pr->variant != ctp::kVariantSummed && pr->variant != ctp::kVariantSlots)
        return fail(CTP_EINVAL, "variant = %d not 0 or 1", pr->variant);
    if (pr->n_nodes == 0 && pr->n_edges > 0) return fail(CTP_EGRAPH, "edges without nodes");
    s->N = pr->n_nodes;
    s->E = pr->n_edges;
    s->C = pr->channels;
    s->D1 = ctp::dim_of(pr->l_in);
    s->D2 = ctp::dim_of(pr->l_sh);
    s->D3 = ctp::out_dim(pr->l_in, pr->l_sh, pr->l_out, pr->variant);   // out and grad_out components
    s->P = ctp::num_paths(pr->l_in, pr->l_sh, pr->l_out, pr->variant);
    s->S = pr->y_mode ? 3 : s->D2;
    return CTP_OK;
}

ctp::LaunchArgs base_args(const conv_tp_problem* pr) {
    ctp::LaunchArgs a{};
    a.l_in = pr->l_in;
    a.l_sh = pr->l_sh;
    a.l_out = pr->l_out;
    a.n_nodes = pr->n_nodes;
    a.n_edges = pr->n_edges;
    a.C = pr->channels;
    a.algo = pr->algo;
    a.vec_mode = pr->y_mode;
    a.variant = pr->variant;
    return a;
}

// Checks shared by the two backward entry points; fills the launch arguments.
int bwd_args(const conv_tp_problem* prob, const float* grad_out, const float* x, const float* y_or_vec,
             const float* w, const int32_t* row_ptr, const int32_t* senders, const int32_t* send_ptr,
             const int32_t* send_perm, const int32_t* send_recv, float* dx, float* dw, float* dy_or_dvec, Shape* sp,
             ctp::LaunchArgs* out) {
    Shape& s = *sp;
    if (int r = check_problem(prob, &s)) return r;
    if (prob->algo == 2 && (prob->y_mode != 1 || prob->variant != ctp::kVariantSummed))
        return fail(CTP_EUNSUPPORTED, "algo 2 (edge frame) needs edge vectors (y_mode 1) and variant 0");
    if (int r = need(grad_out, s.N * s.D3 * s.C, 16, "grad_out")) return r;
    if (int r = need(x, s.N * s.D1 * s.C, 16, "x")) return r;
    if (int r = need(y_or_vec, s.E * s.S, 4, "y_or_vec")) return r;
    if (int r = need(w, s.E * s.P * s.C, 16, "w")) return r;
    if (int r = need(row_ptr, s.N + 1, 4, "row_ptr")) return r;
    if (int r = need(senders, s.E, 4, "senders")) return r;
    if (int r = need(send_ptr, s.N + 1, 4, "send_ptr")) return r;
    if (int r = need(send_perm, s.E, 4, "send_perm")) return r;
    if (int r = need(send_recv, s.E, 4, "send_recv")) return r;
    if (int r = need(dx, s.N * s.D1 * s.C, 16, "dx")) return r;
    if (int r = need(dw, s.E * s.P * s.C, 16, "dw")) return r;
    if (int r = need(dy_or_dvec, s.E * s.S, 4, "dy_or_dvec")) return r;
    ctp::LaunchArgs a = base_args(prob);
    a.grad = grad_out;
    a.x = x;
    a.y = y_or_vec;
    a.w = w;
    a.row_ptr = row_ptr;
    a.senders = senders;
    a.send_ptr = send_ptr;
    a.send_perm = send_perm;
    a.send_recv = send_recv;
    a.dx = dx;
    a.dw = dw;
    a.dy = dy_or_dvec;
    *out = a;
    return CTP_OK;
}

int64_t msg_workspace_bytes(const Shape& s) { return s.E * s.D1 * s.C * (int64_t)sizeof(float); }

std::mutex g_bad_mu;
std::unordered_map<int, unsigned long long*> g_bad_buf;   // per-device counter for conv_tp_check_graph

// Edge-message workspace of conv_tp_bwd_msg_noalloc: a file-scope device
// array, so that call allocates nothing.  Every device the library runs on
// holds its own copy (at its own address) until the process ends.  Its host
// name is only a stand-in for the symbol: host code uses the per-device
// address from hipGetSymbolAddress, never `scratch` itself.
constexpr int64_t kNoAllocScratchBytes = int64_t(256) << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

std::mutex g_scratch_mu;
std::unordered_map<int, float*> g_scratch_ptr;   // device id -> address of that device's `scratch`

// Address of `scratch` on the current device, looked up once per device (with
// that device current) and kept.
int scratch_on_current_device(float** out) {
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_status(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it != g_scratch_ptr.end()) {
        *out = it->second;
        return CTP_OK;
    }
    float* ptr = nullptr;
    if (hipError_t e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)); e != hipSuccess)
        return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(CTP_EHIP, "hipGetSymbolAddress(scratch) returned null");
    g_scratch_ptr[dev] = ptr;
    *out = ptr;
    return CTP_OK;
}

}  // namespace

namespace ctp {

int host_num_paths(int l1, int l2, int l3, int variant) { return num_paths(l1, l2, l3, variant); }

int host_out_dim(int l1, int l2, int l3, int variant) { return out_dim(l1, l2, l3, variant); }

int host_paths(int l_in, int l_sh, int l_out, int32_t* l123, int variant) {
    int n = 0;
    for (int a = 0; a <= l_in; ++a)
        for (int b = 0; b <= l_sh; ++b)
            for (int c = 0; c <= l_out; ++c)
                if (path_ok(a, b, c, variant)) {
                    l123[3 * n] = a;
                    l123[3 * n + 1] = b;
                    l123[3 * n + 2] = c;
                    ++n;
                }
    return n;
}

int host_coupling(int l1, int l2, int l3, double* out) {
    const int n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
    for (int a = 0; a < 2 * l1 + 1; ++a)
        for (int b = 0; b < n2; ++b)
            for (int c = 0; c < n3; ++c)
                out[(a * n2 + b) * n3 + c] = real_coupling(l1, l2, l3, a - l1, b - l2, c - l3);
    return 0;
}

}  // namespace ctp

extern "C" {

int32_t conv_tp_version(void) { return 110; }

const char* conv_tp_last_error(void) { return g_last_error.c_str(); }

int32_t conv_tp_num_paths(int32_t l_in, int32_t l_sh, int32_t l_out) {
    if (check_degree(l_in, "l_in") || check_degree(l_sh, "l_sh") || check_degree(l_out, "l_out")) return -1;
    ok();
    return ctp::host_num_paths(l_in, l_sh, l_out);
}

int32_t conv_tp_paths(int32_t l_in, int32_t l_sh, int32_t l_out, int32_t* l123) {
    if (int r = check_degree(l_in, "l_in")) return r;
    if (int r = check_degree(l_sh, "l_sh")) return r;
    if (int r = check_degree(l_out, "l_out")) return r;
    if (l123 == nullptr) return fail(CTP_EINVAL, "l123 is null");
    ctp::host_paths(l_in, l_sh, l_out, l123);
    return ok();
}

int32_t conv_tp_layout(int32_t variant, int32_t l_in, int32_t l_sh, int32_t l_out, int32_t* n_paths,
                       int32_t* out_dim, int32_t* l123) {
    if (variant != ctp::kVariantSummed && variant != ctp::kVariantSlots)
        return fail(CTP_EINVAL, "variant = %d not 0 or 1", variant);
    if (int r = check_degree(l_in, "l_in")) return r;
    if (int r = check_degree(l_sh, "l_sh")) return r;
    if (int r = check_degree(l_out, "l_out")) return r;
    if (n_paths == nullptr || out_dim == nullptr) return fail(CTP_EINVAL, "n_paths or out_dim is null");
    *n_paths = ctp::host_num_paths(l_in, l_sh, l_out, variant);
    *out_dim = ctp::host_out_dim(l_in, l_sh, l_out, variant);
    if (l123 != nullptr) ctp::host_paths(l_in, l_sh, l_out, l123, variant);
    return ok();
}

int32_t conv_tp_coupling(int32_t l1, int32_t l2, int32_t l3, double* out) {
    if (int r = check_degree(l1, "l1")) return r;
    if (int r = check_degree(l2, "l2")) return r;
    if (int r = check_degree(l3, "l3")) return r;
    if (!ctp::triangle(l1, l2, l3)) return fail(CTP_EINVAL, "path (%d,%d,%d) violates the triangle rule", l1, l2, l3);
    if (out == nullptr) return fail(CTP_EINVAL, "out is null");
    ctp::host_coupling(l1, l2, l3, out);
    return ok();
}

int32_t conv_tp_fwd(const conv_tp_problem* prob, const float* x, const float* y_or_vec, const float* w,
                    const int32_t* row_ptr, const int32_t* senders, float* out, void* stream) {
    Shape s{};
    if (int r = check_problem(prob, &s)) return r;
    if (prob->algo == 2 && (prob->y_mode != 1 || prob->variant != ctp::kVariantSummed))
        return fail(CTP_EUNSUPPORTED, "algo 2 (edge frame) needs edge vectors (y_mode 1) and variant 0");
    if (int r = need(x, s.N * s.D1 * s.C, 16, "x")) return r;
    if (int r = need(y_or_vec, s.E * s.S, 4, "y_or_vec")) return r;
    if (int r = need(w, s.E * s.P * s.C, 16, "w")) return r;
    if (int r = need(row_ptr, s.N + 1, 4, "row_ptr")) return r;
    if (int r = need(senders, s.E, 4, "senders")) return r;
    if (int r = need(out, s.N * s.D3 * s.C, 16, "out")) return r;
    ctp::LaunchArgs a = base_args(prob);
    a.x = x;
    a.y = y_or_vec;
    a.w = w;
    a.row_ptr = row_ptr;
    a.senders = senders;
    a.out = out;
    return hip_status(ctp::launch_fwd(a, static_cast<hipStream_t>(stream)), "conv_tp_fwd launch");
}


int32_t conv_tp_bwd(const conv_tp_problem* prob, const float* grad_out, const float* x, const float* y_or_vec,
                    const float* w, const int32_t* row_ptr, const int32_t* senders, const int32_t* send_ptr,
                    const int32_t* send_perm, const int32_t* send_recv, float* dx, float* dw, float* dy_or_dvec,
                    void* stream) {
    Shape s{};
    ctp::LaunchArgs a{};
    if (int r = bwd_args(prob, grad_out, x, y_or_vec, w, row_ptr, senders, send_ptr, send_perm, send_recv, dx, dw,
                         dy_or_dvec, &s, &a))
        return r;
    return hip_status(ctp::launch_bwd(a, static_cast<hipStream_t>(stream)), "conv_tp_bwd launch");
}

int32_t conv_tp_bwd_dy(const conv_tp_problem* prob, const float* grad_out, const float* x, const float* w,
                       const int32_t* row_ptr, const int32_t* senders, float* dy, void* stream) {
    Shape s{};
    if (int r = check_problem(prob, &s)) return r;
    if (prob->algo != 0) return fail(CTP_EUNSUPPORTED, "conv_tp_bwd_dy has only the deterministic algorithm (algo 0)");
    if (prob->y_mode != 0) return fail(CTP_EUNSUPPORTED, "conv_tp_bwd_dy writes dY: y_mode must be 0");
    if (int r = need(grad_out, s.N * s.D3 * s.C, 16, "grad_out")) return r;
    if (int r = need(x, s.N * s.D1 * s.C, 16, "x")) return r;
    if (int r = need(w, s.E * s.P * s.C, 16, "w")) return r;
    if (int r = need(row_ptr, s.N + 1, 4, "row_ptr")) return r;
    if (int r = need(senders, s.E, 4, "senders")) return r;
    if (int r = need(dy, s.E * s.D2, 4, "dy")) return r;
    ctp::LaunchArgs a = base_args(prob);
    a.grad = grad_out;
    a.x = x;
    a.w = w;
    a.row_ptr = row_ptr;
    a.senders = senders;
    a.dy = dy;
    return hip_status(ctp::launch_bwd_dy(a, static_cast<hipStream_t>(stream)), "conv_tp_bwd_dy launch");
}

int32_t conv_tp_bwd_msg_workspace(const conv_tp_problem* prob, int64_t* bytes) {
    Shape s{};
    if (int r = check_problem(prob, &s)) return r;
    if (bytes == nullptr) return fail(CTP_EINVAL, "bytes is null");
    *bytes = msg_workspace_bytes(s);
    return ok();
}

int32_t conv_tp_bwd_msg(const conv_tp_problem* prob, const float* grad_out, const float* x, const float* y_or_vec,
                        const float* w, const int32_t* row_ptr, const int32_t* senders, const int32_t* send_ptr,
                        const int32_t* send_perm, const int32_t* send_recv, float* dx, float* dw, float* dy_or_dvec,
                        float* workspace, int64_t workspace_bytes, void* stream) {
    Shape s{};
    ctp::LaunchArgs a{};
    if (int r = bwd_args(prob, grad_out, x, y_or_vec, w, row_ptr, senders, send_ptr, send_perm, send_recv, dx, dw,
                         dy_or_dvec, &s, &a))
        return r;
    if (prob->algo != 0) return fail(CTP_EUNSUPPORTED, "conv_tp_bwd_msg has only the direct algorithm (algo 0)");
    const int64_t need_bytes = msg_workspace_bytes(s);
    if (workspace_bytes < need_bytes)
        return fail(CTP_EINVAL, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                    (long long)need_bytes);
    if (int r = need(workspace, s.E * s.D1 * s.C, 16, "workspace")) return r;
    return hip_status(ctp::launch_bwd_msg(a, workspace, static_cast<hipStream_t>(stream)), "conv_tp_bwd_msg launch");
}

int32_t conv_tp_bwd_msg_noalloc(const conv_tp_problem* prob, const float* grad_out, const float* x,
                                const float* y_or_vec, const float* w, const int32_t* row_ptr,
                                const int32_t* senders, const int32_t* send_ptr, const int32_t* send_perm,
                                const int32_t* send_recv, float* dx, float* dw, float* dy_or_dvec, void* stream) {
    Shape s{};
    ctp::LaunchArgs a{};
    if (int r = bwd_args(prob, grad_out, x, y_or_vec, w, row_ptr, senders, send_ptr, send_perm, send_recv, dx, dw,
                         dy_or_dvec, &s, &a))
        return r;
    if (prob->algo != 0)
        return fail(CTP_EUNSUPPORTED, "conv_tp_bwd_msg_noalloc has only the direct algorithm (algo 0)");
    const int64_t need_bytes = msg_workspace_bytes(s);
    if (need_bytes > kNoAllocScratchBytes)
        return fail(CTP_EUNSUPPORTED,
                    "conv_tp_bwd_msg_noalloc: the edge messages need %lld bytes (E * (l_in+1)^2 * C * 4), above its "
                    "fixed scratch of %lld bytes; call conv_tp_bwd_msg with a workspace instead",
                    (long long)need_bytes, (long long)kNoAllocScratchBytes);
    if (prob->n_nodes == 0) return ok();
    float* ws = nullptr;
    if (int r = scratch_on_current_device(&ws)) return r;
    // pass 1 writes every message row before pass 2 reads it: nothing to clear
    return hip_status(ctp::launch_bwd_msg(a, ws, static_cast<hipStream_t>(stream)),
                      "conv_tp_bwd_msg_noalloc launch");
}

int32_t conv_tp_bwd_bwd(const conv_tp_problem* prob, const float* grad_out, const float* x, const float* y,
                        const float* w, const float* a_x, const float* a_w, const float* a_y, const int32_t* row_ptr,
                        const int32_t* senders, const int32_t* send_ptr, const int32_t* send_perm,
                        const int32_t* send_recv, float* g_x, float* g_w, float* g_y, float* g_grad, void* stream) {
    Shape s{};
    if (int r = check_problem(prob, &s)) return r;
    if (prob->algo != 0) return fail(CTP_EUNSUPPORTED, "the double backward has only the deterministic algorithm");
    if (prob->y_mode != 0) return fail(CTP_EUNSUPPORTED, "the double backward takes Y (y_mode 0)");
    if (int r = need(grad_out, s.N * s.D3 * s.C, 16, "grad_out")) return r;
    if (int r = need(x, s.N * s.D1 * s.C, 16, "x")) return r;
    if (int r = need(y, s.E * s.D2, 4, "y")) return r;
    if (int r = need(w, s.E * s.P * s.C, 16, "w")) return r;
    if (int r = need(a_x, s.N * s.D1 * s.C, 16, "a_x")) return r;
    if (int r = need(a_w, s.E * s.P * s.C, 16, "a_w")) return r;
    if (int r = need(a_y, s.E * s.D2, 4, "a_y")) return r;
    if (int r = need(row_ptr, s.N + 1, 4, "row_ptr")) return r;
    if (int r = need(senders, s.E, 4, "senders")) return r;
    if (int r = need(send_ptr, s.N + 1, 4, "send_ptr")) return r;
    if (int r = need(send_perm, s.E, 4, "send_perm")) return r;
    if (int r = need(send_recv, s.E, 4, "send_recv")) return r;
    if (int r = need(g_x, s.N * s.D1 * s.C, 16, "g_x")) return r;
    if (int r = need(g_w, s.E * s.P * s.C, 16, "g_w")) return r;
    if (int r = need(g_y, s.E * s.D2, 4, "g_y")) return r;
    if (int r = need(g_grad, s.N * s.D3 * s.C, 16, "g_grad")) return r;
    ctp::DoubleArgs a{};
    a.l_in = prob->l_in;
    a.l_sh = prob->l_sh;
    a.l_out = prob->l_out;
    a.variant = prob->variant;
    a.n_nodes = prob->n_nodes;
    a.n_edges = prob->n_edges;
    a.C = prob->channels;
    a.x = x;
    a.ax = a_x;
    a.y = y;
    a.ay = a_y;
    a.w = w;
    a.aw = a_w;
    a.grad = grad_out;
    a.row_ptr = row_ptr;
    a.senders = senders;
    a.send_ptr = send_ptr;
    a.send_perm = send_perm;
    a.send_recv = send_recv;
    a.g_x = g_x;
    a.g_w = g_w;
    a.g_y = g_y;
    a.g_grad = g_grad;
    return hip_status(ctp::launch_double_bwd(a, static_cast<hipStream_t>(stream)), "conv_tp_bwd_bwd launch");
}

// Y, a_y and g_y, plus dY when the caller does not pass it: [E][D_sh] fp32 each.
int64_t dd_vec_workspace_bytes(const Shape& s, bool dy_given) {
    return (dy_given ? 3 : 4) * s.E * s.D2 * (int64_t)sizeof(float);
}

int32_t conv_tp_bwd_bwd_vec_workspace(const conv_tp_problem* prob, int32_t dy_given, int64_t* bytes) {
    Shape s{};
    if (int r = check_problem(prob, &s)) return r;
    if (bytes == nullptr) return fail(CTP_EINVAL, "bytes is null");
    *bytes = dd_vec_workspace_bytes(s, dy_given != 0);
    return ok();
}

int32_t conv_tp_bwd_bwd_vec(const conv_tp_problem* prob, const float* grad_out, const float* x, const float* vec,
                            const float* w, const float* a_x, const float* a_w, const float* a_vec, const float* dY,
                            const int32_t* row_ptr, const int32_t* senders, const int32_t* send_ptr,
                            const int32_t* send_perm, const int32_t* send_recv, float* g_x, float* g_w,
                            float* g_vec, float* g_grad, float* workspace, int64_t workspace_bytes, void* stream) {
    Shape s{};
    if (int r = check_problem(prob, &s)) return r;
    if (prob->algo != 0) return fail(CTP_EUNSUPPORTED, "the double backward has only the deterministic algorithm");
    if (prob->y_mode != 1) return fail(CTP_EUNSUPPORTED, "conv_tp_bwd_bwd_vec takes edge vectors (y_mode 1)");
    if (int r = need(grad_out, s.N * s.D3 * s.C, 16, "grad_out")) return r;
    if (int r = need(x, s.N * s.D1 * s.C, 16, "x")) return r;
    if (int r = need(vec, s.E * 3, 4, "vec")) return r;
    if (int r = need(w, s.E * s.P * s.C, 16, "w")) return r;
    if (int r = need(a_x, s.N * s.D1 * s.C, 16, "a_x")) return r;
    if (int r = need(a_w, s.E * s.P * s.C, 16, "a_w")) return r;
    if (int r = need(a_vec, s.E * 3, 4, "a_vec")) return r;
    if (int r = need(dY, 0, 4, "dY")) return r;   // optional
    if (int r = need(row_ptr, s.N + 1, 4, "row_ptr")) return r;
    if (int r = need(senders, s.E, 4, "senders")) return r;
    if (int r = need(send_ptr, s.N + 1, 4, "send_ptr")) return r;
    if (int r = need(send_perm, s.E, 4, "send_perm")) return r;
    if (int r = need(send_recv, s.E, 4, "send_recv")) return r;
    if (int r = need(g_x, s.N * s.D1 * s.C, 16, "g_x")) return r;
    if (int r = need(g_w, s.E * s.P * s.C, 16, "g_w")) return r;
    if (int r = need(g_vec, s.E * 3, 4, "g_vec")) return r;
    if (int r = need(g_grad, s.N * s.D3 * s.C, 16, "g_grad")) return r;
    const int64_t need_bytes = dd_vec_workspace_bytes(s, dY != nullptr);
    if (workspace_bytes < need_bytes)
        return fail(CTP_EINVAL, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                    (long long)need_bytes);
    if (int r = need(workspace, need_bytes / (int64_t)sizeof(float), 16, "workspace")) return r;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t ed = s.E * s.D2;
    float* Y = workspace;
    float* a_y = workspace + ed;
    float* g_y = workspace + 2 * ed;
    const float* dYv = dY;
    if (s.E > 0) {
        if (hipError_t e = ctp::launch_sh(prob->l_sh, s.E, vec, Y, st); e != hipSuccess)
            return hip_status(e, "conv_tp_bwd_bwd_vec: harmonics");
        if (hipError_t e = ctp::launch_sh_jvp(prob->l_sh, s.E, vec, a_vec, a_y, st); e != hipSuccess)
            return hip_status(e, "conv_tp_bwd_bwd_vec: harmonic JVP");
    }
    if (dYv == nullptr) {
        float* dYw = workspace + 3 * ed;
        ctp::LaunchArgs a = base_args(prob);
        a.vec_mode = 0;
        a.grad = grad_out;
        a.x = x;
        a.w = w;
        a.row_ptr = row_ptr;
        a.senders = senders;
        a.dy = dYw;
        if (hipError_t e = ctp::launch_bwd_dy(a, st); e != hipSuccess)
            return hip_status(e, "conv_tp_bwd_bwd_vec: harmonic gradient");
        dYv = dYw;
    }
    ctp::DoubleArgs a{};
    a.l_in = prob->l_in;
    a.l_sh = prob->l_sh;
    a.l_out = prob->l_out;
    a.variant = prob->variant;
    a.n_nodes = prob->n_nodes;
    a.n_edges = prob->n_edges;
    a.C = prob->channels;
    a.x = x;
    a.ax = a_x;
    a.y = Y;
    a.ay = a_y;
    a.w = w;
    a.aw = a_w;
    a.grad = grad_out;
    a.row_ptr = row_ptr;
    a.senders = senders;
    a.send_ptr = send_ptr;
    a.send_perm = send_perm;
    a.send_recv = send_recv;
    a.g_x = g_x;
    a.g_w = g_w;
    a.g_y = g_y;
    a.g_grad = g_grad;
    if (hipError_t e = ctp::launch_double_bwd(a, st); e != hipSuccess)
        return hip_status(e, "conv_tp_bwd_bwd_vec: double backward");
    if (s.E == 0) return ok();
    return hip_status(ctp::launch_sh_bwd_bwd(prob->l_sh, s.E, vec, dYv, a_vec, g_y, g_vec, st),
                      "conv_tp_bwd_bwd_vec: harmonic second-order term");
}

int32_t conv_tp_sh(int32_t n_edges, int32_t l_sh, const float* vec, float* Y, void* stream) {
    if (n_edges < 0) return fail(CTP_EINVAL, "negative edge count");
    if (int r = check_degree(l_sh, "l_sh")) return r;
    if (int r = need(vec, (int64_t)n_edges * 3, 4, "vec")) return r;
    if (int r = need(Y, (int64_t)n_edges * ctp::dim_of(l_sh), 4, "Y")) return r;
    return hip_status(ctp::launch_sh(l_sh, n_edges, vec, Y, static_cast<hipStream_t>(stream)), "conv_tp_sh launch");
}

int32_t conv_tp_sh_bwd(int32_t n_edges, int32_t l_sh, const float* vec, const float* dY, float* dvec,
                       void* stream) {
    if (n_edges < 0) return fail(CTP_EINVAL, "negative edge count");
    if (int r = check_degree(l_sh, "l_sh")) return r;
    if (int r = need(vec, (int64_t)n_edges * 3, 4, "vec")) return r;
    if (int r = need(dY, (int64_t)n_edges * ctp::dim_of(l_sh), 4, "dY")) return r;
    if (int r = need(dvec, (int64_t)n_edges * 3, 4, "dvec")) return r;
    return hip_status(ctp::launch_sh_bwd(l_sh, n_edges, vec, dY, dvec, static_cast<hipStream_t>(stream)),
                      "conv_tp_sh_bwd launch");
}

int32_t conv_tp_sh_jvp(int32_t n_edges, int32_t l_sh, const float* vec, const float* a_vec, float* a_y,
                       void* stream) {
    if (n_edges < 0) return fail(CTP_EINVAL, "negative edge count");
    if (int r = check_degree(l_sh, "l_sh")) return r;
    if (int r = need(vec, (int64_t)n_edges * 3, 4, "vec")) return r;
    if (int r = need(a_vec, (int64_t)n_edges * 3, 4, "a_vec")) return r;
    if (int r = need(a_y, (int64_t)n_edges * ctp::dim_of(l_sh), 4, "a_y")) return r;
    return hip_status(ctp::launch_sh_jvp(l_sh, n_edges, vec, a_vec, a_y, static_cast<hipStream_t>(stream)),
                      "conv_tp_sh_jvp launch");
}

int32_t conv_tp_sh_bwd_bwd(int32_t n_edges, int32_t l_sh, const float* vec, const float* dY, const float* a_vec,
                           const float* g_y, float* g_vec, void* stream) {
    if (n_edges < 0) return fail(CTP_EINVAL, "negative edge count");
    if (int r = check_degree(l_sh, "l_sh")) return r;
    const int64_t D = ctp::dim_of(l_sh);
    if (int r = need(vec, (int64_t)n_edges * 3, 4, "vec")) return r;
    if (int r = need(dY, (int64_t)n_edges * D, 4, "dY")) return r;
    if (int r = need(a_vec, (int64_t)n_edges * 3, 4, "a_vec")) return r;
    if (int r = need(g_y, (int64_t)n_edges * D, 4, "g_y")) return r;
    if (int r = need(g_vec, (int64_t)n_edges * 3, 4, "g_vec")) return r;
    return hip_status(ctp::launch_sh_bwd_bwd(l_sh, n_edges, vec, dY, a_vec, g_y, g_vec,
                                             static_cast<hipStream_t>(stream)),
                      "conv_tp_sh_bwd_bwd launch");
}

int32_t conv_tp_build_transpose(int32_t n_nodes, int32_t n_edges, const int32_t* row_ptr, const int32_t* senders,
                                int32_t* send_ptr, int32_t* send_perm, int32_t* send_recv, void* stream) {
    if (n_nodes < 0 || n_edges < 0) return fail(CTP_EINVAL, "negative node or edge count");
    if (n_nodes == 0 && n_edges > 0) return fail(CTP_EGRAPH, "edges without nodes");
    if (int r = need(row_ptr, (int64_t)n_nodes + 1, 4, "row_ptr")) return r;
    if (int r = need(senders, n_edges, 4, "senders")) return r;
    if (int r = need(send_ptr, (int64_t)n_nodes + 1, 4, "send_ptr")) return r;
    if (int r = need(send_perm, n_edges, 4, "send_perm")) return r;
    if (int r = need(send_recv, n_edges, 4, "send_recv")) return r;
    return hip_status(ctp::launch_transpose(n_nodes, n_edges, row_ptr, senders, send_ptr, send_perm, send_recv,
                                            static_cast<hipStream_t>(stream)),
                      "conv_tp_build_transpose launch");
}

namespace {

int check_node_problem(const conv_tp_node_problem* pr) {
    if (pr == nullptr) return fail(CTP_EINVAL, "problem is null");
    if (pr->n_nodes < 0) return fail(CTP_EINVAL, "negative node count");
    if (pr->channels < 1) return fail(CTP_EINVAL, "channels = %d must be >= 1", pr->channels);
    if (pr->channels > kNodeMaxChannels)
        return fail(CTP_EUNSUPPORTED, "channels = %d above %d", pr->channels, kNodeMaxChannels);
    if (int r = check_degree(pr->l_x, "l_x")) return r;
    if (int r = check_degree(pr->l_y, "l_y")) return r;
    if (int r = check_degree(pr->l_out, "l_out")) return r;
    if (pr->l_x != pr->l_y || pr->l_y != pr->l_out)
        return fail(CTP_EUNSUPPORTED, "degrees (%d,%d,%d) must be equal in this build", pr->l_x, pr->l_y, pr->l_out);
    return CTP_OK;
}

}  // namespace

int32_t conv_tp_node_fwd(const conv_tp_node_problem* prob, const float* x, const float* y, const float* w,
                         float* out, void* stream) {
    if (int r = check_node_problem(prob)) return r;
    const int64_t N = prob->n_nodes, C = prob->channels, D = ctp::dim_of(prob->l_x);
    const int64_t P = ctp::num_paths(prob->l_x, prob->l_y, prob->l_out);
    if (int r = need(x, N * D * C, 16, "x")) return r;
    if (int r = need(y, N * D * C, 16, "y")) return r;
    if (int r = need(w, N * P * C, 16, "w")) return r;
    if (int r = need(out, N * D * C, 16, "out")) return r;
    if (N == 0) return ok();
    return hip_status(ctp::launch_node_fwd(prob->l_x, (int)N, (int)C, x, y, w, out, static_cast<hipStream_t>(stream)),
                      "node forward launch");
}

int32_t conv_tp_node_bwd(const conv_tp_node_problem* prob, const float* grad_out, const float* x, const float* y,
                         const float* w, float* dx, float* dy, float* dw, void* stream) {
    if (int r = check_node_problem(prob)) return r;
    const int64_t N = prob->n_nodes, C = prob->channels, D = ctp::dim_of(prob->l_x);
    const int64_t P = ctp::num_paths(prob->l_x, prob->l_y, prob->l_out);
    if (int r = need(grad_out, N * D * C, 16, "grad_out")) return r;
    if (int r = need(x, N * D * C, 16, "x")) return r;
    if (int r = need(y, N * D * C, 16, "y")) return r;
    if (int r = need(w, N * P * C, 16, "w")) return r;
    if (int r = need(dx, N * D * C, 16, "dx")) return r;
    if (int r = need(dy, N * D * C, 16, "dy")) return r;
    if (int r = need(dw, N * P * C, 16, "dw")) return r;
    if (N == 0) return ok();
    return hip_status(ctp::launch_node_bwd(prob->l_x, (int)N, (int)C, grad_out, x, y, w, dx, dy, dw,
                                           static_cast<hipStream_t>(stream)),
                      "node backward launch");
}

int32_t conv_tp_stream_probe(int32_t kind, const float* src, float* dst, int64_t n_floats, void* stream) {
    if (kind < 0 || kind > 5)
        return fail(CTP_EINVAL, "kind = %d not 0..5 (read, write, copy; 3..5 the same with 4-byte accesses)", kind);
    if (n_floats < 0 || n_floats % 4 != 0) return fail(CTP_EINVAL, "n_floats = %lld must be a non-negative multiple of 4",
                                                       (long long)n_floats);
    const int base_kind = kind % 3;
    if (base_kind != 1)
        if (int r = need(src, n_floats, 16, "src")) return r;
    if (int r = need(dst, base_kind == 0 ? (n_floats > 0 ? 1 : 0) : n_floats, 16, "dst")) return r;
    if (n_floats == 0) return ok();
    return hip_status(ctp::launch_stream_probe(kind, src, dst, (long)n_floats, static_cast<hipStream_t>(stream)),
                      "stream probe launch");
}

int32_t conv_tp_valu_probe(int64_t iterations, float* dst, int64_t* fmas, void* stream) {
    if (iterations < 0) return fail(CTP_EINVAL, "iterations = %lld must be >= 0", (long long)iterations);
    if (fmas == nullptr) return fail(CTP_EINVAL, "fmas is null");
    if (int r = need(dst, 1, 4, "dst")) return r;
    *fmas = ctp::valu_probe_fmas(iterations);
    if (iterations == 0) return ok();
    return hip_status(ctp::launch_valu_probe(iterations, dst, static_cast<hipStream_t>(stream)), "valu probe launch");
}

int32_t conv_tp_check_graph(int32_t n_nodes, int32_t n_edges, const int32_t* row_ptr, const int32_t* senders,
                            int64_t* n_bad, void* stream) {
    if (n_nodes < 0 || n_edges < 0) return fail(CTP_EINVAL, "negative node or edge count");
    if (int r = need(row_ptr, (int64_t)n_nodes + 1, 4, "row_ptr")) return r;
    if (int r = need(senders, n_edges, 4, "senders")) return r;
    if (n_bad == nullptr) return fail(CTP_EINVAL, "n_bad is null");
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_status(e, "hipGetDevice");
    // one counter per device; the lock also serialises concurrent checks that share it
    std::lock_guard<std::mutex> lk(g_bad_mu);
    unsigned long long* d_bad = nullptr;
    auto it = g_bad_buf.find(dev);
    if (it == g_bad_buf.end()) {
        if (hipError_t e = hipMalloc(&d_bad, sizeof(unsigned long long)); e != hipSuccess)
            return hip_status(e, "hipMalloc(check counter)");
        g_bad_buf[dev] = d_bad;
    } else {
        d_bad = it->second;
    }
    unsigned long long h_bad = 0;
    if (hipError_t e = hipMemsetAsync(d_bad, 0, sizeof(h_bad), st); e != hipSuccess) return hip_status(e, "memset");
    if (hipError_t e = ctp::launch_check_graph(n_nodes, n_edges, row_ptr, senders, d_bad, st); e != hipSuccess)
        return hip_status(e, "conv_tp_check_graph launch");
    if (hipError_t e = hipMemcpyAsync(&h_bad, d_bad, sizeof(h_bad), hipMemcpyDeviceToHost, st); e != hipSuccess)
        return hip_status(e, "copy");
    if (hipError_t e = hipStreamSynchronize(st); e != hipSuccess) return hip_status(e, "synchronize");
    *n_bad = static_cast<int64_t>(h_bad);
    return ok();
}

}  // extern "C"
