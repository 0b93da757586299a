// Launch functions of the kernel side, stubbed out for the sanitizer build of
// the C ABI front (tests/test_sanitizers_cpu.py): the host validation in
// convtp_api.hip is linked against these instead of the kernels, so it can be
// built with AddressSanitizer and UndefinedBehaviorSanitizer in seconds and
// exercised without a GPU.  A stub succeeds when its call has nothing to
// launch (no nodes, edges or elements), as the kernel side does, and reports
// an error otherwise: the tests only make calls that are rejected on the host
// or that have nothing to launch.
#include <hip/hip_runtime.h>

#include "../../tensor_product_message_amd/csrc/kernels.hpp"

namespace ctp {

hipError_t launch_fwd(const LaunchArgs& a, hipStream_t) { return a.n_nodes == 0 ? hipSuccess : hipErrorNotSupported; }
hipError_t launch_bwd(const LaunchArgs& a, hipStream_t) { return a.n_nodes == 0 ? hipSuccess : hipErrorNotSupported; }
hipError_t launch_bwd_msg(const LaunchArgs& a, float*, hipStream_t) {
    return a.n_nodes == 0 ? hipSuccess : hipErrorNotSupported;
}
hipError_t launch_bwd_dy(const LaunchArgs& a, hipStream_t) {
    return a.n_nodes == 0 || a.n_edges == 0 ? hipSuccess : hipErrorNotSupported;
}
hipError_t launch_double_bwd(const DoubleArgs& a, hipStream_t) {
    return a.n_nodes == 0 ? hipSuccess : hipErrorNotSupported;
}
hipError_t launch_sh(int, long n, const float*, float*, hipStream_t) { return n == 0 ? hipSuccess : hipErrorNotSupported; }
hipError_t launch_sh_bwd(int, long n, const float*, const float*, float*, hipStream_t) {
    return n == 0 ? hipSuccess : hipErrorNotSupported;
}
hipError_t launch_sh_jvp(int, long n, const float*, const float*, float*, hipStream_t) {
    return n == 0 ? hipSuccess : hipErrorNotSupported;
}
hipError_t launch_sh_bwd_bwd(int, long n, const float*, const float*, const float*, const float*, float*,
                             hipStream_t) {
    return n == 0 ? hipSuccess : hipErrorNotSupported;
}
hipError_t launch_transpose(int, int, const int32_t*, const int32_t*, int32_t*, int32_t*, int32_t*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_node_fwd(int, int, int, const float*, const float*, const float*, float*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_node_bwd(int, int, int, const float*, const float*, const float*, const float*, float*, float*,
                           float*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_stream_probe(int, const float*, float*, long n, hipStream_t) {
    return n == 0 ? hipSuccess : hipErrorNotSupported;
}
hipError_t launch_valu_probe(long n, float*, hipStream_t) { return n == 0 ? hipSuccess : hipErrorNotSupported; }
long valu_probe_fmas(long n) { return n; }
hipError_t launch_check_graph(int, int, const int32_t*, const int32_t*, unsigned long long*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace ctp
