// Kernels of one degree triple (l_in, l_sh, l_out) = (CTP_L1, CTP_L2, CTP_L3).
//
// The build compiles this file once per triple with -DCTP_L1=.. -DCTP_L2=..
// -DCTP_L3=.., so every kernel is specialised at compile time for its degrees
// and path variant (constexpr path tables, unrolled loops, coefficients as
// instruction constants) while the 64 triples build in parallel.  The
// dispatcher (convtp_common.hip) selects Triple<l_in, l_sh, l_out> at run time.
#include <hip/hip_runtime.h>

#ifndef CTP_L1
#error "compile with -DCTP_L1=<l_in> -DCTP_L2=<l_sh> -DCTP_L3=<l_out>"
#endif

#include "device_common.hpp"
#include "kernels.hpp"

namespace ctp {

using SpecSum = Spec<CTP_L1, CTP_L2, CTP_L3, kVariantSummed>;
using SpecSlot = Spec<CTP_L1, CTP_L2, CTP_L3, kVariantSlots>;

// This translation unit's device copies of the slot tables and harmonic coefficients.
static __constant__ SlotTab<SpecSum> kSlotSum = make_slot_tab<SpecSum>();
static __constant__ SlotTab<SpecSlot> kSlotSlot = make_slot_tab<SpecSlot>();
static __constant__ ShTab kShTab = make_sh_tab();

template <>
__device__ __forceinline__ const SlotDev* slot_tab<SpecSum>() { return kSlotSum.s; }
template <>
__device__ __forceinline__ const SlotDev* slot_tab<SpecSlot>() { return kSlotSlot.s; }
__device__ __forceinline__ const ShTab& sh_tab() { return kShTab; }

}  // namespace ctp

#include "conv_bwd.hpp"
#include "conv_dd.hpp"
#include "conv_dy.hpp"
#include "conv_frame.hpp"
#include "conv_fwd.hpp"

namespace ctp {

template <int L1, int L2, int L3>
hipError_t Triple<L1, L2, L3>::fwd(const LaunchArgs& a, hipStream_t st) {
    if (a.variant == kVariantSlots) return conv::fwd_launch<Spec<L1, L2, L3, kVariantSlots>>(a, st);
    return conv::fwd_launch<Spec<L1, L2, L3, kVariantSummed>>(a, st);
}

template <int L1, int L2, int L3>
hipError_t Triple<L1, L2, L3>::fwd_frame(const LaunchArgs& a, hipStream_t st) {
    return conv::frame_launch<Spec<L1, L2, L3, kVariantSummed>>(a, st);
}

template <int L1, int L2, int L3>
hipError_t Triple<L1, L2, L3>::bwd(const LaunchArgs& a, hipStream_t st) {
    if (a.variant == kVariantSlots) return conv::bwd_launch<Spec<L1, L2, L3, kVariantSlots>>(a, st);
    return conv::bwd_launch<Spec<L1, L2, L3, kVariantSummed>>(a, st);
}

template <int L1, int L2, int L3>
hipError_t Triple<L1, L2, L3>::bwd_atomic(const LaunchArgs& a, hipStream_t st) {
    if (a.variant == kVariantSlots) return conv::bwd_atomic_launch<Spec<L1, L2, L3, kVariantSlots>>(a, st);
    return conv::bwd_atomic_launch<Spec<L1, L2, L3, kVariantSummed>>(a, st);
}

template <int L1, int L2, int L3>
hipError_t Triple<L1, L2, L3>::bwd_frame(const LaunchArgs& a, hipStream_t st) {
    return conv::frame_bwd_launch<Spec<L1, L2, L3, kVariantSummed>>(a, st);
}

template <int L1, int L2, int L3>
hipError_t Triple<L1, L2, L3>::bwd_recv(const LaunchArgs& a, float* msg, hipStream_t st) {
    if (a.variant == kVariantSlots) return conv::bwd_recv_launch<Spec<L1, L2, L3, kVariantSlots>>(a, msg, st);
    return conv::bwd_recv_launch<Spec<L1, L2, L3, kVariantSummed>>(a, msg, st);
}

template <int L1, int L2, int L3>
hipError_t Triple<L1, L2, L3>::bwd_dy(const LaunchArgs& a, hipStream_t st) {
    if (a.variant == kVariantSlots) return conv::dy_launch<Spec<L1, L2, L3, kVariantSlots>>(a, st);
    return conv::dy_launch<Spec<L1, L2, L3, kVariantSummed>>(a, st);
}

template <int L1, int L2, int L3>
hipError_t Triple<L1, L2, L3>::double_bwd(const DoubleArgs& a, hipStream_t st) {
    if (a.variant == kVariantSlots) return conv::dd_launch<Spec<L1, L2, L3, kVariantSlots>>(a, st);
    return conv::dd_launch<Spec<L1, L2, L3, kVariantSummed>>(a, st);
}

template struct Triple<CTP_L1, CTP_L2, CTP_L3>;

}  // namespace ctp
