// gemm256_mixed.hip — instantiations of the 256x256-tile GEMM for block-scaled
// operands of two different kinds among OCP E4M3, E2M3, E3M2 and padded E2M1
// (both K-major; the eight-wave 16x16 pipeline only), except E4M3 A with fp32
// D and K a multiple of the K step (gemm256_mixed_e4m3_f32.hip).
#include "gemm256_kernel.hpp"

namespace mswz {
namespace {

template <int KA, int KB>
hipError_t launch_pair(const MxArgs &a, hipStream_t stream)
{
    // MN-major scales: the per-step loop for every K (with the wide loop
    // alone an fp32 D spilled 28-44 registers; the per-step kernels none)
    if (a.sf_mn)
        return launch_out<KA, false, false, KB, 32, false, true, false>(a, stream);
    return launch_cfg<KA, false, false, KB>(a, stream);
}

// E4M3 A with a bf16 / fp16 D and MN-major scales: the wide loop alone for K
// a multiple of 2048, else the per-step loop
template <int KB, int OUT>
hipError_t launch_e4m3_mn(const MxArgs &a, hipStream_t stream)
{
    return a.K % 2048 == 0 ? launch_kind<kE4m3, false, false, OUT, KB, 32, false, true, true>(a, stream)
                           : launch_kind<kE4m3, false, false, OUT, KB, 32, false, true, false>(a, stream);
}

// B's kind KB for A's kind KA; one kind on both sides is not a mix (those
// plans take the single-kind kernels) and is not instantiated here.  E4M3 A
// with fp32 D and K a multiple of the K step goes to
// gemm256_mixed_e4m3_f32.hip (compiled with another scheduling strategy).
template <int KA, int KB>
hipError_t launch_if_mixed(const MxArgs &a, hipStream_t stream)
{
    if constexpr (KA == KB) {
        return hipErrorInvalidValue;
    } else if constexpr (KA == kE4m3) {
        if (a.K % 128 != 0)
            return launch_out<KA, false, false, KB, 32, true>(a, stream);
        switch (a.out) {
        case kOutBf16:
            return a.sf_mn ? launch_e4m3_mn<KB, kOutBf16>(a, stream) : launch_kind<KA, false, false, kOutBf16, KB>(a, stream);
        case kOutF16:
            return a.sf_mn ? launch_e4m3_mn<KB, kOutF16>(a, stream) : launch_kind<KA, false, false, kOutF16, KB>(a, stream);
        default:
            return launch256_mixed_e4m3_f32(a, KB == kE2m3 ? kMxE2m3 : KB == kE3m2 ? kMxE3m2 : kMxE2m1p, stream);
        }
    } else {
        return launch_pair<KA, KB>(a, stream);
    }
}

template <int KA>
hipError_t launch_b(const MxArgs &a, MxKind kb, hipStream_t stream)
{
    switch (kb) {
    case kMxE4m3: return launch_if_mixed<KA, kE4m3>(a, stream);
    case kMxE2m3: return launch_if_mixed<KA, kE2m3>(a, stream);
    case kMxE3m2: return launch_if_mixed<KA, kE3m2>(a, stream);
    case kMxE2m1p: return launch_if_mixed<KA, kE2m1p>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch256_mixed(const MxArgs &a, MxKind ka, MxKind kb, hipStream_t stream)
{
    switch (ka) {
    case kMxE4m3: return launch_b<kE4m3>(a, kb, stream);
    case kMxE2m3: return launch_b<kE2m3>(a, kb, stream);
    case kMxE3m2: return launch_b<kE3m2>(a, kb, stream);
    case kMxE2m1p: return launch_b<kE2m1p>(a, kb, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mswz
