// gemm256_mixed.hip — instantiations of the 256x256-tile GEMM for block-scaled
// operands of two different kinds among OCP E4M3, E2M3, E3M2 and padded E2M1
// (both K-major; the eight-wave 16x16 pipeline only).
#include "gemm256_kernel.hpp"

namespace mswz {
namespace {

template <int KA, int KB>
hipError_t launch_pair(const MxArgs &a, hipStream_t stream)
{
    return launch_cfg<KA, false, false, KB>(a, stream);
}

// B's kind KB for A's kind KA; one kind on both sides is not a mix (those
// plans take the single-kind kernels) and is not instantiated here
template <int KA, int KB>
hipError_t launch_if_mixed(const MxArgs &a, hipStream_t stream)
{
    if constexpr (KA == KB)
        return hipErrorInvalidValue;
    else
        return launch_pair<KA, KB>(a, stream);
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
