// gemm256_mixed.hip — instantiations of the 256x256-tile GEMM for block-scaled
// operands of two different kinds among OCP E4M3, E2M3 and E3M2 (both
// K-major; the eight-wave 16x16 pipeline only).
#include "gemm256_kernel.hpp"

namespace mswz {
namespace {

template <int KA, int KB>
hipError_t launch_pair(const MxArgs &a, hipStream_t stream)
{
    return a.out == kOutF32 ? launch_kind<KA, false, false, 8, 8, kOutF32, KB>(a, stream)
                            : launch_out<KA, false, false, KB>(a, stream);
}

}  // namespace

hipError_t launch256_mixed(const MxArgs &a, MxKind ka, MxKind kb, hipStream_t stream)
{
    if (ka == kMxE4m3 && kb == kMxE2m3) return launch_pair<kE4m3, kE2m3>(a, stream);
    if (ka == kMxE4m3 && kb == kMxE3m2) return launch_pair<kE4m3, kE3m2>(a, stream);
    if (ka == kMxE2m3 && kb == kMxE4m3) return launch_pair<kE2m3, kE4m3>(a, stream);
    if (ka == kMxE3m2 && kb == kMxE4m3) return launch_pair<kE3m2, kE4m3>(a, stream);
    if (ka == kMxE2m3 && kb == kMxE3m2) return launch_pair<kE2m3, kE3m2>(a, stream);
    if (ka == kMxE3m2 && kb == kMxE2m3) return launch_pair<kE3m2, kE2m3>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace mswz
