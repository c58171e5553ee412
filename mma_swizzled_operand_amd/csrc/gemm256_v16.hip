// gemm256_v16.hip — instantiations of the 256x256-tile GEMM with 16-element
// scale blocks (one E8M0 scale per 16 K elements) for OCP E2M1 (dense or
// padded), E2M3 and E3M2 operands (both K-major, the same kind; the eight-wave
// 16x16 pipeline only).
#include "gemm256_kernel.hpp"

namespace mswz {
namespace {

template <int K>
hipError_t launch16(const MxArgs &a, hipStream_t stream)
{
    return launch_cfg<K, false, false, -1, 16>(a, stream);
}

}  // namespace

hipError_t launch256_v16(const MxArgs &a, MxKind kind, hipStream_t stream)
{
    switch (kind) {
    case kMxE2m1: return launch16<kE2m1>(a, stream);
    case kMxE2m1p: return launch16<kE2m1p>(a, stream);
    case kMxE2m3: return launch16<kE2m3>(a, stream);
    case kMxE3m2: return launch16<kE3m2>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mswz
