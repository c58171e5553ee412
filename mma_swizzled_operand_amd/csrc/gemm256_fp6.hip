// gemm256_fp6.hip — instantiations of the 256x256-tile GEMM for block-scaled
// padded sub-byte operands: OCP E2M3 and E3M2 (sixteen 6-bit values and four
// bytes of padding per 16-byte block) and E2M1 in the padded form (sixteen
// 4-bit values and eight bytes of padding); both K-major, the eight-wave
// 16x16 pipeline only.
#include "gemm256_kernel.hpp"

namespace mswz {
namespace {

template <int K>
hipError_t launch_padded(const MxArgs &a, hipStream_t stream)
{
    if (a.sf_mn)   // MN-major scales (K a multiple of the step): the wide loop alone, or the per-step loop
        return a.K % 2048 == 0 ? launch_out<K, false, false, -1, 32, false, true, true>(a, stream)
                               : launch_out<K, false, false, -1, 32, false, true, false>(a, stream);
    return launch_cfg<K, false, false>(a, stream);
}

}  // namespace

hipError_t launch256_padded(const MxArgs &a, MxKind kind, hipStream_t stream)
{
    switch (kind) {
    case kMxE2m3: return launch_padded<kE2m3>(a, stream);
    case kMxE3m2: return launch_padded<kE3m2>(a, stream);
    case kMxE2m1p: return launch_padded<kE2m1p>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mswz
