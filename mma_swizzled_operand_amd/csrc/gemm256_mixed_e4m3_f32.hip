// gemm256_mixed_e4m3_f32.hip — the 256x256-tile GEMM for E4M3 A with a
// 6-bit or padded 4-bit B (block-scaled, both K-major), fp32 D and K a
// multiple of the 128-element K step: kernels whose 32-byte scale groups fit
// the registers only under LLVM's iterative ILP scheduling strategy, which
// this unit is compiled with (_build.py); the other mixed kernels spill more
// under it and stay in gemm256_mixed.hip.
#include "gemm256_kernel.hpp"

namespace mswz {

namespace {

// scales row-major or MN-major (sf_mn); with a padded E2M1 B and K a
// multiple of 2048 the kernel with the wide loop alone
template <int KB>
hipError_t launch_b(const MxArgs &a, hipStream_t stream)
{
    if (a.sf_mn)   // MN-major scales: the wide loop alone, or the per-step loop alone
        return a.K % 2048 == 0 ? launch_kind<kE4m3, false, false, kOutF32, KB, 32, false, true, true>(a, stream)
                               : launch_kind<kE4m3, false, false, kOutF32, KB, 32, false, true, false>(a, stream);
    if constexpr (KB == kE2m1p) {
        if (a.K % 2048 == 0)   // the wide loop alone (8192^3 -3.2 %; with a 6-bit B 0.6 % slower)
            return launch_kind<kE4m3, false, false, kOutF32, KB, 32, false, false, true>(a, stream);
    }
    return launch_kind<kE4m3, false, false, kOutF32, KB>(a, stream);
}

}  // namespace

hipError_t launch256_mixed_e4m3_f32(const MxArgs &a, MxKind kb, hipStream_t stream)
{
    switch (kb) {
    case kMxE2m3: return launch_b<kE2m3>(a, stream);
    case kMxE3m2: return launch_b<kE3m2>(a, stream);
    case kMxE2m1p: return launch_b<kE2m1p>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mswz
