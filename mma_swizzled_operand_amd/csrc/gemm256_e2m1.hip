// gemm256_e2m1.hip — instantiations of the 256x256-tile GEMM for block-scaled
// OCP E2M1 (FP4) operands (both K-major).
#include "gemm256_kernel.hpp"

namespace mswz {

hipError_t launch256_e2m1(const MxArgs &a, hipStream_t stream)
{
    if (a.sf_mn)   // MN-major scales (K a multiple of the step): the wide loop alone, or the per-step loop
        return a.K % 2048 == 0 ? launch_out<kE2m1, false, false, -1, 32, false, true, true>(a, stream)
                               : launch_out<kE2m1, false, false, -1, 32, false, true, false>(a, stream);
    return launch_cfg<kE2m1, false, false>(a, stream);
}

}  // namespace mswz
