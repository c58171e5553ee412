// gemm256_pair.hip — instantiations of the 256x256-tile GEMM for OCP E4M3
// paired with dense (unpadded) OCP E2M1, either operand the E2M1 one (both
// K-major, 32-element scale blocks, K a multiple of 256; compute_pair in
// gemm256_kernel.hpp).
#include "gemm256_kernel.hpp"

namespace mswz {

hipError_t launch256_pair(const MxArgs &a, MxKind ka, MxKind kb, hipStream_t stream)
{
    // MN-major scales (E4M3 A only: with an E2M1 A the kernels spilled 9-33
    // registers): the per-step loop, one 1 KiB copy per operand and step
    if (ka == kMxE4m3 && kb == kMxE2m1)
        return a.sf_mn ? launch_out<kE4m3, false, false, kE2m1, 32, false, true, false>(a, stream)
                       : launch_cfg<kE4m3, false, false, kE2m1>(a, stream);
    if (ka == kMxE2m1 && kb == kMxE4m3)
        return launch_cfg<kE2m1, false, false, kE4m3>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace mswz
