// gemm256_e4m3_f32.hip — the 256x256-tile GEMM for block-scaled OCP E4M3
// operands with fp32 D and K a multiple of the 128-element K step: the
// kernels whose 32-byte scale groups fit the registers only under LLVM's
// iterative ILP scheduling strategy, which this unit alone is compiled with
// (_build.py); under it the other E4M3 kernels spill more, so they stay in
// gemm256_e4m3.hip.
#include "gemm256_kernel.hpp"

namespace mswz {

hipError_t launch256_e4m3_f32(const MxArgs &a, hipStream_t stream)
{
    if (a.sf_mn)   // MN-major scales: the wide loop alone, or the per-step loop alone
        return a.K % 2048 == 0 ? launch_kind<kE4m3, false, false, kOutF32, -1, 32, false, true, true>(a, stream)
                               : launch_kind<kE4m3, false, false, kOutF32, -1, 32, false, true, false>(a, stream);
    if (a.K % 2048 == 0)   // the wide loop alone (8192^3 MX-fp8 -1.9 %)
        return launch_kind<kE4m3, false, false, kOutF32, -1, 32, false, false, true>(a, stream);
    return launch_kind<kE4m3, false, false, kOutF32>(a, stream);
}

}  // namespace mswz
