// gemm256_e4m3.hip — instantiations of the 256x256-tile GEMM for block-scaled
// OCP E4M3 operands (both K-major), except fp32 D with K a multiple of the K
// step (gemm256_e4m3_f32.hip, a unit compiled with another scheduling
// strategy).
#include "gemm256_kernel.hpp"

namespace mswz {

hipError_t launch256_e4m3(const MxArgs &a, hipStream_t stream)
{
    if (a.K % 128 != 0)
        return launch_out<kE4m3, false, false, -1, 32, true>(a, stream);
    switch (a.out) {
    case kOutBf16:
        if (a.sf_mn)
            return a.K % 2048 == 0 ? launch_kind<kE4m3, false, false, kOutBf16, -1, 32, false, true, true>(a, stream)
                                   : launch_kind<kE4m3, false, false, kOutBf16, -1, 32, false, true, false>(a, stream);
        return launch_kind<kE4m3, false, false, kOutBf16>(a, stream);
    case kOutF16:
        if (a.sf_mn)
            return a.K % 2048 == 0 ? launch_kind<kE4m3, false, false, kOutF16, -1, 32, false, true, true>(a, stream)
                                   : launch_kind<kE4m3, false, false, kOutF16, -1, 32, false, true, false>(a, stream);
        return launch_kind<kE4m3, false, false, kOutF16>(a, stream);
    default: return launch256_e4m3_f32(a, stream);
    }
}

}  // namespace mswz
