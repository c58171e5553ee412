// gemm256_fp6.hip — instantiations of the 256x256-tile GEMM for block-scaled
// 6-bit operands, OCP E2M3 and E3M2 in the padded sixteen-per-16-byte form
// (both K-major; the eight-wave 16x16 pipeline only).
#include "gemm256_kernel.hpp"

namespace mswz {

hipError_t launch256_fp6(const MxArgs &a, bool e3m2, hipStream_t stream)
{
    if (e3m2)
        return a.out == kOutF32 ? launch_kind<kE3m2, false, false, 8, 8>(a, stream)
                                : launch_out<kE3m2, false, false>(a, stream);
    return a.out == kOutF32 ? launch_kind<kE2m3, false, false, 8, 8>(a, stream)
                            : launch_out<kE2m3, false, false>(a, stream);
}

}  // namespace mswz
