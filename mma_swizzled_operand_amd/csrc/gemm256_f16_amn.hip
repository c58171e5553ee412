// gemm256_f16_amn.hip — instantiations of the 256x256-tile GEMM for f16 operands, A MN-major,
// B K-major; both MN-major in gemm256_f16_amn_bmn.hip (a unit compiled with
// another scheduling strategy).
#include "gemm256_kernel.hpp"

namespace mswz {

hipError_t launch256_f16_amn(bool b_mn, const MxArgs &a, hipStream_t stream)
{
    return b_mn ? launch256_f16_amn_bmn(a, stream) : launch_cfg<kF16, true, false>(a, stream);
}

}  // namespace mswz
