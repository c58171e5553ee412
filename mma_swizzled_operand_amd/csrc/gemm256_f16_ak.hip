// gemm256_f16_ak.hip — instantiations of the 256x256-tile GEMM for fp16 operands, A K-major (B either major).
#include "gemm256_kernel.hpp"

namespace mswz {

hipError_t launch256_f16_ak(bool b_mn, const MxArgs &a, hipStream_t stream)
{
    return b_mn ? launch_cfg<kF16, false, true>(a, stream) : launch_cfg<kF16, false, false>(a, stream);
}

}  // namespace mswz
