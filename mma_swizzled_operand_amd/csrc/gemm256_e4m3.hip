// gemm256_e4m3.hip — instantiations of the 256x256-tile GEMM for block-scaled
// OCP E4M3 operands (both K-major).
#include "gemm256_kernel.hpp"

namespace mswz {

hipError_t launch256_e4m3(const MxArgs &a, hipStream_t stream)
{
    return launch_cfg<kE4m3, false, false>(a, stream);
}

}  // namespace mswz
