// gemm256_bf16_amn_bmn.hip — instantiations of the 256x256-tile GEMM for bf16 operands, both
// MN-major (the 32x32x16 MFMA path), in a unit of their own: they run faster
// under LLVM's max-ILP scheduling strategy, the other 16-bit kernels slower.
#include "gemm256_kernel.hpp"

namespace mswz {

hipError_t launch256_bf16_amn_bmn(const MxArgs &a, hipStream_t stream)
{
    return launch_cfg<kBf16, true, true>(a, stream);
}

}  // namespace mswz
