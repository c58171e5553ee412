// gemm256.hip — run-time dispatch of the 256x256-tile GEMM (gemm256_kernel.hpp)
// to its instantiations, one translation unit per operand kind and A major
// (gemm256_bf16_ak.hip, gemm256_bf16_amn.hip, gemm256_f16_ak.hip,
// gemm256_f16_amn.hip, gemm256_f16_amn_bmn.hip, gemm256_e4m3.hip, gemm256_e4m3_f32.hip, gemm256_e2m1.hip, gemm256_fp6.hip,
// gemm256_mixed.hip, gemm256_mixed_e4m3_f32.hip, gemm256_pair.hip, gemm256_v16.hip),
// so that they
// compile in parallel.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace mswz {

hipError_t launch_dense256(bool bf16, bool a_mn, bool b_mn, const DenseArgs &d, hipStream_t stream)
{
    const MxArgs a{d.A, d.B, nullptr, nullptr, d.D, d.M, d.N, d.K, d.beta, d.group_m, d.out,
                   d.lda, d.ldb, d.ldd, d.opts};
    if (bf16)
        return a_mn ? launch256_bf16_amn(b_mn, a, stream) : launch256_bf16_ak(b_mn, a, stream);
    return a_mn ? launch256_f16_amn(b_mn, a, stream) : launch256_f16_ak(b_mn, a, stream);
}

hipError_t launch_mx256(const MxArgs &a, MxKind kind, MxKind kind_b, hipStream_t stream)
{
    if (a.sv == 16)
        return kind_b == kind ? launch256_v16(a, kind, stream) : hipErrorInvalidValue;
    if (kind_b != kind) {
        if (kind == kMxE2m1 || kind_b == kMxE2m1)
            return launch256_pair(a, kind, kind_b, stream);
        return launch256_mixed(a, kind, kind_b, stream);
    }
    switch (kind) {
    case kMxE2m1: return launch256_e2m1(a, stream);
    case kMxE2m3: case kMxE3m2: case kMxE2m1p: return launch256_padded(a, kind, stream);
    default: return launch256_e4m3(a, stream);
    }
}

}  // namespace mswz
