// gemm256.hip — run-time dispatch of the 256x256-tile GEMM (gemm256_kernel.hpp)
// to its instantiations, one translation unit per operand kind and A major
// (gemm256_bf16_ak.hip, gemm256_bf16_amn.hip, gemm256_f16_ak.hip,
// gemm256_f16_amn.hip, gemm256_e4m3.hip, gemm256_e2m1.hip, gemm256_fp6.hip,
// gemm256_mixed.hip, gemm256_v16.hip),
// so that they
// compile in parallel.
#include <hip/hip_runtime.h>
#include <stdlib.h>

#include "kernels.hpp"

namespace mswz {

// Pipeline configuration of the 256x256 tile, selected at run time by the
// environment variable MSWZ_TILE256 (tuning only): 1 = four waves (else
// eight); 4 / 8 / 12 = K-major A / B / both staged through registers;
// 16 = the ping-pong kernel for 16-bit K-major operands with K % 128 == 0;
// 32 = MN-major operands through register transposes; 64 = 16x16x32 MFMAs
// in every case; 128 = 32x32x16 MFMAs in every case.
int config256()
{
    static int cfg = [] {
        const char *e = getenv("MSWZ_TILE256");
        return e ? atoi(e) : 0;
    }();
    return cfg;
}

hipError_t launch_dense256(bool bf16, bool a_mn, bool b_mn, const DenseArgs &d, hipStream_t stream)
{
    if (config256() == 16 && !a_mn && !b_mn && d.K % 128 == 0 && d.M % 256 == 0 && d.N % 256 == 0 &&
        d.out == kOutF32 && d.lda == d.K && d.ldb == d.K && d.ldd == d.N && !d.opts.neg && !d.opts.sat &&
        !d.opts.row_mask && !d.opts.col_zero)
        return launch_dense256pp(bf16, d, stream);
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
    if (kind_b != kind)
        return launch256_mixed(a, kind, kind_b, stream);
    switch (kind) {
    case kMxE2m1: return launch256_e2m1(a, stream);
    case kMxE2m3: case kMxE3m2: case kMxE2m1p: return launch256_padded(a, kind, stream);
    default: return launch256_e4m3(a, stream);
    }
}

}  // namespace mswz
