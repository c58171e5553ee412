// kernels.hpp — internal interface between the C ABI (abi.hip) and the gfx950
// kernel families (gemm_dense.hip, gemm_mx.hip, gemm_skinny.hip).  Not installed.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mswz {

// Kernel variants a plan can select.  The tile is BM x BN output elements per
// 256-thread workgroup; each K step stages 128 bytes of every operand row.
enum Variant : int {
    kVarDense256 = 1,   // 16-bit, 256x256 tile, 8 waves of 128x64 (gemm256_kernel.hpp)
    kVarDense128 = 2,   // 16-bit, 128x128 tile, 4 waves of 64x64
    kVarDense64 = 3,    // 16-bit, 64x64 tile, 4 waves of 32x32
    kVarMx256 = 11,     // E4M3 block-scaled, 256x256 tile, 8 waves (gemm256_kernel.hpp)
    kVarMx128 = 12,     // E4M3 block-scaled, 128x128 tile
    kVarMx64 = 13,      // E4M3 block-scaled, 64x64 tile
    kVarSkinny = 21,    // 16-bit, M <= 64: weight streaming, split K inside the workgroup
};

// Output element kind of D: fp32, or the fp32 result rounded to nearest even
// into bf16 / fp16 (beta = 1 then reads D in that kind).
enum OutKind { kOutF32 = 0, kOutBf16 = 1, kOutF16 = 2 };

// Epilogue options of the 256x256 kernel (all off by default): the product
// enters D negated; D values stored clamped to D's largest finite magnitude;
// rows of D whose bit is set in row_mask left untouched; columns whose bit is
// set in col_zero receive a zero product (bit x of word x / 32 in both).
struct EpiOpts {
    int neg = 0;
    int sat = 0;
    const uint32_t *row_mask = nullptr;
    const uint32_t *col_zero = nullptr;
};

struct DenseArgs {
    const void *A;
    const void *B;
    float *D;          // element kind given by `out`
    int M, N, K;
    int beta;
    int group_m;
    int out = kOutF32;
    // elements from one stored row to the next: A, B (K-major: >= K;
    // MN-major: >= M / N) and D (>= N)
    int lda = 0, ldb = 0, ldd = 0;
    EpiOpts opts = {};
};

struct MxArgs {
    const void *A;
    const void *B;
    const uint8_t *SFA;
    const uint8_t *SFB;
    float *D;          // element kind given by `out`
    int M, N, K;
    int beta;
    int group_m;
    int out = kOutF32;
    int lda = 0, ldb = 0, ldd = 0;   // as in DenseArgs (scale arrays are packed)
    EpiOpts opts = {};
    int sv = 32;                     // K elements per scale byte (32, or 16)
    int sf_mn = 0;                   // scales stored [K/sv][M] and [K/sv][N] (wide-stage kernels only)
};

struct VariantInfo {
    int tile_m, tile_n, tile_k, threads, lds_bytes;
};

bool variant_info(int variant, bool one_byte_elems, VariantInfo *info);

hipError_t launch_dense(int variant, bool bf16, bool a_mn, bool b_mn, const DenseArgs &args,
                        hipStream_t stream);
hipError_t launch_dense256(bool bf16, bool a_mn, bool b_mn, const DenseArgs &args, hipStream_t stream);
// block-scaled element kinds of the 256x256 tile
enum MxKind { kMxE4m3 = 0, kMxE2m1 = 1, kMxE2m3 = 2, kMxE3m2 = 3, kMxE2m1p = 4 };
hipError_t launch_mx256(const MxArgs &args, MxKind kind_a, MxKind kind_b, hipStream_t stream);
// the 256x256-tile instantiations, one translation unit each (gemm256_*.hip)
hipError_t launch256_bf16_ak(bool b_mn, const MxArgs &args, hipStream_t stream);
hipError_t launch256_bf16_amn(bool b_mn, const MxArgs &args, hipStream_t stream);
hipError_t launch256_bf16_amn_bmn(const MxArgs &args, hipStream_t stream);   // both MN-major
hipError_t launch256_f16_ak(bool b_mn, const MxArgs &args, hipStream_t stream);
hipError_t launch256_f16_amn(bool b_mn, const MxArgs &args, hipStream_t stream);
hipError_t launch256_f16_amn_bmn(const MxArgs &args, hipStream_t stream);   // both MN-major
hipError_t launch256_e4m3(const MxArgs &args, hipStream_t stream);
// fp32 D, K a multiple of 128 (gemm256_e4m3_f32.hip)
hipError_t launch256_e4m3_f32(const MxArgs &args, hipStream_t stream);
hipError_t launch256_e2m1(const MxArgs &args, hipStream_t stream);
hipError_t launch256_padded(const MxArgs &args, MxKind kind, hipStream_t stream);
hipError_t launch256_mixed(const MxArgs &args, MxKind kind_a, MxKind kind_b, hipStream_t stream);
// E4M3 A, fp32 D, K a multiple of 128 (gemm256_mixed_e4m3_f32.hip)
hipError_t launch256_mixed_e4m3_f32(const MxArgs &args, MxKind kind_b, hipStream_t stream);
// E4M3 with dense E2M1 (either side), K % 256 == 0
hipError_t launch256_pair(const MxArgs &args, MxKind kind_a, MxKind kind_b, hipStream_t stream);
hipError_t launch256_v16(const MxArgs &args, MxKind kind, hipStream_t stream);
hipError_t launch_mx(int variant, const MxArgs &args, hipStream_t stream);
hipError_t launch_skinny(bool bf16, const DenseArgs &args, hipStream_t stream);

// Weight streaming with K split over workgroups (gemm_skinny_sk.hip): the
// number of K parts for an (M, N, K) problem (0 when the split kernel does not
// apply), the workspace it needs, and the launch on a caller's workspace.
struct SplitK {
    int parts;
    float *partials;      // parts x M x N fp32
};
int skinny_split_parts(int64_t M, int64_t N, int64_t K);
int64_t skinny_split_workspace_bytes(int64_t M, int64_t N, int parts);
hipError_t launch_skinny_split(bool bf16, const DenseArgs &args, void *workspace, hipStream_t stream);

}  // namespace mswz
