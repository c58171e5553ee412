// abi.hip — the C ABI of libmswz.so (declared in include/mswz_gemm.h):
// plan creation and validation, argument checks, and kernel dispatch.
//
// The checks follow the pages' contract style: layouts and shapes are checked
// against explicit arguments, nothing is inferred, and whatever the library
// cannot run is rejected with a status before any GPU work (tcgen05.mma page,
// "Shared descriptors are byte-stride contracts"; ldmatrix / stmatrix page,
// "Transpose and stores": misaligned rows and partial participation are
// rejected).  Pointers must be 16-byte aligned, the pages' origin and row rule.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <stdlib.h>

#include <new>

#include "../../include/mswz_gemm.h"
#include "device_common.hpp"
#include "kernels.hpp"
#include "layout.hpp"

struct gemm_plan {
    int64_t M, N, K;
    int a_dt, b_dt, d_dt, a_major, b_major;
    int32_t scale_vec_len;
    int variant;
    int group_m;
    mswz::VariantInfo info;
    int64_t blocks;
    int split_parts;        // K parts of the split weight-streaming kernel (0: none)
    int64_t ws_bytes;       // workspace gemm_run_ws needs for it
    int64_t lda, ldb, ldd;  // row pitches in elements (packed values when none were given)
    int sf_major;           // MSWZ_MAJOR_K: SFA [M][K/V]; MSWZ_MAJOR_MN: SFA [K/V][M] (gemm_plan_set_scale_major)
    int variant_k;          // the variant chosen at creation, for row-major scales
};

namespace mswz {

bool variant_info(int variant, bool one_byte_elems, VariantInfo *info)
{
    const int tk = one_byte_elems ? 128 : 64;
    int t = 0;
    switch (variant) {
    case kVarDense256: case kVarMx256: t = 256; break;
    case kVarDense128: case kVarMx128: t = 128; break;
    case kVarDense64: case kVarMx64: t = 64; break;
    case kVarSkinny:
        info->tile_m = 64;
        info->tile_n = 64;
        info->tile_k = 64;
        info->threads = 512;
        info->lds_bytes = 8 * 64 * 68 * 4;
        return true;
    default: return false;
    }
    info->tile_m = t;
    info->tile_n = t;
    info->tile_k = tk;
    info->threads = t == 256 ? 512 : 256;
    info->lds_bytes = 2 * (t + t) * 128;
    return true;
}

}  // namespace mswz

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 20;

bool is_aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mswz::MxKind mx_kind(int dt)
{
    return dt == MSWZ_DT_E2M1 ? mswz::kMxE2m1 : dt == MSWZ_DT_E2M3 ? mswz::kMxE2m3
                                              : dt == MSWZ_DT_E3M2 ? mswz::kMxE3m2
                                              : dt == MSWZ_DT_E2M1_P64 ? mswz::kMxE2m1p : mswz::kMxE4m3;
}

int out_kind(int d_dt)
{
    return d_dt == MSWZ_DT_BF16 ? mswz::kOutBf16 : d_dt == MSWZ_DT_F16 ? mswz::kOutF16 : mswz::kOutF32;
}

// Whether the 256x256 kernel for these kinds stages 32 bytes of scales per
// row (the kernels' kWideStage): 32-element blocks, K a multiple of the K
// step, and one padded 6- or 4-bit kind or dense E2M1 on both sides, or an
// E4M3 A (with B E4M3 or a padded kind) and fp32 D.
bool wide_scale_stage(int a_dt, int b_dt, int d_dt, int32_t v, int64_t K)
{
    auto padded = [](int d) { return d == MSWZ_DT_E2M3 || d == MSWZ_DT_E3M2 || d == MSWZ_DT_E2M1_P64; };
    if (v != 32 || K % (a_dt == MSWZ_DT_E2M1 ? 256 : 128) != 0)
        return false;
    if (a_dt == b_dt && (padded(a_dt) || a_dt == MSWZ_DT_E2M1))
        return true;
    return a_dt == MSWZ_DT_E4M3 && (b_dt == MSWZ_DT_E4M3 || padded(b_dt)) && d_dt == MSWZ_DT_F32;
}

// Whether the 256x256 kernels take MN-major scales for these kinds (their
// one-loop MN-major kernels all have the 32-byte stage): 32-element blocks,
// K a multiple of the K step, dense E2M1 on both sides, any of E4M3, E2M3,
// E3M2 and padded E2M1 on either side, or E4M3 A with dense E2M1 B (K a
// multiple of 256), any D.
bool mn_scales(int a_dt, int b_dt, int d_dt, int32_t v, int64_t K)
{
    auto byte_row = [](int d) {
        return d == MSWZ_DT_E4M3 || d == MSWZ_DT_E2M3 || d == MSWZ_DT_E3M2 || d == MSWZ_DT_E2M1_P64;
    };
    (void)d_dt;
    const bool pair = a_dt == MSWZ_DT_E4M3 && b_dt == MSWZ_DT_E2M1;   // (not E2M1 A with E4M3 B)
    if (v != 32 || K % (a_dt == MSWZ_DT_E2M1 || pair ? 256 : 128) != 0)
        return false;
    return (a_dt == MSWZ_DT_E2M1 && b_dt == MSWZ_DT_E2M1) || (byte_row(a_dt) && byte_row(b_dt)) || pair;
}

// Choose the tile for an (M, N) output: the largest square tile dividing both
// sizes, dropping to a smaller one while the grid would leave most compute
// units idle (fewer than 128 tiles of 256 or 256 tiles of 128).  The
// environment variable MSWZ_TILE (64, 128 or 256) overrides the choice when
// that tile divides both sizes; it exists for tuning and tests.
int pick_tile(int64_t M, int64_t N)
{
    if (const char *env = getenv("MSWZ_TILE")) {
        const int t = atoi(env);
        if ((t == 64 || t == 128 || t == 256) && M % t == 0 && N % t == 0)
            return t;
    }
    auto tiles = [&](int t) { return (M / t) * (N / t); };
    if (M % 256 == 0 && N % 256 == 0 && tiles(256) >= 128)
        return 256;
    if (M % 128 == 0 && N % 128 == 0 && (tiles(128) >= 128 || M % 64 || N % 64))
        return 128;
    if (M % 64 == 0 && N % 64 == 0)
        return 64;
    return 0;
}

}  // namespace

extern "C" {

int gemm_plan_create(gemm_plan **out, int64_t M, int64_t N, int64_t K, int a_dt, int b_dt,
                     int d_dt, int a_major, int b_major, int32_t scale_vec_len)
{
    return gemm_plan_create_ld(out, M, N, K, a_dt, b_dt, d_dt, a_major, b_major, scale_vec_len, 0, 0, 0);
}

int gemm_plan_create_ld(gemm_plan **out, int64_t M, int64_t N, int64_t K, int a_dt, int b_dt,
                        int d_dt, int a_major, int b_major, int32_t scale_vec_len, int64_t lda,
                        int64_t ldb, int64_t ldd)
{
    if (!out)
        return MSWZ_ERR_INVALID;
    *out = nullptr;
    if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return MSWZ_ERR_INVALID;
    auto known_dt = [](int d) { return d >= MSWZ_DT_F16 && d <= MSWZ_DT_E2M1_P64; };
    if (!known_dt(a_dt) || !known_dt(b_dt) || !known_dt(d_dt))
        return MSWZ_ERR_INVALID;
    if ((a_major != MSWZ_MAJOR_K && a_major != MSWZ_MAJOR_MN) ||
        (b_major != MSWZ_MAJOR_K && b_major != MSWZ_MAJOR_MN))
        return MSWZ_ERR_INVALID;
    if (scale_vec_len < 0)
        return MSWZ_ERR_INVALID;
    // A and B share a kind, except that E4M3, E2M3, E3M2 and padded E2M1 mix
    // freely, and E4M3 pairs with dense E2M1
    auto byte_mx = [](int d) {
        return d == MSWZ_DT_E4M3 || d == MSWZ_DT_E2M3 || d == MSWZ_DT_E3M2 || d == MSWZ_DT_E2M1_P64;
    };
    const bool pair = (a_dt == MSWZ_DT_E4M3 && b_dt == MSWZ_DT_E2M1) || (a_dt == MSWZ_DT_E2M1 && b_dt == MSWZ_DT_E4M3);
    if ((a_dt != b_dt && !(byte_mx(a_dt) && byte_mx(b_dt)) && !pair) || a_dt == MSWZ_DT_F32)
        return MSWZ_ERR_UNSUPPORTED;
    const bool mixed = a_dt != b_dt;
    // D: fp32, or the fp32 result rounded to bf16 / fp16 (the 256 tile only)
    if (d_dt != MSWZ_DT_F32 && d_dt != MSWZ_DT_BF16 && d_dt != MSWZ_DT_F16)
        return MSWZ_ERR_UNSUPPORTED;
    const bool narrow_d = d_dt != MSWZ_DT_F32;
    const bool fp4 = a_dt == MSWZ_DT_E2M1 && !pair, any_fp4 = a_dt == MSWZ_DT_E2M1 || b_dt == MSWZ_DT_E2M1;
    // padded sub-byte kinds (sixteen values per 16-byte block)
    const bool fp6 = a_dt == MSWZ_DT_E2M3 || a_dt == MSWZ_DT_E3M2 || a_dt == MSWZ_DT_E2M1_P64;
    const bool fp8 = a_dt == MSWZ_DT_E4M3 || a_dt == MSWZ_DT_E2M1 || fp6;   // block-scaled formats
    if (fp8 != (scale_vec_len != 0))
        return MSWZ_ERR_UNSUPPORTED;     // 8-, 6- and 4-bit kinds are block-scaled only; 16-bit is dense only
    // 32 K elements per scale byte; 16 (the pages' scale_vec::4X for 4-bit
    // operands) for E2M1 and the padded kinds, A and B of one kind
    if (fp8 && scale_vec_len != 32 &&
        !(scale_vec_len == 16 && (fp4 || fp6) && a_dt == b_dt))
        return MSWZ_ERR_UNSUPPORTED;
    if (fp8 && (a_major != MSWZ_MAJOR_K || b_major != MSWZ_MAJOR_K))
        return MSWZ_ERR_UNSUPPORTED;     // MN-major operands are built for 16-bit formats
    // block-scaled: any K that is a multiple of the scale block and keeps
    // stored rows 16-byte aligned (E2M1: K % 32 == 0, two elements a byte);
    // a K that is not a multiple of the K step (128, E2M1 256) takes the
    // 256x256 tile with a zero-padded last step and scale words assembled in
    // registers.  16-bit: any K whose K-major rows keep 16-byte alignment
    // (K % 8 == 0 unless both operands are MN-major); a K that is not a
    // multiple of 64 takes the 256x256 tile with a zero-padded last step.
    if (fp8 && (K % scale_vec_len != 0 || (any_fp4 && K % 32 != 0)))
        return MSWZ_ERR_UNSUPPORTED;
    // E4M3 with dense E2M1: the E2M1 operand's 128-byte rows hold two K steps
    // of the E4M3 one, staged together
    if (pair && K % 256 != 0)
        return MSWZ_ERR_UNSUPPORTED;
    const bool ktail = fp8 ? K % (fp4 ? 256 : 128) != 0 : K % 64 != 0;
    if (ktail && K % 8 != 0 && (a_major == MSWZ_MAJOR_K || b_major == MSWZ_MAJOR_K))
        return MSWZ_ERR_UNSUPPORTED;
    // M or N not a multiple of 64: the 256x256 tile with masked stores; D rows
    // (and MN-major operand rows) must keep 16-byte alignment
    const bool tail = M % 64 != 0 || N % 64 != 0;
    if (tail && (N % 4 != 0 || (a_major == MSWZ_MAJOR_MN && M % 8 != 0) ||
                 (b_major == MSWZ_MAJOR_MN && N % 8 != 0)))
        return MSWZ_ERR_UNSUPPORTED;
    // row pitches (0: packed).  A stored row of A or B must start 16 bytes
    // aligned (the copies move 16-byte chunks), a row of D on a 4-element
    // boundary (D is written four elements per store).
    if (lda < 0 || ldb < 0 || ldd < 0)
        return MSWZ_ERR_INVALID;
    const int64_t a_cols = a_major == MSWZ_MAJOR_MN ? M : K, b_cols = b_major == MSWZ_MAJOR_MN ? N : K;
    const int64_t lda_v = lda ? lda : a_cols, ldb_v = ldb ? ldb : b_cols, ldd_v = ldd ? ldd : N;
    if (lda_v < a_cols || ldb_v < b_cols || ldd_v < N)
        return MSWZ_ERR_INVALID;
    constexpr int64_t kMaxLd = int64_t(1) << 22;
    if (lda_v > kMaxLd || ldb_v > kMaxLd || ldd_v > kMaxLd)
        return MSWZ_ERR_UNSUPPORTED;
    auto align_elems = [&](int dt) { return dt == MSWZ_DT_E2M1 ? 32 : fp8 ? 16 : 8; };   // elements in 16 bytes
    const bool strided = lda_v != a_cols || ldb_v != b_cols || ldd_v != N;
    if (strided && (lda_v % align_elems(a_dt) || ldb_v % align_elems(b_dt) || ldd_v % 4))
        return MSWZ_ERR_UNSUPPORTED;
    // MN-major operands are addressed with 32-bit offsets from the start of
    // the [K][M] / [K][N] array
    // (256 bytes short of 4 GiB: a masked copy points at the range's end,
    // which must not wrap around)
    constexpr int64_t kMaxMnBytes = (int64_t(1) << 32) - 256;
    if ((a_major == MSWZ_MAJOR_MN && ((K - 1) * lda_v + M) * 2 >= kMaxMnBytes) ||
        (b_major == MSWZ_MAJOR_MN && ((K - 1) * ldb_v + N) * 2 >= kMaxMnBytes))
        return MSWZ_ERR_UNSUPPORTED;
    // weight streaming: few rows of K-major 16-bit A against a large B
    const bool skinny = !fp8 && !narrow_d && !strided && a_major == MSWZ_MAJOR_K &&
                        b_major == MSWZ_MAJOR_K && M <= 64 && N % 64 == 0 &&
                        K % 1024 == 0 && !getenv("MSWZ_TILE");
    const int tile = skinny ? 64 : (tail || ktail || fp4 || fp6 || mixed || narrow_d || strided) ? 256 : pick_tile(M, N);
    if (!tile)
        return MSWZ_ERR_UNSUPPORTED;

    gemm_plan *p = new (std::nothrow) gemm_plan{};
    if (!p)
        return MSWZ_ERR_INVALID;
    p->M = M;
    p->N = N;
    p->K = K;
    p->a_dt = a_dt;
    p->b_dt = b_dt;
    p->d_dt = d_dt;
    p->a_major = a_major;
    p->b_major = b_major;
    p->scale_vec_len = scale_vec_len;
    p->lda = lda_v;
    p->ldb = ldb_v;
    p->ldd = ldd_v;
    if (fp8)
        p->variant = tile == 256 ? mswz::kVarMx256 : tile == 128 ? mswz::kVarMx128 : mswz::kVarMx64;
    else if (skinny)
        p->variant = mswz::kVarSkinny;
    else
        p->variant = tile == 256 ? mswz::kVarDense256 : tile == 128 ? mswz::kVarDense128
                                                                     : mswz::kVarDense64;
    p->group_m = -4;   // 2-D XCD regions, groups of 4 tile rows (device_common.hpp)
    mswz::variant_info(p->variant, fp8, &p->info);
    if (fp4)
        p->info.tile_k = 256;                              // K elements per 128-byte row step
    if (p->variant == mswz::kVarMx256)   // the two scale stages: 32 bytes per row where the kernel has the wide ones
        p->info.lds_bytes += 2 * 512 * (wide_scale_stage(a_dt, b_dt, d_dt, scale_vec_len, K) ? 32 : 16);
    if (skinny) {
        p->info.tile_m = M > 32 ? 64 : 32;   // M padded to 32 or 64 rows
        p->info.lds_bytes = 8 * p->info.tile_m * 68 * 4;
    }
    p->blocks = ((M + p->info.tile_m - 1) / p->info.tile_m) * ((N + p->info.tile_n - 1) / p->info.tile_n);
    p->sf_major = MSWZ_MAJOR_K;
    p->variant_k = p->variant;
    if (skinny) {
        p->split_parts = mswz::skinny_split_parts(M, N, K);
        p->ws_bytes = p->split_parts ? mswz::skinny_split_workspace_bytes(M, N, p->split_parts) : 0;
    }
    *out = p;
    return MSWZ_OK;
}

int64_t gemm_plan_workspace_size(const gemm_plan *p)
{
    return p ? p->ws_bytes : int64_t(MSWZ_ERR_INVALID);
}

int gemm_plan_set_scale_major(gemm_plan *p, int sf_major)
{
    if (!p || (sf_major != MSWZ_MAJOR_K && sf_major != MSWZ_MAJOR_MN))
        return MSWZ_ERR_INVALID;
    if (p->scale_vec_len == 0)
        return MSWZ_ERR_KIND;
    int variant = p->variant_k;
    if (sf_major == MSWZ_MAJOR_MN) {
        // the kinds with the wide scale stage (K a multiple of the K step),
        // whole 16-byte chunks of 16 rows (M, N % 16), and the [K/V][M] and
        // [K/V][N] arrays below 2^31 bytes (32-bit offsets; the kernels'
        // unused copies point at 2^31, outside every array's range)
        const int64_t kb = p->K / p->scale_vec_len;
        if (!mn_scales(p->a_dt, p->b_dt, p->d_dt, p->scale_vec_len, p->K) ||
            p->M % 16 != 0 || p->N % 16 != 0 || kb * p->M > (int64_t(1) << 31) ||
            kb * p->N > (int64_t(1) << 31))
            return MSWZ_ERR_UNSUPPORTED;
        variant = mswz::kVarMx256;
    }
    p->variant = variant;
    mswz::variant_info(variant, true, &p->info);
    if (p->a_dt == MSWZ_DT_E2M1)
        p->info.tile_k = 256;
    if (variant == mswz::kVarMx256)   // MN-major scales always take the 32-byte stages
        p->info.lds_bytes += 2 * 512 * (sf_major == MSWZ_MAJOR_MN ||
                                                wide_scale_stage(p->a_dt, p->b_dt, p->d_dt, p->scale_vec_len, p->K)
                                            ? 32 : 16);
    p->blocks = ((p->M + p->info.tile_m - 1) / p->info.tile_m) * ((p->N + p->info.tile_n - 1) / p->info.tile_n);
    p->sf_major = sf_major;
    return MSWZ_OK;
}

int gemm_run(const gemm_plan *p, const void *A, const void *B, void *D, int beta, void *stream)
{
    if (!p || !A || !B || !D)
        return MSWZ_ERR_INVALID;
    if (p->scale_vec_len != 0)
        return MSWZ_ERR_KIND;
    if (beta != 0 && beta != 1)
        return MSWZ_ERR_INVALID;
    if (!is_aligned16(A) || !is_aligned16(B) || !is_aligned16(D))
        return MSWZ_ERR_ALIGN;
    mswz::DenseArgs a{A, B, static_cast<float *>(D), int(p->M), int(p->N), int(p->K), beta,
                      p->group_m, out_kind(p->d_dt), int(p->lda), int(p->ldb), int(p->ldd)};
    const bool bf16 = p->a_dt == MSWZ_DT_BF16, a_mn = p->a_major == MSWZ_MAJOR_MN,
               b_mn = p->b_major == MSWZ_MAJOR_MN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = p->variant == mswz::kVarDense256 ? mswz::launch_dense256(bf16, a_mn, b_mn, a, st)
                   : p->variant == mswz::kVarSkinny  ? mswz::launch_skinny(bf16, a, st)
                                                     : mswz::launch_dense(p->variant, bf16, a_mn, b_mn, a, st);
    return e == hipSuccess ? MSWZ_OK : MSWZ_ERR_HIP;
}

int gemm_run_ws(const gemm_plan *p, const void *A, const void *B, void *D, int beta, void *workspace,
                int64_t workspace_bytes, void *stream)
{
    if (!p || p->ws_bytes == 0)
        return gemm_run(p, A, B, D, beta, stream);
    if (!A || !B || !D || !workspace || workspace_bytes < p->ws_bytes)
        return MSWZ_ERR_INVALID;
    if (beta != 0 && beta != 1)
        return MSWZ_ERR_INVALID;
    if (!is_aligned16(A) || !is_aligned16(B) || !is_aligned16(D) || !is_aligned16(workspace))
        return MSWZ_ERR_ALIGN;
    mswz::DenseArgs a{A, B, static_cast<float *>(D), int(p->M), int(p->N), int(p->K), beta,
                      p->group_m, mswz::kOutF32, int(p->lda), int(p->ldb), int(p->ldd)};
    const hipError_t e = mswz::launch_skinny_split(p->a_dt == MSWZ_DT_BF16, a, workspace,
                                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MSWZ_OK : MSWZ_ERR_HIP;
}

int gemm_run_blockscaled(const gemm_plan *p, const void *A, const void *B, const uint8_t *SFA,
                         const uint8_t *SFB, void *D, int beta, void *stream)
{
    if (!p || !A || !B || !SFA || !SFB || !D)
        return MSWZ_ERR_INVALID;
    if (p->scale_vec_len == 0)
        return MSWZ_ERR_KIND;
    if (beta != 0 && beta != 1)
        return MSWZ_ERR_INVALID;
    if (!is_aligned16(A) || !is_aligned16(B) || !is_aligned16(D) || !is_aligned16(SFA) ||
        !is_aligned16(SFB))
        return MSWZ_ERR_ALIGN;
    mswz::MxArgs a{A, B, SFA, SFB, static_cast<float *>(D), int(p->M), int(p->N), int(p->K), beta,
                   p->group_m, out_kind(p->d_dt), int(p->lda), int(p->ldb), int(p->ldd), {}, p->scale_vec_len,
                   p->sf_major == MSWZ_MAJOR_MN};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = p->variant == mswz::kVarMx256 ? mswz::launch_mx256(a, mx_kind(p->a_dt), mx_kind(p->b_dt), st)
                                                  : mswz::launch_mx(p->variant, a, st);
    return e == hipSuccess ? MSWZ_OK : MSWZ_ERR_HIP;
}

int gemm_run_opts(const gemm_plan *p, const void *A, const void *B, const uint8_t *SFA, const uint8_t *SFB,
                  void *D, int beta, const gemm_opts *o, void *stream)
{
    if (!p || !A || !B || !D)
        return MSWZ_ERR_INVALID;
    const bool mx = p->scale_vec_len != 0;
    if (mx != (SFA != nullptr) || mx != (SFB != nullptr))
        return MSWZ_ERR_INVALID;
    if (beta != 0 && beta != 1)
        return MSWZ_ERR_INVALID;
    if (!is_aligned16(A) || !is_aligned16(B) || !is_aligned16(D) || (mx && (!is_aligned16(SFA) || !is_aligned16(SFB))))
        return MSWZ_ERR_ALIGN;
    mswz::EpiOpts e{};
    if (o) {
        e.neg = (o->neg_a != 0) != (o->neg_b != 0);
        e.sat = o->sat_d != 0;
        e.row_mask = o->row_mask;
        e.col_zero = o->col_zero;
        if ((reinterpret_cast<uintptr_t>(e.row_mask) & 3u) || (reinterpret_cast<uintptr_t>(e.col_zero) & 3u))
            return MSWZ_ERR_ALIGN;
        if (!o->pred)
            return MSWZ_OK;
    }
    if (!e.neg && !e.sat && !e.row_mask && !e.col_zero)
        return mx ? gemm_run_blockscaled(p, A, B, SFA, SFB, D, beta, stream) : gemm_run(p, A, B, D, beta, stream);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool a_mn = p->a_major == MSWZ_MAJOR_MN, b_mn = p->b_major == MSWZ_MAJOR_MN;
    hipError_t err;
    if (mx) {
        mswz::MxArgs a{A, B, SFA, SFB, static_cast<float *>(D), int(p->M), int(p->N), int(p->K), beta,
                       p->group_m, out_kind(p->d_dt), int(p->lda), int(p->ldb), int(p->ldd), e,
                       p->scale_vec_len, p->sf_major == MSWZ_MAJOR_MN};
        err = mswz::launch_mx256(a, mx_kind(p->a_dt), mx_kind(p->b_dt), st);
    } else {
        mswz::DenseArgs a{A, B, static_cast<float *>(D), int(p->M), int(p->N), int(p->K), beta,
                          p->group_m, out_kind(p->d_dt), int(p->lda), int(p->ldb), int(p->ldd), e};
        err = mswz::launch_dense256(p->a_dt == MSWZ_DT_BF16, a_mn, b_mn, a, st);
    }
    return err == hipSuccess ? MSWZ_OK : MSWZ_ERR_HIP;
}

void gemm_plan_destroy(gemm_plan *p) { delete p; }

const char *gemm_status_str(int status)
{
    switch (status) {
    case MSWZ_OK: return "ok";
    case MSWZ_ERR_INVALID: return "invalid argument (size, null pointer, beta or enum value)";
    case MSWZ_ERR_UNSUPPORTED: return "unsupported: no kernel for this dtype/major combination or shape";
    case MSWZ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MSWZ_ERR_HIP: return "HIP runtime error on launch";
    case MSWZ_ERR_KIND: return "plan kind does not match the run function (dense vs block-scaled)";
    case MSWZ_ERR_SCRATCH: return "the plan's workspace exceeds the library's static scratch (gemm_noalloc_scratch_bytes)";
    default: return "unknown status";
    }
}

int gemm_plan_describe(const gemm_plan *p, int64_t *info, int n)
{
    if (!p || (!info && n > 0) || n < 0)
        return MSWZ_ERR_INVALID;
    const int64_t v[8] = {p->variant,      p->info.tile_m, p->info.tile_n,    p->info.tile_k,
                          p->info.threads, p->blocks,      p->info.lds_bytes, p->group_m};
    const int w = n < 8 ? n : 8;
    for (int i = 0; i < w; ++i)
        info[i] = v[i];
    return w;
}

int64_t mswz_desc_address(int64_t r, int64_t w, int64_t ldo, int64_t sdo, int mode, int major,
                          int64_t origin)
{
    return mswz::desc_address(r, w, ldo, sdo, mode, major, origin);
}

int mswz_desc_check(int64_t ldo, int64_t sdo, int mode, int64_t origin)
{
    return mswz::desc_check(ldo, sdo, mode, origin);
}

uint32_t mswz_tile_offset(uint32_t row, uint32_t chunk) { return mswz::tile_offset(row, chunk); }

int mswz_lds_lanes(int pattern, int p0, int p1, uint32_t *out, int n)
{
    using namespace mswz;
    constexpr int W = 8;   // waves of the 256x256 kernel
    auto in = [](int v, int lo, int hi) { return v >= lo && v < hi; };
    const int count = (pattern == MSWZ_LDS_DMA_K || pattern == MSWZ_LDS_DMA_MN || pattern == MSWZ_LDS_FRAG_MN16 ||
                       pattern == MSWZ_LDS_FRAG_E4M3 || pattern == MSWZ_LDS_FRAG_PAD ||
                       pattern == MSWZ_LDS_FRAG_E4M3_MIXED || pattern == MSWZ_LDS_FRAG_E4M3_FP4 ||
                       pattern == MSWZ_LDS_SCALE_DMA || pattern == MSWZ_LDS_SCALE_DMA_WIDE ||
                       pattern == MSWZ_LDS_SCALE_DMA_WIDE_NAT || pattern == MSWZ_LDS_SCALE_DMA_MN)
                          ? 128 : 64;
    if (!out || n < count)
        return MSWZ_ERR_INVALID;
    for (int l = 0; l < 64; ++l) {
        const int g = l >> 4;
        switch (pattern) {
        case MSWZ_LDS_DMA_K:
            if (!in(p0, 0, 32))
                return MSWZ_ERR_INVALID;
            out[2 * l] = uint32_t(1024 * p0 + 16 * l);
            out[2 * l + 1] = dma_row(p0, l) * kTileRowBytes + 16 * dma_chunk(p0, l);
            break;
        case MSWZ_LDS_DMA_MN:
            if (!in(p0, 0, 32))
                return MSWZ_ERR_INVALID;
            out[2 * l] = uint32_t(1024 * p0 + 16 * l);
            out[2 * l + 1] = dma_mn_krow(p0, l) * kMnRowBytes + 16 * dma_mn_chunk(p0, l);
            break;
        case MSWZ_LDS_FRAG_K16:
        case MSWZ_LDS_FRAG_E2M1:
            if (!in(p0, 0, 16) || !in(p1, 0, 2))
                return MSWZ_ERR_INVALID;
            out[l] = kfrag_base<false>(0, 0, p0, kblk16(g), l) ^ uint32_t(p1 << 6);
            break;
        case MSWZ_LDS_FRAG_MN16: {
            if (!in(p0, 0, 16) || !in(p1, 0, 2))
                return MSWZ_ERR_INVALID;
            const uint32_t base = mn_frag_base16(0, 16 * p0, l);
            out[2 * l] = base + uint32_t(32 * p1) * kMnRowBytes;
            out[2 * l + 1] = base + uint32_t(32 * p1 + 4) * kMnRowBytes;
            break;
        }
        case MSWZ_LDS_FRAG_E4M3:
        case MSWZ_LDS_FRAG_E4M3_MIXED:
        case MSWZ_LDS_FRAG_PAD: {
            if (!in(p0, 0, 16))
                return MSWZ_ERR_INVALID;
            const int c = pattern == MSWZ_LDS_FRAG_E4M3 ? mx_chunk16(g)
                          : pattern == MSWZ_LDS_FRAG_PAD ? fp6_chunk16(g) : mx_chunk16_mixed(g);
            const uint32_t base = kfrag_base<true>(0, 0, p0, c, l);
            out[2 * l] = base;
            out[2 * l + 1] = base ^ (pattern == MSWZ_LDS_FRAG_PAD ? 16u : 64u);
            break;
        }
        case MSWZ_LDS_FRAG_E4M3_FP4: {
            if (!in(p0, 0, 16))
                return MSWZ_ERR_INVALID;
            const uint32_t base = kfrag_base<true>(0, 0, p0, pair_chunk16(g), l);
            out[2 * l] = base;
            out[2 * l + 1] = base ^ 32u;
            break;
        }
        case MSWZ_LDS_SCALE_GRP:
            // grouped scale stage: 16 bytes per row slot, block b of row x in slot 16b + x
            if (!in(p0, 0, 8) || !in(p1, 0, 4))
                return MSWZ_ERR_INVALID;
            out[l] = uint32_t(16 * ((l & 15) + 16 * p0) + g + 4 * p1);
            break;
        case MSWZ_LDS_SCALE_DMA:
            if (!in(p0, 0, W))
                return MSWZ_ERR_INVALID;
            out[2 * l] = uint32_t(1024 * p0 + 16 * l);
            out[2 * l + 1] = uint32_t(sf_slot_row(l));
            break;
        case MSWZ_LDS_SCALE_GRP_WIDE:
            if (!in(p0, 0, 8) || !in(p1, 0, 8))
                return MSWZ_ERR_INVALID;
            out[l] = sf_wide_read(0, p0, uint32_t(p1 >> 2), uint32_t(4 * (p1 & 3) + g), l);
            break;
        case MSWZ_LDS_SCALE_FP4_WIDE: {
            if (!in(p0, 0, 8) || !in(p1, 0, 8))
                return MSWZ_ERR_INVALID;
            const int widx = p1 >> 1, ks = p1 & 1;
            out[l] = sf_wide_read(0, p0, uint32_t(widx >> 1), uint32_t(8 * (widx & 1) + 4 * ks + kblk16(g)), l);
            break;
        }
        case MSWZ_LDS_SCALE_DMA_WIDE:
        case MSWZ_LDS_SCALE_DMA_WIDE_NAT: {
            if (!in(p0, 0, W) || !in(p1, 0, 2))
                return MSWZ_ERR_INVALID;
            const int slot = l & 31;
            const int row = 32 * p1 + (pattern == MSWZ_LDS_SCALE_DMA_WIDE ? sf_slot_row(slot) : slot);
            out[2 * l] = uint32_t(2048 * p0 + 1024 * p1 + 16 * l);
            out[2 * l + 1] = uint32_t(2 * row + (l >> 5));
            break;
        }
        case MSWZ_LDS_SCALE_DMA_MN: {
            if (!in(p0, 0, W) || !in(p1, 0, 2))
                return MSWZ_ERR_INVALID;
            const int i = 2 * (p0 & 3) + p1;
            out[2 * l] = uint32_t(2048 * p0 + 1024 * p1 + 16 * l);
            out[2 * l + 1] = 256u * sf_mn_copy_block(i, l) + sf_mn_copy_row(l);
            break;
        }
        case MSWZ_LDS_SCALE_GRP_MN:
            if (!in(p0, 0, 8) || !in(p1, 0, 8))
                return MSWZ_ERR_INVALID;
            out[l] = sf_mn_offset(uint32_t(4 * p1 + g), uint32_t(row16<true>(p0, l & 15)));
            break;
        case MSWZ_LDS_SCALE_FP4_MN:
            if (!in(p0, 0, 8) || !in(p1, 0, 8))
                return MSWZ_ERR_INVALID;
            out[l] = sf_mn_offset(uint32_t(4 * p1 + kblk16(g)), uint32_t(16 * p0 + (l & 15)));
            break;
        case MSWZ_LDS_EPI_WRITE: {
            const int rows = p1 >> 4, ii = (p1 >> 2) & 3, j = p1 & 3;
            if (!in(p0, 0, 4) || rows > 3 || ii > 1 || p1 < 0)
                return MSWZ_ERR_INVALID;
            out[l] = rows == 0 ? epi_write_offset<false, false>(p0, ii, j, l)
                     : rows == 1 ? epi_write_offset<true, true>(p0, ii, j, l)
                     : rows == 2 ? epi_write_offset<true, false>(p0, ii, j, l)
                                 : epi_write_offset<false, true>(p0, ii, j, l);
            break;
        }
        case MSWZ_LDS_EPI_READ:
            if (!in(p0, 0, 8))
                return MSWZ_ERR_INVALID;
            out[l] = epi_read_offset(p0, l);
            break;
        default:
            return MSWZ_ERR_INVALID;
        }
    }
    return count;
}

int mswz_tile_of_block(int block, int tiles_m, int tiles_n, int group_m, int *tile_m, int *tile_n)
{
    if (!tile_m || !tile_n || tiles_m <= 0 || tiles_n <= 0 || block < 0 || block >= tiles_m * tiles_n ||
        group_m == 0 || group_m > 64 || group_m < -64)
        return MSWZ_ERR_INVALID;
    mswz::tile_of_block(block, tiles_m, tiles_n, group_m, *tile_m, *tile_n);
    return MSWZ_OK;
}

}  // extern "C"
