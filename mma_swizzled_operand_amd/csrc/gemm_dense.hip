// gemm_dense.hip — fp16 / bf16 GEMM for gfx950: D = beta*D + A.B^T, fp32
// accumulate (tcgen05.mma page, "Operands and repeat axes" and the
// 128x64x64 example; operand majors from "Shared descriptors are byte-stride
// contracts").
//
// The 128x128 and 64x64 tiles (the 256x256 tile lives in gemm256_kernel.hpp).
// Structure of one 256-thread workgroup (4 waves) computing a BM x BN tile:
//   * K advances 64 elements per step; each step stages a [BM][128 B] A tile
//     and a [BN][128 B] B tile in LDS, in the swizzled tile layout of
//     layout.hpp, double-buffered: while the MFMAs consume stage k, the
//     16-byte global loads of step k+1 are in flight in registers and are
//     written to the other stage afterwards; one barrier per step.
//   * K-major operands are copied row by row (8 lanes cover one 128-byte row,
//     so each wave-wide load reads eight whole rows).  An MN-major operand
//     ([K][M] or [K][N]) is read as 8x8 blocks (eight 16-byte pieces of eight
//     consecutive K rows), transposed in registers and written as K-contiguous
//     tile rows, so the MFMA read path is the same for both majors.
//   * Each wave owns a WM x WN sub-tile made of 32x32 MFMA blocks.  The MFMA's
//     first operand is the B fragment and its second the A fragment, which
//     puts four consecutive N columns of one M row in four consecutive
//     accumulator registers: the epilogue writes D with 16-byte stores.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mswz {
namespace {

constexpr int kThreads = 256;

template <int BM, int BN, int WM, int WN, bool BF16, bool A_MN, bool B_MN, bool BETA>
__global__ void __launch_bounds__(kThreads)
gemm16_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, float *__restrict__ D,
              int M, int N, int K, int tiles_m, int tiles_n, int group_m)
{
    constexpr int kWavesN = BN / WN;
    static_assert((BM / WM) * kWavesN == 4, "four waves per workgroup");
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int kATile = BM * 128, kBTile = BN * 128, kStage = kATile + kBTile;
    constexpr int NA = A_MN ? 8 : BM / 32;   // 16-byte pieces of A per thread per step
    constexpr int NB = B_MN ? 8 : BN / 32;   // 16-byte pieces of B per thread per step
    static_assert(!A_MN || BM <= kThreads, "one 8x8 block per thread at most");
    static_assert(!B_MN || BN <= kThreads, "one 8x8 block per thread at most");

    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int wm = (wave / kWavesN) * WM, wn = (wave % kWavesN) * WN;

    // ---- staging assignment (constant over the K loop) ----------------------
    const size_t row_bytes = size_t(K) * 2;   // one K-major row of A or B
    const int srow = tid >> 3, schunk = tid & 7;
    const uint8_t *gb;
    uint32_t lb[NB];
    bool b_active = true;
    if constexpr (B_MN) {
        // block (nb, kc): tile rows 8*nb .. 8*nb+7 (N), K rows 8*kc .. 8*kc+7
        const int nb = tid % (BN / 8), kc = tid / (BN / 8);
        b_active = tid < BN;
        gb = B + (size_t(8 * kc) * N + n0 + 8 * nb) * 2;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            lb[i] = kATile + tile_offset(8 * nb + i, kc & 7);
    } else {
        gb = B + size_t(n0 + srow) * row_bytes + schunk * 16;
#pragma unroll
        for (int i = 0; i < NB; ++i)
            lb[i] = kATile + tile_offset(srow + 32 * i, schunk);
    }
    const size_t b_mn_row = size_t(N) * 2;    // bytes between K rows of an MN-major B

    const uint8_t *ga;
    uint32_t la[A_MN ? 8 : NA];
    bool a_active = true;
    if constexpr (A_MN) {
        // block (mb, kc): tile rows 8*mb .. 8*mb+7 (M), K rows 8*kc .. 8*kc+7
        const int mb = tid % (BM / 8), kc = tid / (BM / 8);
        a_active = tid < BM;
        ga = A + (size_t(8 * kc) * M + m0 + 8 * mb) * 2;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            la[i] = tile_offset(8 * mb + i, kc & 7);
    } else {
        ga = A + size_t(m0 + srow) * row_bytes + schunk * 16;
#pragma unroll
        for (int i = 0; i < NA; ++i)
            la[i] = tile_offset(srow + 32 * i, schunk);
    }
    const size_t a_mn_row = size_t(M) * 2;    // bytes between K rows of an MN-major A

    u32x4 ra[NA], rb[NB];
    auto load_step = [&](int kt) {
        const size_t kb = size_t(kt) * 128;   // 64 K elements
        if constexpr (A_MN) {
            if (a_active) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    ra[j] = global_read16(ga + (size_t(kt) * 64 + j) * a_mn_row);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NA; ++i)
                ra[i] = global_read16(ga + size_t(32 * i) * row_bytes + kb);
        }
        if constexpr (B_MN) {
            if (b_active) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    rb[j] = global_read16(gb + (size_t(kt) * 64 + j) * b_mn_row);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NB; ++i)
                rb[i] = global_read16(gb + size_t(32 * i) * row_bytes + kb);
        }
    };
    auto store_step = [&](int stage) {
        uint8_t *s = lds + stage * kStage;
        if constexpr (A_MN) {
            if (a_active) {
                u32x4 t[8];
                transpose8x8_b16(ra, t);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    lds_write16(s, la[i], t[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NA; ++i)
                lds_write16(s, la[i], ra[i]);
        }
        if constexpr (B_MN) {
            if (b_active) {
                u32x4 t[8];
                transpose8x8_b16(rb, t);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    lds_write16(s, lb[i], t[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NB; ++i)
                lds_write16(s, lb[i], rb[i]);
        }
    };

    // ---- MFMA operand read offsets -------------------------------------------
    // Lane (lr, lh) of a 32-row block reads row lr, 16-byte chunk 2*ks + lh of
    // K sub-step ks; in the tile layout that chunk sits at (2*ks) ^ (key ^ lh).
    uint32_t aoff[TM], akey[TM], boff[TN], bkey[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const uint32_t row = wm + 32 * i + lr;
        aoff[i] = row * kTileRowBytes;
        akey[i] = tile_key(row) ^ lh;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const uint32_t row = wn + 32 * j + lr;
        boff[j] = kATile + row * kTileRowBytes;
        bkey[j] = tile_key(row) ^ lh;
    }

    f32x16 acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
            acc[j][i] = f32x16{};

    const int KT = K / 64;
    load_step(0);
    store_step(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT)
            load_step(kt + 1);
        const uint8_t *s = lds + cur * kStage;
        // fragments of sub-step ks+1 are read while the MFMAs of ks run
        u32x4 af[2][TM], bf[2][TN];
        auto read_frags = [&](int ks, u32x4 *a, u32x4 *b) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                a[i] = lds_read16(s, aoff[i] + (((2u * ks) ^ akey[i]) << 4));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                b[j] = lds_read16(s, boff[j] + (((2u * ks) ^ bkey[j]) << 4));
        };
        read_frags(0, af[0], bf[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4)
                read_frags(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    acc[j][i] = mfma_32x32x16<BF16>(bf[ks & 1][j], af[ks & 1][i], acc[j][i]);
        }
        if (kt + 1 < KT)
            store_step(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane (lr, lh), registers 4q..4q+3 of block (j, i) hold
    // D[m0+wm+32i+lr][n0+wn+32j+8q+4lh .. +3] ----------------------------------
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const size_t m = size_t(m0 + wm + 32 * i + lr);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn + 32 * j + 8 * q + 4 * lh;
                f32x4 v = {acc[j][i][4 * q + 0], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                           acc[j][i][4 * q + 3]};
                f32x4 *p = reinterpret_cast<f32x4 *>(D + m * N + n);
                if constexpr (BETA)
                    v += *p;
                *p = v;
            }
        }
}

template <int BM, int BN, int WM, int WN, bool BF16, bool A_MN, bool B_MN>
hipError_t launch_one(const DenseArgs &a, hipStream_t stream)
{
    const int tiles_m = a.M / BM, tiles_n = a.N / BN;
    const int blocks = tiles_m * tiles_n;
    const uint8_t *A = static_cast<const uint8_t *>(a.A);
    const uint8_t *B = static_cast<const uint8_t *>(a.B);
    if (a.beta)
        hipLaunchKernelGGL((gemm16_kernel<BM, BN, WM, WN, BF16, A_MN, B_MN, true>), dim3(blocks),
                           dim3(kThreads), 0, stream, A, B, a.D, a.M, a.N, a.K, tiles_m, tiles_n,
                           a.group_m);
    else
        hipLaunchKernelGGL((gemm16_kernel<BM, BN, WM, WN, BF16, A_MN, B_MN, false>), dim3(blocks),
                           dim3(kThreads), 0, stream, A, B, a.D, a.M, a.N, a.K, tiles_m, tiles_n,
                           a.group_m);
    return hipGetLastError();
}

template <bool BF16, bool A_MN, bool B_MN>
hipError_t launch_variant(int variant, const DenseArgs &a, hipStream_t stream)
{
    switch (variant) {
    case kVarDense128: return launch_one<128, 128, 64, 64, BF16, A_MN, B_MN>(a, stream);
    case kVarDense64: return launch_one<64, 64, 32, 32, BF16, A_MN, B_MN>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <bool BF16>
hipError_t launch_majors(int variant, bool a_mn, bool b_mn, const DenseArgs &a, hipStream_t stream)
{
    if (a_mn)
        return b_mn ? launch_variant<BF16, true, true>(variant, a, stream)
                    : launch_variant<BF16, true, false>(variant, a, stream);
    return b_mn ? launch_variant<BF16, false, true>(variant, a, stream)
                : launch_variant<BF16, false, false>(variant, a, stream);
}

}  // namespace

hipError_t launch_dense(int variant, bool bf16, bool a_mn, bool b_mn, const DenseArgs &args,
                        hipStream_t stream)
{
    return bf16 ? launch_majors<true>(variant, a_mn, b_mn, args, stream)
                : launch_majors<false>(variant, a_mn, b_mn, args, stream);
}

}  // namespace mswz
