// gemm_mx.hip — block-scaled OCP E4M3 GEMM for gfx950 (MX-fp8):
//     D = beta*D + sum_k (2^(SFA[m][k/32]-127) a(m,k)) (2^(SFB[n][k/32]-127) b(n,k))
// (tcgen05.mma page, "Weight-stationary and block scaling": per-row scale
// vectors for A and B, one scale per block of consecutive K elements).
//
// The 128x128 and 64x64 tiles (the 256x256 tile lives in gemm256_kernel.hpp).
// Same workgroup structure as gemm_dense.hip: 4 waves, a BM x BN tile,
// double-buffered swizzled LDS stages of 128 bytes per operand row (here 128
// K elements), 16-byte global loads prefetched one K step ahead in registers.
// The multiply is the gfx950 scaled MFMA 32x32x64.  Its operand image, pinned
// by an on-device probe: lane (r, h) of a 32-row block (r = lane % 32,
// h = lane / 32) holds row r, K elements 16h..16h+15 in bytes 0..15 and
// 32+16h..32+16h+15 in bytes 16..31; the scale of K block 0 (K 0..31) of row
// r is taken from lane r and that of block 1 (K 32..63) from lane 32+r, byte
// `op_sel` of the 32-bit scale operand.  So each lane supplies the scale of
// block h of its row while its data straddles both blocks.
// Scale bytes are read straight from global memory: the four bytes of one
// row that cover a 128-element K step form one aligned 32-bit word, loaded one
// step ahead with the tiles; each lane shifts its own half of the word into
// place and the instruction's byte select picks the sub-step.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mswz {
namespace {

constexpr int kThreads = 256;

template <int BM, int BN, int WM, int WN, bool BETA>
__global__ void __launch_bounds__(kThreads)
gemm_mx_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ B,
               const uint8_t *__restrict__ SFA, const uint8_t *__restrict__ SFB,
               float *__restrict__ D, int M, int N, int K, int tiles_m, int tiles_n, int group_m)
{
    constexpr int kWavesN = BN / WN;
    static_assert((BM / WM) * kWavesN == 4, "four waves per workgroup");
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int kATile = BM * 128, kBTile = BN * 128, kStage = kATile + kBTile;
    constexpr int NA = BM / 32, NB = BN / 32;

    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int wm = (wave / kWavesN) * WM, wn = (wave % kWavesN) * WN;
    (void)M;

    // ---- staging: 8 lanes per 128-byte row ------------------------------------
    const size_t row_bytes = size_t(K);
    const int srow = tid >> 3, schunk = tid & 7;
    const uint8_t *ga = A + size_t(m0 + srow) * row_bytes + schunk * 16;
    const uint8_t *gb = B + size_t(n0 + srow) * row_bytes + schunk * 16;
    uint32_t la[NA], lb[NB];
#pragma unroll
    for (int i = 0; i < NA; ++i)
        la[i] = tile_offset(srow + 32 * i, schunk);
#pragma unroll
    for (int i = 0; i < NB; ++i)
        lb[i] = kATile + tile_offset(srow + 32 * i, schunk);

    // ---- scale rows this lane multiplies with ---------------------------------
    const int sf_row = K / 32;   // bytes per scale row
    const uint32_t *sfa_p[TM];
    const uint32_t *sfb_p[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
        sfa_p[i] = reinterpret_cast<const uint32_t *>(SFA + size_t(m0 + wm + 32 * i + lr) * sf_row);
#pragma unroll
    for (int j = 0; j < TN; ++j)
        sfb_p[j] = reinterpret_cast<const uint32_t *>(SFB + size_t(n0 + wn + 32 * j + lr) * sf_row);

    u32x4 ra[NA], rb[NB];
    uint32_t sa_next[TM], sb_next[TN];
    auto load_step = [&](int kt) {
        const size_t kb = size_t(kt) * 128;
#pragma unroll
        for (int i = 0; i < NA; ++i)
            ra[i] = global_read16(ga + size_t(32 * i) * row_bytes + kb);
#pragma unroll
        for (int i = 0; i < NB; ++i)
            rb[i] = global_read16(gb + size_t(32 * i) * row_bytes + kb);
#pragma unroll
        for (int i = 0; i < TM; ++i)
            sa_next[i] = sfa_p[i][kt];
#pragma unroll
        for (int j = 0; j < TN; ++j)
            sb_next[j] = sfb_p[j][kt];
    };
    auto store_step = [&](int stage) {
        uint8_t *s = lds + stage * kStage;
#pragma unroll
        for (int i = 0; i < NA; ++i)
            lds_write16(s, la[i], ra[i]);
#pragma unroll
        for (int i = 0; i < NB; ++i)
            lds_write16(s, lb[i], rb[i]);
    };

    // ---- MFMA operand read offsets -------------------------------------------
    // Sub-step ks (64 K elements): lane (lr, lh) reads 16-byte chunks
    // 4ks + lh and 4ks + 2 + lh of its row; they sit at 4ks ^ (key ^ lh) and
    // 4ks ^ (key ^ (2 + lh)).
    uint32_t aoff[TM], ak0[TM], ak1[TM], boff[TN], bk0[TN], bk1[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const uint32_t row = wm + 32 * i + lr;
        aoff[i] = row * kTileRowBytes;
        ak0[i] = tile_key(row) ^ lh;
        ak1[i] = tile_key(row) ^ (2 + lh);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const uint32_t row = wn + 32 * j + lr;
        boff[j] = kATile + row * kTileRowBytes;
        bk0[j] = tile_key(row) ^ lh;
        bk1[j] = tile_key(row) ^ (2 + lh);
    }

    f32x16 acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
            acc[j][i] = f32x16{};

    const int KT = K / 128;
    uint32_t sa[TM], sb[TN];
    load_step(0);
    store_step(0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
        sa[i] = sa_next[i] >> (8 * lh);
#pragma unroll
    for (int j = 0; j < TN; ++j)
        sb[j] = sb_next[j] >> (8 * lh);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT)
            load_step(kt + 1);
        const uint8_t *s = lds + cur * kStage;
        i32x8 af[2][TM], bf[2][TN];
        auto read_frags = [&](int ks, i32x8 *a, i32x8 *b) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const u32x4 lo = lds_read16(s, aoff[i] + (((4u * ks) ^ ak0[i]) << 4));
                const u32x4 hi = lds_read16(s, aoff[i] + (((4u * ks) ^ ak1[i]) << 4));
                a[i] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const u32x4 lo = lds_read16(s, boff[j] + (((4u * ks) ^ bk0[j]) << 4));
                const u32x4 hi = lds_read16(s, boff[j] + (((4u * ks) ^ bk1[j]) << 4));
                b[j] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        };
        read_frags(0, af[0], bf[0]);
        read_frags(1, af[1], bf[1]);
        // sub-step 0 uses scale byte 0 (block 4kt + lh), sub-step 1 byte 2 (block 4kt + 2 + lh)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[j][i] = mfma_scale_32x32x64_e4m3<0>(bf[0][j], af[0][i], acc[j][i], sb[j], sa[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[j][i] = mfma_scale_32x32x64_e4m3<2>(bf[1][j], af[1][i], acc[j][i], sb[j], sa[i]);
        if (kt + 1 < KT) {
            store_step(cur ^ 1);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                sa[i] = sa_next[i] >> (8 * lh);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                sb[j] = sb_next[j] >> (8 * lh);
        }
        __syncthreads();
    }

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

template <int BM, int BN, int WM, int WN>
hipError_t launch_one(const MxArgs &a, hipStream_t stream)
{
    const int tiles_m = a.M / BM, tiles_n = a.N / BN;
    const int blocks = tiles_m * tiles_n;
    const uint8_t *A = static_cast<const uint8_t *>(a.A);
    const uint8_t *B = static_cast<const uint8_t *>(a.B);
    if (a.beta)
        hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, WM, WN, true>), dim3(blocks), dim3(kThreads), 0,
                           stream, A, B, a.SFA, a.SFB, a.D, a.M, a.N, a.K, tiles_m, tiles_n,
                           a.group_m);
    else
        hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, WM, WN, false>), dim3(blocks), dim3(kThreads), 0,
                           stream, A, B, a.SFA, a.SFB, a.D, a.M, a.N, a.K, tiles_m, tiles_n,
                           a.group_m);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mx(int variant, const MxArgs &args, hipStream_t stream)
{
    switch (variant) {
    case kVarMx128: return launch_one<128, 128, 64, 64>(args, stream);
    case kVarMx64: return launch_one<64, 64, 32, 32>(args, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mswz
