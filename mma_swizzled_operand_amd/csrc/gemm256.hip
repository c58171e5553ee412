// gemm256.hip — the large-tile GEMM for gfx950: one 512-thread workgroup (8
// waves, two per SIMD) computes a 256 x 256 tile of
//     D = beta*D + A.B^T                                   (fp16 / bf16)
//     D = beta*D + sum_k (2^(SFA-127) a) (2^(SFB-127) b)   (OCP E4M3, 32-element blocks)
// (tcgen05.mma page, "Operands and repeat axes", "Shared descriptors are
// byte-stride contracts", "Weight-stationary and block scaling").
//
// Staging.  Each K step moves 128 bytes of every A and B tile row (64 16-bit
// or 128 8-bit K elements) into one of two LDS stages, held in two distinct
// LDS arrays with the K loop unrolled by two, so that reads of one stage never
// wait for copies into the other.  K-major operands are copied with direct
// global-to-LDS 16-byte loads: one wave instruction fills 1 KiB of LDS
// contiguously, lane l at byte 16*l, i.e. eight 128-byte tile rows.  The
// tile layout (layout.hpp) permutes 16-byte chunks inside a row, and the
// permutation is its own inverse, so lane l simply fetches the source chunk
// that belongs at its destination: chunk (l % 8) ^ key(row).  An MN-major A
// ([K][M]) is read into registers as 8x8 blocks, transposed, and written with
// 16-byte LDS stores into the same K-contiguous layout.
//
// Compute.  Wave w owns output rows 128*(w/4) .. +127 and columns 64*(w%4)
// .. +63: 4 x 2 blocks of 32x32 MFMA output, 128 fp32 accumulators per lane.
// The MFMA's first operand is the B fragment and its second the A fragment,
// so four consecutive accumulator registers hold four consecutive N columns
// of one M row and the epilogue stores 16 bytes per lane.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mswz {
namespace {

constexpr int kThreads = 512;
constexpr int kBM = 256, kBN = 256;
constexpr int kATile = kBM * 128, kBTile = kBN * 128, kStage = kATile + kBTile;
constexpr int TM = 4, TN = 2;   // 32x32 blocks per wave along M and N

enum Kind { kBf16 = 0, kF16 = 1, kE4m3 = 2 };

// Direct-to-LDS copy of one K-major operand tile (256 rows x 128 bytes per K
// step) through a buffer resource on the workgroup's 256-row panel.  Wave w
// copies rows 8*(w + 8i) .. +7 for i = 0..3; lane l takes row 8*(w + 8i) + l/8,
// whose layout key is (l/8) ^ w, so it fetches chunk (l % 8) ^ (l/8) ^ w.
struct DmaOperand {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t voff;       // this lane's byte offset in the panel for i = 0, K step 0
    uint32_t step64;     // bytes between the row groups of consecutive i (64 rows)
    uint32_t lds_off;    // LDS offset of this wave's first destination row inside a stage

    __device__ void init(const uint8_t *X, int row0, uint32_t row_bytes, int wave, int lane,
                         uint32_t tile_off)
    {
        rsrc = make_rsrc(X + size_t(row0) * row_bytes, 256u * row_bytes);
        const int r = 8 * wave + (lane >> 3);
        const int chunk = (lane & 7) ^ (((lane >> 3) ^ wave) & 7);
        voff = uint32_t(r) * row_bytes + chunk * 16;
        step64 = 64u * row_bytes;
        lds_off = tile_off + 8 * wave * kTileRowBytes;
    }

    __device__ void issue(uint8_t *stage, int kt) const
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            buffer_load_lds16(rsrc, stage + lds_off + i * 64 * kTileRowBytes, voff,
                              i * step64 + uint32_t(kt) * 128);
    }
};

template <int KIND, bool A_MN, bool BETA>
__global__ void __launch_bounds__(kThreads)
gemm256_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ B,
               const uint8_t *__restrict__ SFA, const uint8_t *__restrict__ SFB,
               float *__restrict__ D, int M, int N, int K, int tiles_m, int tiles_n, int group_m)
{
    static_assert(!(A_MN && KIND == kE4m3), "MN-major A is built for 16-bit operands only");
    constexpr bool kMx = KIND == kE4m3;
    constexpr int kElem = kMx ? 1 : 2;
    constexpr int kStepK = 128 / kElem;   // K elements per step

    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, lh = lane >> 5;
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int wm = (wave >> 2) * 128, wn = (wave & 3) * 64;
    const uint32_t row_bytes = uint32_t(K) * kElem;

    // ---- staging state ---------------------------------------------------------
    DmaOperand db;
    db.init(B, n0, row_bytes, wave, lane, kATile);
    DmaOperand da;
    if constexpr (!A_MN)
        da.init(A, m0, row_bytes, wave, lane, 0);

    // MN-major A ([K][M]): waves 0..3 each stage one 8x8 block per lane:
    // tile rows 8*mb .. +7 (M), K rows 8*kc .. +7 of the step, mb = tid % 32,
    // kc = tid / 32.  Read through a buffer resource on columns m0.. of A.
    const bool a_mn_active = tid < 256;
    __amdgpu_buffer_rsrc_t ra_rsrc;
    uint32_t ra_voff = 0, la_mn0 = 0;
    const uint32_t a_mn_row = uint32_t(M) * 2;
    u32x4 ra[A_MN ? 8 : 1];
    if constexpr (A_MN) {
        const int mb = tid & 31, kc = (tid >> 5) & 7;
        ra_rsrc = make_rsrc(A + size_t(m0) * 2, uint32_t(K) * a_mn_row - uint32_t(m0) * 2);
        ra_voff = uint32_t(8 * kc) * a_mn_row + 16 * mb;
        la_mn0 = tile_offset(8 * mb, kc);   // rows 8mb+i: key = i ^ mb, chunk kc
        (void)la_mn0;
    }
    auto a_mn_load = [&](int kt) {
        if (a_mn_active) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                ra[j] = buffer_load16(ra_rsrc, ra_voff, (uint32_t(kt) * 64 + j) * a_mn_row);
        }
    };
    auto a_mn_store = [&](uint8_t *stage) {
        if (a_mn_active) {
            const int mb = tid & 31, kc = (tid >> 5) & 7;
            u32x4 t[8];
            transpose8x8_b16(ra, t);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                lds_write16(stage, tile_offset(8 * mb + i, kc), t[i]);
        }
    };

    // ---- scales (MX): one 32-bit word of 4 scale bytes per row per K step -------
    __amdgpu_buffer_rsrc_t sfa_rsrc, sfb_rsrc;
    uint32_t sfa_voff = 0, sfb_voff = 0;
    const uint32_t sf_row = uint32_t(K) / 32;
    uint32_t sa[TM], sb[TN], sa_n[TM], sb_n[TN];
    if constexpr (kMx) {
        sfa_rsrc = make_rsrc(SFA + size_t(m0) * sf_row, 256u * sf_row);
        sfb_rsrc = make_rsrc(SFB + size_t(n0) * sf_row, 256u * sf_row);
        sfa_voff = uint32_t(wm + lr) * sf_row;
        sfb_voff = uint32_t(wn + lr) * sf_row;
    }
    auto scales_load = [&](int kt) {
        if constexpr (kMx) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                sa_n[i] = buffer_load4(sfa_rsrc, sfa_voff, uint32_t(32 * i) * sf_row + 4u * kt);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                sb_n[j] = buffer_load4(sfb_rsrc, sfb_voff, uint32_t(32 * j) * sf_row + 4u * kt);
        }
    };
    auto scales_take = [&]() {
        if constexpr (kMx) {
            // lane half lh supplies the scale of K block lh of its row
#pragma unroll
            for (int i = 0; i < TM; ++i)
                sa[i] = sa_n[i] >> (8 * lh);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                sb[j] = sb_n[j] >> (8 * lh);
        }
    };

    auto issue_step = [&](uint8_t *stage, int kt) {
        if constexpr (A_MN)
            a_mn_load(kt);
        else
            da.issue(stage, kt);
        db.issue(stage, kt);
        scales_load(kt);
    };

    // ---- MFMA operand read addresses -------------------------------------------
    // Block row `row` of a fragment, 16-byte chunk c, sits at
    // row*128 + ((c ^ key(row)) << 4).  For sub-step ks the chunk is
    // 2ks ^ lh (16-bit) or 4ks ^ lh and 4ks ^ 2 ^ lh (8-bit), so every address
    // is one per-fragment base XOR a constant.
    uint32_t abase[TM], bbase[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const uint32_t row = wm + 32 * i + lr;
        abase[i] = row * kTileRowBytes + ((lh ^ tile_key(row)) << 4);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const uint32_t row = wn + 32 * j + lr;
        bbase[j] = kATile + row * kTileRowBytes + ((lh ^ tile_key(row)) << 4);
    }

    f32x16 acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
            acc[j][i] = f32x16{};

    auto compute16 = [&](const uint8_t *s) {
        uint32_t ab[TM], bb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            ab[i] = opaque(abase[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            bb[j] = opaque(bbase[j]);
        u32x4 af[2][TM], bf[2][TN];
        auto rd = [&](int ks, u32x4 *a, u32x4 *b) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                a[i] = lds_read16(s, ab[i] ^ (ks << 5));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                b[j] = lds_read16(s, bb[j] ^ (ks << 5));
        };
        rd(0, af[0], bf[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4)
                rd(ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    acc[j][i] = mfma_32x32x16<KIND == kBf16>(bf[ks & 1][j], af[ks & 1][i], acc[j][i]);
        }
    };

    auto compute_mx = [&](const uint8_t *s) {
        uint32_t ab[TM], bb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            ab[i] = opaque(abase[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            bb[j] = opaque(bbase[j]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            i32x8 af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const u32x4 lo = lds_read16(s, ab[i] ^ (ks << 6));
                const u32x4 hi = lds_read16(s, ab[i] ^ (ks << 6) ^ 32u);
                af[i] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const u32x4 lo = lds_read16(s, bb[j] ^ (ks << 6));
                const u32x4 hi = lds_read16(s, bb[j] ^ (ks << 6) ^ 32u);
                bf[j] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    if (ks == 0)
                        acc[j][i] = mfma_scale_32x32x64_e4m3<0>(bf[j], af[i], acc[j][i], sb[j], sa[i]);
                    else
                        acc[j][i] = mfma_scale_32x32x64_e4m3<2>(bf[j], af[i], acc[j][i], sb[j], sa[i]);
                }
        }
    };

    auto compute = [&](const uint8_t *s) {
        if constexpr (kMx)
            compute_mx(s);
        else
            compute16(s);
    };

    // ---- main loop: two K steps per iteration, one stage array each; an odd
    // final step (already in lds0) is computed after the loop ------------------
    const int KT = K / kStepK;
    issue_step(lds0, 0);
    if constexpr (A_MN)
        a_mn_store(lds0);
    __syncthreads();
    scales_take();

    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
        issue_step(lds1, kt + 1);
        compute(lds0);
        if constexpr (A_MN)
            a_mn_store(lds1);
        __syncthreads();
        scales_take();
        const bool more = kt + 2 < KT;
        if (more)
            issue_step(lds0, kt + 2);
        compute(lds1);
        if constexpr (A_MN) {
            if (more)
                a_mn_store(lds0);
        }
        __syncthreads();
        scales_take();
    }
    if (kt < KT)
        compute(lds0);

    // ---- epilogue -------------------------------------------------------------
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

template <int KIND, bool A_MN>
hipError_t launch_kind(const MxArgs &a, hipStream_t stream)
{
    const int tiles_m = a.M / kBM, tiles_n = a.N / kBN;
    const int blocks = tiles_m * tiles_n;
    const uint8_t *A = static_cast<const uint8_t *>(a.A);
    const uint8_t *B = static_cast<const uint8_t *>(a.B);
    if (a.beta)
        hipLaunchKernelGGL((gemm256_kernel<KIND, A_MN, true>), dim3(blocks), dim3(kThreads), 0, stream,
                           A, B, a.SFA, a.SFB, a.D, a.M, a.N, a.K, tiles_m, tiles_n, a.group_m);
    else
        hipLaunchKernelGGL((gemm256_kernel<KIND, A_MN, false>), dim3(blocks), dim3(kThreads), 0, stream,
                           A, B, a.SFA, a.SFB, a.D, a.M, a.N, a.K, tiles_m, tiles_n, a.group_m);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dense256(bool bf16, bool a_mn, const DenseArgs &d, hipStream_t stream)
{
    const MxArgs a{d.A, d.B, nullptr, nullptr, d.D, d.M, d.N, d.K, d.beta, d.group_m};
    if (bf16)
        return a_mn ? launch_kind<kBf16, true>(a, stream) : launch_kind<kBf16, false>(a, stream);
    return a_mn ? launch_kind<kF16, true>(a, stream) : launch_kind<kF16, false>(a, stream);
}

hipError_t launch_mx256(const MxArgs &a, hipStream_t stream)
{
    return launch_kind<kE4m3, false>(a, stream);
}

}  // namespace mswz
