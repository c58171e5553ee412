// gemm_skinny.hip — weight-streaming GEMM for small M on gfx950:
//     D[M][N] = beta*D + A[M][K] . B[N][K]^T,  1 <= M <= 64, fp16 / bf16
// (tcgen05.mma page, "Operands and repeat axes"; the weight-stationary
// workload of "Weight-stationary and block scaling": few activation rows
// against a large weight matrix streamed once).
//
// The product is bound by reading B once from HBM.  One 512-thread
// workgroup (8 waves) owns 64 columns of D (N/64 workgroups) and the full K
// range, cut into 64-element blocks; wave w multiplies blocks w, w+8, w+16,
// ..., holding the whole M x 64 output block in accumulators (split K inside
// the workgroup), so at any moment the eight waves read 1 KiB of contiguous
// K from each of the 64 rows.  The eight partial blocks are summed through
// LDS in a fixed order at the end, so the result is deterministic.
//
// No LDS in the main loop: fragments go straight from global memory into
// registers in the operand form of the 16x16x32 MFMA, whose lane l supplies
// row l % 16.  The K index inside a 64-element block is permuted identically
// for A and B (a sum over K does not depend on its order) so that for
// sub-step s the four lanes of a row read bytes 64s .. 64s+63 of it: every
// 16-byte load instruction consumes whole 64-byte lines of 16 rows.  Blocks
// are double-buffered two ahead in registers.
//
// M is padded to BM = 32 or 64 rows: every A load carries its row in the
// range-checked per-lane offset and the buffer covers the M rows of A, so the
// rows beyond M read as zeros without a memory access, and only rows below M
// are stored.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mswz {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;
constexpr int kRedPitch = 68;   // floats per row of a partial block in LDS (padded against bank conflicts)

template <bool BF16, int BM, bool BETA>
__global__ void __launch_bounds__(kThreads)
gemm_skinny_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, float *__restrict__ D,
                   int M, int N, int K)
{
    constexpr int TM = BM / 16, TN = kBN / 16;   // 16-row operand blocks of A and of B
    __shared__ __attribute__((aligned(16))) float red[kWaves * BM * kRedPitch];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * kBN;
    const uint32_t row_bytes = uint32_t(K) * 2;
    const int blocks = K / 64 / kWaves;   // 64-element K blocks per wave

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, uint32_t(M) * row_bytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + size_t(n0) * row_bytes, uint32_t(kBN) * row_bytes);
    // lane (lr, lg): row lr of each 16-row block, bytes 64s + 16lg of the wave's block
    const uint32_t voff = uint32_t(lr) * row_bytes + uint32_t(wave) * 128 + 16 * lg;
    // A's row (16i + lr) is in the per-lane offset, which the range check covers
    uint32_t voff_a[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i)
        voff_a[i] = voff + uint32_t(16 * i) * row_bytes;

    // fragment buffers: [buffer][16-row block][sub-step]
    u32x4 fa[2][TM][2], fb[2][TN][2];
    auto load = [&](int buf, int b) {
        const uint32_t kb = uint32_t(b) * (128 * kWaves);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                fb[buf][j][s] = buffer_load16(rb, voff + 64 * s, uint32_t(16 * j) * row_bytes + kb);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                fa[buf][i][s] = buffer_load16(ra, voff_a[i] + 64 * s, kb);
    };

    f32x4 acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
            acc[j][i] = f32x4{};

    auto compute = [&](int buf) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    acc[j][i] = mfma_16x16x32<BF16>(fb[buf][j][s], fa[buf][i][s], acc[j][i]);
    };

    // blocks is even (K % 1024 == 0 is required by the plan); the final pair
    // re-loads the last block into a buffer that is not used again, so the
    // loop body has no branches
    // The fences keep each buffer's 16 loads together and in this order, so
    // the wait before computing on one buffer leaves the other buffer's loads
    // in flight (without them the compiler interleaves the two buffers' loads
    // and has to wait for all of them).
    load(0, 0);
    sched_fence();
    load(1, min(1, blocks - 1));
    sched_fence();
    for (int b = 0; b < blocks; b += 2) {
        compute(0);
        sched_fence();
        load(0, min(b + 2, blocks - 1));
        sched_fence();
        compute(1);
        sched_fence();
        load(1, min(b + 3, blocks - 1));
        sched_fence();
    }

    // ---- reduce the eight K-slice partials through LDS ---------------------------
    // lane (lr, lg), register r of block (j, i): row 16i + lr, column 16j + 4lg + r
    float *mine = red + wave * BM * kRedPitch;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
            *reinterpret_cast<f32x4 *>(mine + (16 * i + lr) * kRedPitch + 16 * j + 4 * lg) = acc[j][i];
    __syncthreads();
    // thread t sums BM*64/512 consecutive outputs of one row, in wave order;
    // rows beyond M are not stored
    constexpr int kPer = BM * kBN / kThreads;   // 8 (BM = 64) or 4 (BM = 32)
    const int e0 = tid * kPer;
    const int m = e0 / kBN, c0 = e0 % kBN;
    if (m >= M)
        return;
#pragma unroll
    for (int c = 0; c < kPer; c += 4) {
        f32x4 s = *reinterpret_cast<const f32x4 *>(red + m * kRedPitch + c0 + c);
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            s += *reinterpret_cast<const f32x4 *>(red + w * BM * kRedPitch + m * kRedPitch + c0 + c);
        f32x4 *p = reinterpret_cast<f32x4 *>(D + size_t(m) * N + n0 + c0 + c);
        if constexpr (BETA)
            s += *p;
        *p = s;
    }
}

template <bool BF16, int BM>
hipError_t launch_bm(const DenseArgs &a, hipStream_t stream)
{
    const uint8_t *A = static_cast<const uint8_t *>(a.A);
    const uint8_t *B = static_cast<const uint8_t *>(a.B);
    const dim3 grid(a.N / kBN);
    if (a.beta)
        hipLaunchKernelGGL((gemm_skinny_kernel<BF16, BM, true>), grid, dim3(kThreads), 0, stream, A, B, a.D,
                           a.M, a.N, a.K);
    else
        hipLaunchKernelGGL((gemm_skinny_kernel<BF16, BM, false>), grid, dim3(kThreads), 0, stream, A, B, a.D,
                           a.M, a.N, a.K);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(bool bf16, const DenseArgs &a, hipStream_t stream)
{
    if (a.M < 1 || a.M > 64)
        return hipErrorInvalidValue;
    if (a.M > 32)
        return bf16 ? launch_bm<true, 64>(a, stream) : launch_bm<false, 64>(a, stream);
    return bf16 ? launch_bm<true, 32>(a, stream) : launch_bm<false, 32>(a, stream);
}

}  // namespace mswz
