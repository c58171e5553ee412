// gemm256pp.hip — 256x256-tile GEMM for gfx950 with a ping-pong schedule:
// D = beta*D + A.B^T, fp16 / bf16, A and B K-major (tcgen05.mma page,
// "Operands and repeat axes" and the 128x64x64 example).
//
// Same tile, LDS layout, direct buffer-to-LDS copies and epilogue as
// gemm256_kernel.hpp (eight waves of 128x64 outputs, two waves per SIMD, two LDS
// stages), but the eight waves run in two groups, waves 0-3 (group 0) and
// waves 4-7 (group 1), so that the two waves on a SIMD (w and w+4) never
// issue MFMAs at the same time.  Each wave repeats four phases per K step k
// (stage s = k % 2):
//     L01  read the fragments of sub-steps 0 and 1 of step k from stage s,
//          issue this group's half of the copy of step k+1 into the other
//          stage (group 0: the A tile, group 1: the B tile)
//     C01  16 MFMAs on those fragments (no memory operations)
//     L23  read the fragments of sub-steps 2 and 3; then wait for this
//          wave's copies to land
//     C23  16 MFMAs
// and every phase ends at a workgroup barrier.  Group 1 runs one phase behind
// group 0 (it passes one extra barrier first, group 0 one extra at the end),
// so at every barrier-delimited interval one wave per SIMD computes while the
// other reads LDS and issues copies.  Hazards, in global phase numbers P
// (group 0 executes its position q at P = q, group 1 at P = q + 1):
//   * the stage of step k+1 was last read by group 1's L23(k-1) at
//     P = 4k-1, and every memory phase ends with all its LDS reads complete,
//     so the copies of step k+1 (group 0 at P = 4k, group 1 at P = 4k+1)
//     never overwrite unread data;
//   * those copies are first read at P = 4k+4 (group 0's L01(k+1)); group 0
//     waits for its copies at the end of its L23(k) (P = 4k+2), group 1 at
//     the end of its L23(k) (P = 4k+3): three phases of MFMA work each.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mswz {
namespace {

constexpr int kThreads = 512;
constexpr int kBM = 256, kBN = 256;
constexpr int kATile = kBM * 128, kStage = 2 * kATile;
constexpr int TM = 4, TN = 2;

// Direct-to-LDS copy of one 256-row K-major operand tile by the four waves
// of one group: group wave v (0..3) copies rows 8*(v + 4i) .. +7, i = 0..7;
// lane l takes row 8*(v + 4i) + l/8, layout key (l/8) ^ ((v + 4i) % 8).
struct GroupCopy {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t voff[2];   // even / odd i
    uint32_t row_bytes, lds_off;

    __device__ void init(const uint8_t *X, int row0, uint32_t rb, int v, int lane, uint32_t tile_off)
    {
        row_bytes = rb;
        rsrc = make_rsrc(X + size_t(row0) * rb, 256u * rb);
        const int r = 8 * v + (lane >> 3);
#pragma unroll
        for (int odd = 0; odd < 2; ++odd) {
            const int chunk = (lane & 7) ^ (((lane >> 3) ^ (v + 4 * odd)) & 7);
            voff[odd] = uint32_t(r) * rb + chunk * 16;
        }
        lds_off = tile_off + 8 * v * kTileRowBytes;
    }
    __device__ void issue(uint8_t *stage, int kt) const
    {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            buffer_load_lds16(rsrc, stage + lds_off + i * 32 * kTileRowBytes, voff[i & 1],
                              uint32_t(32 * i) * row_bytes + uint32_t(kt) * 128);
    }
};

// Barrier ending a phase; no instruction is moved across it in either
// direction, and all of this wave's LDS reads (and, with VM = 0, its copies)
// are complete when it is passed.
template <int VM>
__device__ __forceinline__ void phase_end()
{
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier_keep_vm<VM>();
    __builtin_amdgcn_sched_barrier(0);
}

template <bool BF16, bool BETA>
__global__ void __launch_bounds__(kThreads)
gemm256pp_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, float *__restrict__ D,
                 int M, int N, int K, int tiles_m, int tiles_n, int group_m)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage];
    (void)M;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = wave >> 2, v = wave & 3;
    const int lr = lane & 31, lh = lane >> 5;
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int wm = group * 128, wn = v * 64;
    const uint32_t row_bytes = uint32_t(K) * 2;
    const int KT = K / 64;   // even (the plan requires K % 128 == 0)

    // group 0 copies the A tile, group 1 the B tile
    GroupCopy cp;
    if (group == 0)
        cp.init(A, m0, row_bytes, v, lane, 0);
    else
        cp.init(B, n0, row_bytes, v, lane, kATile);

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

    u32x4 fa[2][TM], fb[2][TN];   // fragments of two sub-steps
    // sub-step ks reads chunk 2ks ^ lh of each fragment row (base XOR ks << 5)
    auto read2 = [&](const uint8_t *s, int ks0) {
        uint32_t ab[TM], bb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            ab[i] = opaque(abase[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            bb[j] = opaque(bbase[j]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                fa[h][i] = lds_read16(s, ab[i] ^ ((ks0 + h) << 5));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                fb[h][j] = lds_read16(s, bb[j] ^ ((ks0 + h) << 5));
        }
    };
    auto mma2 = [&]() {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    acc[j][i] = mfma_32x32x16<BF16>(fb[h][j], fa[h][i], acc[j][i]);
    };
    // one K step on stage s, copying step kc into the other stage during L01
    auto step = [&](uint8_t *s, uint8_t *other, int kc) {
        read2(s, 0);
        cp.issue(other, kc);
        phase_end<8>();   // L01: fragment reads done; this phase's copies stay in flight
        mma2();
        phase_end<8>();   // C01
        read2(s, 2);
        phase_end<0>();   // L23: fragments read and this wave's copies landed
        mma2();
        phase_end<0>();   // C23
    };

    // prologue: step 0 into lds0 (step k's L01 issues step k+1).  In the last
    // step the copy repeats step KT-1 into a stage that is not read again,
    // which keeps the loop body free of branches.
    cp.issue(lds0, 0);
    __syncthreads();
    if (group == 1)
        phase_end<0>();   // group 1 runs one phase behind

    for (int kt = 0; kt < KT; kt += 2) {
        step(lds0, lds1, kt + 1);
        step(lds1, lds0, min(kt + 2, KT - 1));
    }
    if (group == 0)
        phase_end<0>();   // balances group 1's extra barrier
    __syncthreads();      // no copy may still be writing LDS when the workgroup ends

#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const size_t m = size_t(m0 + wm + 32 * i + lr);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn + 32 * j + 8 * q + 4 * lh;
                f32x4 val = {acc[j][i][4 * q + 0], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                             acc[j][i][4 * q + 3]};
                f32x4 *p = reinterpret_cast<f32x4 *>(D + m * N + n);
                if constexpr (BETA)
                    val += *p;
                *p = val;
            }
        }
}

template <bool BF16>
hipError_t launch_bf(const DenseArgs &a, hipStream_t stream)
{
    const int tiles_m = a.M / kBM, tiles_n = a.N / kBN;
    const uint8_t *A = static_cast<const uint8_t *>(a.A);
    const uint8_t *B = static_cast<const uint8_t *>(a.B);
    if (a.beta)
        hipLaunchKernelGGL((gemm256pp_kernel<BF16, true>), dim3(tiles_m * tiles_n), dim3(kThreads), 0,
                           stream, A, B, a.D, a.M, a.N, a.K, tiles_m, tiles_n, a.group_m);
    else
        hipLaunchKernelGGL((gemm256pp_kernel<BF16, false>), dim3(tiles_m * tiles_n), dim3(kThreads), 0,
                           stream, A, B, a.D, a.M, a.N, a.K, tiles_m, tiles_n, a.group_m);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dense256pp(bool bf16, const DenseArgs &a, hipStream_t stream)
{
    return bf16 ? launch_bf<true>(a, stream) : launch_bf<false>(a, stream);
}

}  // namespace mswz
