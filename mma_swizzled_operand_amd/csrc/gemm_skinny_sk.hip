// gemm_skinny_sk.hip — weight-streaming GEMM with K split over workgroups:
//     D[M][N] = beta*D + A[M][K] . B[N][K]^T,  1 <= M <= 64, fp16 / bf16, K-major A and B
// (tcgen05.mma page, "Operands and repeat axes"; the weight-stationary
// workload of "Weight-stationary and block scaling").
//
// Why split K.  With 64 columns per workgroup (gemm_skinny.hip) every
// workgroup reads all of A (64 x K) for 64 x K of B: half of the bytes its
// loads move are A re-reads from L2, and those, not HBM, bound the kernel.  A
// workgroup here owns 256 columns and 1/S of K, so it reads 256 rows of B
// against 64 rows of A, and the N/256 x S workgroups still cover the chip.
//
// Workgroup (512 threads, 8 waves): column block cb (256 columns of D), K part
// `part`.  Every wave takes 32 of the 256 columns (two 16-row blocks of B) and
// all waves walk the part's 64-element K blocks together:
//   * A's K block (64 rows x 128 bytes) is copied global -> LDS with direct
//     16-byte buffer-to-LDS loads, one instruction per wave, into a ring of
//     kSlots stages (layout.hpp tile layout), kAhead = kSlots - 1 blocks
//     ahead; one barrier per block makes each stage visible and frees the
//     oldest one.  The stages are distinct LDS arrays and the K loop is
//     unrolled kSlots times, so the compiler sees which stage each copy
//     writes and never waits for copies into other stages before a read;
//   * B's fragments go straight from global memory into registers in the
//     16x16x32 operand form, kAhead blocks ahead (no LDS);
//   * the K order inside a 32-wide sub-step is kblk16 (gemm256_kernel.hpp), the same
//     for A and B, so the LDS fragment reads are free of bank conflicts.
//
// M is padded to 64 rows: A's copies carry the row in the range-checked
// per-lane offset and the buffer covers the M rows of A, so the rows beyond M
// land in LDS as zeros without a memory access; only rows below M are
// stored (partials and D).
//
// Reduction (deterministic, no waiting): each workgroup stores its 64 x 256
// fp32 partial into the caller's workspace; a second kernel
// (splitk_reduce_kernel) sums the S partials of every output in part order
// 0 .. S-1 and adds beta*D.  (An in-kernel reduction by the last workgroup of
// each column block, behind a counter, was measured: all workgroups finish
// streaming at about the same time, so its store acknowledgements, L2
// write-backs, atomic round trip and partial reads formed an exposed tail of
// ~16 us on 64 x 16384 x 8192, against ~6 us for the second kernel.)
#include <hip/hip_runtime.h>
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mswz {
namespace {

constexpr int kThreads = 512;
constexpr int kBM = 64;            // rows of the padded tile (M <= 64 rows of A and D)
constexpr int kBN = 256;           // columns of D per workgroup
constexpr int kSlots = 4;          // A stages and B register slots
constexpr int kAhead = kSlots - 1; // K blocks in flight ahead of the one computed
constexpr int kStageBytes = kBM * 128;


// The column-split streaming kernel: stores the workgroup's partial, which
// splitk_reduce_kernel then sums with the others.
template <bool BF16>
__global__ void __launch_bounds__(kThreads)
gemm_skinny_sk_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ B,
                      float *__restrict__ part_ws, int M, int N, int K, int S)
{
    __shared__ __attribute__((aligned(1024))) uint8_t st0[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t st3[kStageBytes];
    static_assert(kSlots == 4, "one named LDS array per stage");
    auto stage = [&](int u) { return u == 0 ? st0 : u == 1 ? st1 : u == 2 ? st2 : st3; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_cb = N / kBN;
    // consecutive workgroups take consecutive column blocks, so the S parts of
    // a column block run on the same XCD (workgroup b runs on XCD b % 8)
    const int cb = blockIdx.x % n_cb, part = blockIdx.x / n_cb;
    const int n0 = cb * kBN;
    const uint32_t row_bytes = uint32_t(K) * 2;
    const int T = K / 64 / S;          // K blocks of this part (a multiple of kSlots)
    const int kb0 = part * T;

    // ---- A: direct copy of one K block per step, wave w fills tile rows 8w .. 8w+7
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, uint32_t(M) * row_bytes);
    const int arow = 8 * wave + (lane >> 3);
    const uint32_t a_voff = uint32_t(arow) * row_bytes + 16u * uint32_t((lane & 7) ^ tile_key(arow));
    auto issue_a = [&](int slot, int t) {
        buffer_load_lds16(ra, stage(slot) + wave * 1024, a_voff, uint32_t(kb0 + t) * 128);
    };

    // ---- B: wave w owns rows 32w .. 32w+31 of the workgroup's 256; lane
    // (r, g) = (l % 16, l / 16) loads row r of a 16-row block, K chunk
    // 4s + kblk16(g) of sub-step s
    const int r16 = lane & 15, g = lane >> 4;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + size_t(n0) * row_bytes, uint32_t(kBN) * row_bytes);
    const uint32_t b_voff = uint32_t(32 * wave + r16) * row_bytes + 16u * uint32_t(kblk16(g));
    u32x4 bf[kSlots][2][2];   // [slot][16-row block][sub-step]
    auto issue_b = [&](int slot, int t) {
        const uint32_t k_off = uint32_t(kb0 + t) * 128;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                bf[slot][jb][s] = buffer_load16(rb, b_voff + 64 * s, k_off + uint32_t(16 * jb) * row_bytes);
    };

    // A fragment bases: 16-row block i, lane row 16i + r16, chunk kblk16(g)
    uint32_t abase[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * i + r16;
        abase[i] = uint32_t(row) * kTileRowBytes + (uint32_t(kblk16(g) ^ tile_key(row)) << 4);
    }

    f32x4 acc[2][4];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[jb][i] = f32x4{};

    // prologue: blocks 0 .. kAhead-1 into slots 0 .. kAhead-1
#pragma unroll
    for (int t = 0; t < kAhead; ++t) {
        issue_b(t, t);
        issue_a(t, t);
        sched_fence();
    }

    // Step t uses slot t % kSlots.  Wait until this wave's B loads and A copy
    // of block t have landed (the kAhead-1 younger steps' 5 operations each
    // may stay in flight), barrier (every wave's copy of block t is in LDS,
    // and every wave has finished reading slot (t-1) % kSlots, which the next
    // copy overwrites), MFMAs, then the loads of block t + kAhead into that
    // slot, clamped to the last block so that the loop has no branches (the
    // repeated loads are never used).
    for (int t0 = 0; t0 < T; t0 += kSlots) {
#pragma unroll
        for (int u = 0; u < kSlots; ++u) {
            const int t = t0 + u;
            lds_barrier_keep_vm<(kAhead - 1) * 5>();
            sched_fence();
            const uint8_t *st = stage(u);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                u32x4 af[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    af[i] = lds_read16(st, opaque(abase[i]) ^ uint32_t(s << 6));
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[jb][i] = mfma_16x16x32<BF16>(bf[u][jb][s], af[i], acc[jb][i]);
            }
            sched_fence();
            const int tn = min(t + kAhead, T - 1);
            issue_b((u + kAhead) % kSlots, tn);
            issue_a((u + kAhead) % kSlots, tn);
            sched_fence();
        }
    }
    // no copy may still be writing LDS when the workgroup ends
    lds_barrier_keep_vm<0>();

    // ---- partial -> workspace ([part][M][N]); lane holds row 16i + r16,
    // columns 32w + 16jb + 4g .. +3
    const size_t MN = size_t(M) * N;
    float *mine = part_ws + size_t(part) * MN;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (16 * i + r16 >= M)
                continue;
            const size_t idx = size_t(16 * i + r16) * N + n0 + 32 * wave + 16 * jb + 4 * g;
            *reinterpret_cast<f32x4 *>(mine + idx) = acc[jb][i];
        }
}

// K-sliced variant, used where a part holds 8 x KS K elements (KS = 128 or
// 256).  The workgroup covers the same 256 columns x K part as above, but its
// 8 waves split the part's K range instead of its columns: wave w owns the
// KS-element slice [w KS, (w+1) KS) of the part, keeps A's slice (MT 16-row
// blocks x KS) in registers for the whole kernel, and streams B in groups of
// 16 rows: group G is rows 16G .. 16G+15 of the 256, of which the wave loads
// its slice (16 rows x 2 KS bytes, one 16x16x32 operand fragment per load, K
// in natural order).  All 8 waves load group G at the same time, so each
// B row's whole K-part segment is requested together, which is what makes
// the streaming efficient from DRAM (the column-split kernel requests 128
// bytes of each of 256 rows per step, and from cold memory streams about 25 %
// slower).  Each load slot is reissued for group G+1 as soon as the MFMAs of
// group G have read it, so one group per wave stays in flight throughout.
// The 8 waves' 64 x 16 partials of group G are summed through LDS in wave
// order (double-buffered, one barrier per group; waves 0-3 reduce the even
// groups and 4-7 the odd ones); the sums are stored to the part's fp32
// partial after the last group, and splitk_reduce_kernel adds the parts as
// for the column-split kernel.
template <bool BF16, int MT, int KS>
__global__ void __launch_bounds__(kThreads)
gemm_skinny_ks_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ B,
                      float *__restrict__ part_ws, int M, int N, int K)
{
    static_assert(MT == 1 || MT == 2 || MT == 4, "16, 32 or 64 padded rows");
    static_assert(KS % 32 == 0 && KS <= 256, "whole 16x16x32 steps, A slice in registers");
    constexpr int kSteps = KS / 32;
    constexpr int kGroups = kBN / 16;
    constexpr int kRedBytes = 8 * MT * 64 * 16;   // one group: [wave][mt][lane] f32x4
    __shared__ __attribute__((aligned(16))) uint8_t red0[kRedBytes];
    __shared__ __attribute__((aligned(16))) uint8_t red1[kRedBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_cb = N / kBN;
    const int cb = blockIdx.x % n_cb, part = blockIdx.x / n_cb;
    const int n0 = cb * kBN;
    const uint32_t row_bytes = uint32_t(K) * 2;
    // byte offset of this wave's K slice within a row
    const uint32_t k_off = (uint32_t(part) * 8u + uint32_t(wave)) * uint32_t(KS) * 2u;
    const int r16 = lane & 15, g = lane >> 4;

    // B: lane (r16, g) of step s loads row 16G + r16, K elements 32s + 8g .. +7 of the slice
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + size_t(n0) * row_bytes, uint32_t(kBN) * row_bytes);
    const uint32_t b_voff = uint32_t(r16) * row_bytes + 16u * uint32_t(g);
    u32x4 bf[kSteps];
    auto issue_b = [&](int G, int s) {
        bf[s] = buffer_load16(rb, b_voff + 64u * uint32_t(s), k_off + uint32_t(16 * G) * row_bytes);
    };
    // A: row 16 mt + r16 (rows >= M lie beyond the buffer's range and read as
    // zeros).  Loaded step by step with group 0's B fragments, in the order the
    // first group's MFMAs use them, so that they start before all of A is in.
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, uint32_t(M) * row_bytes);
    u32x4 af[MT][kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        issue_b(0, s);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            af[mt][s] = buffer_load16(ra, uint32_t(16 * mt + r16) * row_bytes + 16u * uint32_t(g) + 64u * uint32_t(s),
                                      k_off);
    }
    sched_fence();

    // The reducing waves keep their groups' sums in registers and store them
    // after the last group: stores issued during the streaming cost more than
    // their bytes (each one is waited for at the next barrier, and the writes
    // interleave with the stream's reads in DRAM).
    f32x4 sums[kGroups / 2];
    // One group: MFMAs step by step, each step's load slot reissued for group
    // G+1 right after its MFMAs (NEXT), partials to LDS, barrier, and the
    // reducing waves' fixed-order sum.
    auto group = [&](int G, uint8_t *red, int red_wave0, auto next) {
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            acc[mt] = f32x4{};
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = mfma_16x16x32<BF16>(bf[s], af[mt][s], acc[mt]);
            if constexpr (decltype(next)::value)
                issue_b(G + 1, s);
            sched_fence();
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            *reinterpret_cast<f32x4 *>(red + ((wave * MT + mt) * 64 + lane) * 16) = acc[mt];
        // the partials are in LDS; the next group's loads stay in flight
        lds_barrier_keep_vm<decltype(next)::value ? kSteps : 0>();
        const int mt = wave - red_wave0;
        if (mt >= 0 && mt < MT) {
            f32x4 v[8];
#pragma unroll
            for (int w = 0; w < 8; ++w)
                v[w] = *reinterpret_cast<const f32x4 *>(red + ((w * MT + mt) * 64 + lane) * 16);
            sched_fence();
            f32x4 sum = v[0];
#pragma unroll
            for (int w = 1; w < 8; ++w)
                sum += v[w];
            sums[G >> 1] = sum;
        }
    };
    // Group G's LDS buffer is rewritten by group G+2 only after the barrier of
    // group G+1, which every wave reaches after its reads of group G.
    // (unrolled in full, so that every index into sums is a constant)
    using yes = std::true_type;
#pragma unroll
    for (int G = 0; G < kGroups - 2; G += 2) {
        group(G, red0, 0, yes{});
        group(G + 1, red1, 4, yes{});
    }
    group(kGroups - 2, red0, 0, yes{});
    group(kGroups - 1, red1, 4, std::false_type{});

    // wave w reduced the groups of parity w / 4 for 16-row block w % 4: lane
    // holds row 16 mt + r16, columns 16G + 4g .. +3 of the workgroup's block
    const int mt = wave & 3, odd = wave >> 2;
    const int m = 16 * mt + r16;
    if (mt < MT && m < M) {
        float *const mine = part_ws + size_t(part) * size_t(M) * N + size_t(m) * N + n0 + 4 * g;
#pragma unroll
        for (int h = 0; h < kGroups / 2; ++h)
            *reinterpret_cast<f32x4 *>(mine + 16 * (2 * h + odd)) = sums[h];
    }
}

// Second pass of the two-kernel reduction: D = sum_p partial[p] (+ D), the S
// partials added in part order, one 16-byte group of outputs per thread.
template <bool BETA>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float *__restrict__ part_ws, float *__restrict__ D, int64_t n4, int S)
{
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n4)
        return;
    const f32x4 *p = reinterpret_cast<const f32x4 *>(part_ws) + i;
    f32x4 sum = p[0];
    for (int s = 1; s < S; ++s)
        sum += p[int64_t(s) * n4];
    f32x4 *d = reinterpret_cast<f32x4 *>(D) + i;
    if constexpr (BETA)
        sum += *d;
    // streamed to memory (consecutive threads write whole lines): 1 us less
    // per 64 x 16384 call than plain stores; the partials, read again right
    // after, are stored plainly
    __builtin_nontemporal_store(sum, d);
}

template <bool BF16, int MT>
void launch_ks(const DenseArgs &a, const SplitK &sk, hipStream_t stream)
{
    const uint8_t *A = static_cast<const uint8_t *>(a.A);
    const uint8_t *B = static_cast<const uint8_t *>(a.B);
    const dim3 grid(a.N / kBN * sk.parts);
    if (a.K / sk.parts == 8 * 256)
        hipLaunchKernelGGL((gemm_skinny_ks_kernel<BF16, MT, 256>), grid, dim3(kThreads), 0, stream, A, B,
                           sk.partials, a.M, a.N, a.K);
    else
        hipLaunchKernelGGL((gemm_skinny_ks_kernel<BF16, MT, 128>), grid, dim3(kThreads), 0, stream, A, B,
                           sk.partials, a.M, a.N, a.K);
}

// The K-sliced kernel wherever a part holds 2048 or 1024 K elements, the
// column-split kernel elsewhere; then the reduction.
template <bool BF16, bool BETA>
hipError_t launch_bb(const DenseArgs &a, const SplitK &sk, hipStream_t stream)
{
    const uint8_t *A = static_cast<const uint8_t *>(a.A);
    const uint8_t *B = static_cast<const uint8_t *>(a.B);
    const dim3 grid(a.N / kBN * sk.parts);
    const int kpart = a.K / sk.parts;
    if (kpart == 8 * 256 || kpart == 8 * 128) {
        if (a.M <= 16)
            launch_ks<BF16, 1>(a, sk, stream);
        else if (a.M <= 32)
            launch_ks<BF16, 2>(a, sk, stream);
        else
            launch_ks<BF16, 4>(a, sk, stream);
    } else {
        hipLaunchKernelGGL((gemm_skinny_sk_kernel<BF16>), grid, dim3(kThreads), 0, stream, A, B, sk.partials,
                           a.M, a.N, a.K, sk.parts);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t n4 = int64_t(a.M) * a.N / 4;
    hipLaunchKernelGGL((splitk_reduce_kernel<BETA>), dim3(unsigned((n4 + 255) / 256)), dim3(256), 0, stream,
                       sk.partials, a.D, n4, sk.parts);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_bf(const DenseArgs &a, const SplitK &sk, hipStream_t stream)
{
    return a.beta ? launch_bb<BF16, true>(a, sk, stream) : launch_bb<BF16, false>(a, sk, stream);
}

}  // namespace

// K parts: the smallest power of two up to 16 that gives at least 256
// workgroups, else the largest one that fits K; each part must hold a
// multiple of kSlots 64-element K blocks.
int skinny_split_parts(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || M > kBM || N % kBN != 0)
        return 0;
    const int64_t n_cb = N / kBN;
    int best = 0;
    for (int s = 2; s <= 16; s *= 2) {
        if (K % (int64_t(64) * kSlots * s) != 0)
            continue;
        best = s;
        if (n_cb * s >= 256)
            break;
    }
    return best;
}

int64_t skinny_split_workspace_bytes(int64_t M, int64_t N, int parts)
{
    return int64_t(parts) * M * N * 4;   // the fp32 partials
}

hipError_t launch_skinny_split(bool bf16, const DenseArgs &a, void *workspace, hipStream_t stream)
{
    SplitK sk;
    sk.parts = skinny_split_parts(a.M, a.N, a.K);
    if (!sk.parts)
        return hipErrorInvalidValue;
    sk.partials = static_cast<float *>(workspace);
    return bf16 ? launch_bf<true>(a, sk, stream) : launch_bf<false>(a, sk, stream);
}

}  // namespace mswz
