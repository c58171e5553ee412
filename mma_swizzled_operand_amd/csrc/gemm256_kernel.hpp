// gemm256_kernel.hpp — the large-tile GEMM kernel for gfx950, included by the
// translation units that instantiate it (gemm256_*.hip): one 512-thread
// workgroup (8 waves, two per SIMD) computes a 256 x 256 tile of
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
// that belongs at its destination: chunk (l % 8) ^ key(row).  An MN-major
// operand ([K][M] or [K][N]) is copied the same way into an MN-major tile (64
// K rows of 512 bytes, chunks XOR-permuted by K row) and its MFMA fragments
// are read with gfx950's transposing LDS reads, which hand each lane one M
// (or N) row with four consecutive K values.
// Scale bytes (MX) for the step's 256 A rows and 256 B rows are copied into a
// small LDS stage by direct 4-byte loads, one wave instruction per 64 rows.
//
// Compute.  Wave w owns output rows 128*(w/4) .. +127 and columns 64*(w%4)
// .. +63, 128 fp32 accumulators per lane: 8 x 4 blocks of 16x16x32 MFMA
// output for 16-bit operands (4 x 2 blocks of 32x32x16 when both are
// MN-major), 8 x 4 blocks of the scaled 16x16x128 MFMA for the block-scaled
// kinds.  The
// 16x16 shape moves fewer register bytes per flop than the 32x32 one; under
// the chip's power limit it runs at a higher clock and is faster overall.
// The MFMA's first operand is the B fragment and its second the A fragment,
// so four consecutive accumulator registers hold four consecutive N columns
// of one M row and the epilogue stores 16 bytes per lane.
#pragma once
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace mswz {
namespace {

constexpr int kBM = 256, kBN = 256;
constexpr int kATile = kBM * 128, kBTile = kBN * 128, kStage = kATile + kBTile;
constexpr int kScaleStage = (kBM + kBN) * 16;  // up to 16 scale bytes (four K steps) per row
// grouped scale copies of 32 bytes per row (eight E4M3 / padded K steps or
// four E2M1 steps; layout.hpp sf_wide_offset)
constexpr int kScaleStageWide = (kBM + kBN) * 32;
// MN-major scales in the wide stage: A's 32 K blocks of 256 rows
// (sf_mn_offset), then B's
constexpr uint32_t kSfMnB = uint32_t(kBM) * 32;
static_assert(kScaleStageWide == 2 * int(kSfMnB) && kBM == 256 && kBN == 256, "two 8 KiB halves");


// kE2m1p: E2M1 in the padded sixteen-per-16-byte form (eight bytes of nibbles,
// eight of padding), with the byte layout of E4M3 and the 6-bit kinds
enum Kind { kBf16 = 0, kF16 = 1, kE4m3 = 2, kE2m1 = 3, kE2m3 = 4, kE3m2 = 5, kE2m1p = 6 };

// Direct-to-LDS copy of one K-major operand tile (256 rows x 128 bytes per K
// step) through a buffer resource on the workgroup's 256-row panel.  With W
// waves, wave w copies rows 8*(w + W*i) .. +7 for i = 0 .. 32/W - 1; lane l
// takes row 8*(w + W*i) + l/8, whose layout key is (l/8) ^ ((w + W*i) % 8), so
// it fetches chunk (l % 8) ^ (l/8) ^ ((w + W*i) % 8).
//
// The row is part of the per-lane offset, which the buffer's range check
// covers (the scalar offset, here only the K step, is not checked), so in a
// tail panel the rows beyond the operand read as zeros and no address beyond
// the operand is formed.
template <int W>
struct DmaOperand {
    static constexpr int kInstr = 32 / W;
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t voff[kInstr];   // this lane's byte offset in the panel at K step 0, per instruction
    uint32_t lds_off;        // LDS offset of this wave's first destination row inside a stage
    uint32_t nbytes;         // the buffer's range: bytes of the panel inside the operand

    // rows: rows of the panel inside the operand (fewer than 256 in a tail panel)
    __device__ void init(const uint8_t *X, int row0, int rows, uint32_t rb, int wave, int lane,
                         uint32_t tile_off)
    {
        nbytes = uint32_t(rows) * rb;
        rsrc = make_rsrc(X + size_t(row0) * rb, nbytes);
#pragma unroll
        for (int i = 0; i < kInstr; ++i)
            voff[i] = dma_row(wave + W * i, lane) * rb + dma_chunk(wave + W * i, lane) * 16;
        lds_off = tile_off + 8 * wave * kTileRowBytes;
    }

    __device__ void issue(uint8_t *stage, int kt) const
    {
#pragma unroll
        for (int i = 0; i < kInstr; ++i)
            buffer_load_lds16(rsrc, stage + lds_off + i * 8 * W * kTileRowBytes, voff[i], uint32_t(kt) * 128);
    }

    // instructions [half * kInstr / 2, (half + 1) * kInstr / 2) of issue()
    __device__ void issue_half(uint8_t *stage, int kt, int half) const
    {
#pragma unroll
        for (int i = 0; i < kInstr / 2; ++i) {
            const int q = half * (kInstr / 2) + i;
            buffer_load_lds16(rsrc, stage + lds_off + q * 8 * W * kTileRowBytes, voff[q], uint32_t(kt) * 128);
        }
    }

    // The partial last K step kt of a K that is not a multiple of the step:
    // only the first `lim` bytes of each row's 128-byte slice lie inside K (a
    // multiple of 16, so chunks are whole).  The whole offset goes into the
    // range-checked per-lane offset and a chunk beyond K points at the end
    // of the range, so it reads as zeros without forming an address outside
    // the operand.
    __device__ void issue_tail(uint8_t *stage, int kt, uint32_t lim, int wave, int lane) const
    {
#pragma unroll
        for (int i = 0; i < kInstr; ++i) {
            const uint32_t off = 16 * dma_chunk(wave + W * i, lane) < lim ? voff[i] + uint32_t(kt) * 128 : nbytes;
            buffer_load_lds16(rsrc, stage + lds_off + i * 8 * W * kTileRowBytes, off, 0);
        }
    }
};

// Direct-to-LDS copy of one MN-major 16-bit operand ([K][R] storage, R = M
// or N) for a 256-wide tile.  The step's tile is 64 K rows of 512 bytes (256
// values); 16-byte chunk c of K row k (values 8c .. 8c+7) sits at position
// c ^ mn_key(k) of the row, mn_key(k) = 4 * (k % 4) ^ 2 * ((k / 16) % 2).
// Wave instruction q = w + W*i fills K rows 2q and 2q+1, lane l writing
// position l % 32 of row k = 2q + l/32, so it fetches chunk
// (l % 32) ^ mn_key(k).  Since 2w + l/32 < 2W and 2W*i is a multiple of 2W,
// k % 4 comes from the lane and wave only and bit 4 of k from i only.  The
// fragments are read back with transposing LDS reads (mn_frag_base below).
template <int W>
struct DmaMnOperand {
    static constexpr int kInstr = 32 / W;
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t voff[2], pitch, lds_off;   // voff[bit 4 of the instruction's K rows]
    uint32_t nbytes;                    // the buffer's range

    // A chunk whose columns lie beyond the operand (a tail tile) is fetched
    // from the tile's first columns instead: its values only reach outputs
    // beyond M or N, and every address stays inside the operand.
    // ld: elements from one K row of the operand to the next (>= R)
    __device__ void init(const uint8_t *X, int R, int ld, int row0, int K, int wave, int lane,
                         uint32_t tile_off)
    {
        pitch = uint32_t(ld) * 2;
        nbytes = uint32_t(K - 1) * pitch + uint32_t(R - row0) * 2;
        rsrc = make_rsrc(X + size_t(row0) * 2, nbytes);
        const int kr = lane >> 5;
#pragma unroll
        for (int b4 = 0; b4 < 2; ++b4) {
            // instructions q = wave + W*i with i % 2 == b4 (bit 4 of their K rows)
            const int c = int(dma_mn_chunk(wave + W * b4, lane));
            const int cs = row0 + 8 * c < R ? c : 0;
            voff[b4] = uint32_t(2 * wave + kr) * pitch + 16 * cs;
        }
        lds_off = tile_off + 2 * wave * kMnRowBytes;
    }
    __device__ void issue(uint8_t *stage, int kt) const
    {
#pragma unroll
        for (int i = 0; i < kInstr; ++i)
            buffer_load_lds16(rsrc, stage + lds_off + i * 2 * W * kMnRowBytes, voff[((2 * W * i) >> 4) & 1],
                              (uint32_t(kt) * 64 + 2 * W * i) * pitch);
    }

    // The partial last K step kt: K rows at or beyond K read as zeros.  The
    // whole offset goes into the range-checked per-lane offset and a row
    // beyond K points at the end of the range, so no address outside the
    // operand is formed.
    __device__ void issue_tail(uint8_t *stage, int kt, int K, int wave, int lane) const
    {
#pragma unroll
        for (int i = 0; i < kInstr; ++i) {
            const int k = 64 * kt + 2 * (wave + W * i) + (lane >> 5);
            const uint32_t off = k < K ? voff[((2 * W * i) >> 4) & 1] + (uint32_t(kt) * 64 + 2 * W * i) * pitch
                                       : nbytes;
            buffer_load_lds16(rsrc, stage + lds_off + i * 2 * W * kMnRowBytes, off, 0);
        }
    }
};

// MFMA format code of a block-scaled element kind (E4M3 0, E2M3 2, E3M2 3,
// E2M1 4).
template <int KIND_>
constexpr int mx_format()
{
    return KIND_ == kE3m2 ? 3 : KIND_ == kE2m3 ? 2 : (KIND_ == kE2m1 || KIND_ == kE2m1p) ? 4 : 0;
}

// Padded sub-byte kinds (6-bit, and 4-bit in the padded form): sixteen values
// per 16-byte chunk, a lane's 32 values all in one scale block (the FP4
// operand image has the block structure of the FP6 one: lane (row i, group g)
// holds values j at bits 4j of registers 0..3, all in block g).
constexpr bool padded_kind(int k) { return k == kE2m3 || k == kE3m2 || k == kE2m1p; }
constexpr bool byte_row_kind(int k) { return k == kE4m3 || padded_kind(k); }

// Compile-time loop: fn(std::integral_constant<int, F>), ..., up to L - 1.
template <int F, int L, class Fn>
__device__ __forceinline__ void static_for(Fn &&fn)
{
    if constexpr (F < L) {
        fn(std::integral_constant<int, F>{});
        static_for<F + 1, L>(fn);
    }
}

// Read order of one K step's fragments for a TM x TN grid of 16x16 MFMAs
// issued A-block-major (MFMA m = TN * i + j): every A block i and B block j
// is read before the first MFMA that uses it (MFMA TN * i, resp. j), in the
// order of that first use, and `ahead` MFMAs early.  issued(m) counts the
// reads issued before MFMA m + 1; item(r) names read r: i + 1 for A block i,
// -(j + 1) for B block j.
template <int TM, int TN, int ahead>
struct FragSchedule {
    static constexpr int issued(int m)
    {
        int c = 0;
        for (int i = 0; i < TM; ++i)
            c += TN * i <= m + ahead;
        for (int j = 0; j < TN; ++j)
            c += j <= m + ahead;
        return c;
    }
    static constexpr int item(int r)
    {
        int ia = 0, ib = 0;
        for (int k = 0; k < TM + TN; ++k) {
            const int na = ia < TM ? TN * ia : 1 << 20, nb = ib < TN ? ib : 1 << 20;
            if (na <= nb) {
                if (k == r)
                    return ia + 1;
                ++ia;
            } else {
                if (k == r)
                    return -(ib + 1);
                ++ib;
            }
        }
        return 0;
    }
};

// Four consecutive outputs of one row of D, as fp32 or rounded to nearest
// even into bf16 / fp16 (OUT, see OutKind); with BETA the old values, read in
// the same kind, are added first.
// NT: non-temporal stores, for epilogues whose store instructions cover
// whole 64-byte pieces of D rows (16 lanes x 16 bytes of four consecutive
// lanes per row); the others leave their smaller pieces to be merged into
// lines in L2.
template <int OUT, bool BETA, bool NT = false>
__device__ __forceinline__ void store_d4(void *D, size_t idx, f32x4 v, bool sat = false)
{
    // largest finite magnitude of D's format (sat: larger magnitudes, infinities
    // included, are stored as it with their sign; NaN passes unchanged)
    constexpr float kMax = OUT == kOutF32 ? 3.40282347e38f : OUT == kOutBf16 ? 3.38953139e38f : 65504.0f;
    auto clamp = [&](f32x4 &x) {
        if (sat) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[e] = __builtin_fabsf(x[e]) > kMax ? __builtin_copysignf(kMax, x[e]) : x[e];
        }
    };
    // Non-temporal stores stream D to memory without taking L2 / MALL lines
    // from the operand panels that the other tiles still read (8192^3 bf16:
    // 6 % faster than plain stores, 4096^3 bf16 2 %, 8192^3 E2M1 4 %).  For
    // 32-byte pieces per row they are 14-18 % slower (E4M3, padded 6-bit).
    if constexpr (OUT == kOutF32) {
        f32x4 *p = reinterpret_cast<f32x4 *>(static_cast<float *>(D) + idx);
        if constexpr (BETA)
            v += *p;
        clamp(v);
        if constexpr (NT)
            __builtin_nontemporal_store(v, p);
        else
            *p = v;
    } else {
        using T = std::conditional_t<OUT == kOutBf16, __bf16, _Float16>;
        typedef T t4 __attribute__((ext_vector_type(4)));
        t4 *p = reinterpret_cast<t4 *>(static_cast<T *>(D) + idx);
        if constexpr (BETA) {
            const t4 old = *p;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] += float(old[e]);
        }
        clamp(v);
        t4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            out[e] = T(v[e]);
        if constexpr (NT)
            __builtin_nontemporal_store(out, p);
        else
            *p = out;
    }
}

// Four consecutive outputs of D read in D's format, as fp32 (the old D of
// beta = 1, loaded ahead of its store so that the loads of several pieces
// are in flight together).
template <int OUT>
__device__ __forceinline__ f32x4 load_d4(const void *D, size_t idx)
{
    if constexpr (OUT == kOutF32) {
        return *reinterpret_cast<const f32x4 *>(static_cast<const float *>(D) + idx);
    } else {
        using T = std::conditional_t<OUT == kOutBf16, __bf16, _Float16>;
        typedef T t4 __attribute__((ext_vector_type(4)));
        const t4 old = *reinterpret_cast<const t4 *>(static_cast<const T *>(D) + idx);
        return f32x4{float(old[0]), float(old[1]), float(old[2]), float(old[3])};
    }
}

// The epilogue options applied to four outputs of row m, columns n .. n+3
// before they are stored: false if row m is masked out (not stored at all).
__device__ __forceinline__ bool apply_opts(const EpiOpts &o, int m, int n, f32x4 &v)
{
    if (o.row_mask && ((o.row_mask[m >> 5] >> (m & 31)) & 1u))
        return false;
    if (o.col_zero) {
        const uint32_t w = o.col_zero[n >> 5] >> (n & 31);   // n % 4 == 0: the four bits share a word
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if ((w >> e) & 1u)
                v[e] = 0.0f;
    }
    if (o.neg)
        v = -v;
    return true;
}

// Eight waves per workgroup, each owning a 128 x 64 output sub-tile (two
// waves per SIMD).
constexpr int W = 8;

// KIND: element kind of A (and of B unless KB >= 0); KB: B's kind when it
// differs (block-scaled E4M3 / E2M3 / E3M2 / padded E2M1 among themselves,
// or E4M3 with dense E2M1 on either side); SV: K
// elements per scale byte (32, or 16 for E2M1 and the padded kinds); MF16:
// 16x16 MFMAs (every kind), else 32x32x16 (16-bit operands, both MN-major);
// SB: block-scaled K that is not a multiple of the K step (scale bytes
// assembled in registers, see below); SM: scales stored MN-major,
// SFA [K/SV][M] and SFB [K/SV][N] (the wide-stage kinds, K a multiple of the
// K step, M and N multiples of 16); WO: K a multiple of 2048, only the wide
// loop compiled (with SM and not WO: only the per-step loop).
template <int KIND, bool A_MN, bool B_MN, bool BETA, bool MF16, int OUT = kOutF32, int KB = -1, int SV = 32,
          bool SB = false, bool SM = false, bool WO = false>
__global__ void __launch_bounds__(64 * W)
gemm256_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ B,
               const uint8_t *__restrict__ SFA, const uint8_t *__restrict__ SFB,
               void *__restrict__ D, int M, int N, int K, int lda, int ldb, int ldd, int tiles_m,
               int tiles_n, int group_m, EpiOpts opts)
{
    static_assert(!((A_MN || B_MN) && KIND != kBf16 && KIND != kF16), "MN-major operands are built for 16-bit only");
    constexpr int TM = 4, TN = 2;                // 32x32 blocks per wave along M and N
    constexpr int kWavesN = 256 / (32 * TN);     // waves along N
    constexpr int kKindB = KB < 0 ? KIND : KB;
    constexpr bool kMixed = kKindB != KIND;
    // E4M3 paired with dense E2M1 (compute_pair): kPairB with E2M1 as B,
    // kPairA with E2M1 as A
    constexpr bool kPairB = KIND == kE4m3 && kKindB == kE2m1, kPairA = KIND == kE2m1 && kKindB == kE4m3;
    constexpr bool kPair = kPairA || kPairB;
    static_assert(!kMixed || kPair || (byte_row_kind(KIND) && byte_row_kind(kKindB)),
                  "mixed operand kinds: E4M3 and the padded 6- and 4-bit kinds, or E4M3 with dense E2M1");
    constexpr bool kFp6B = padded_kind(kKindB);
    // A's kind below; B's differs only in the fragment reads and the MFMA format.
    // kFp6: a padded sub-byte kind (E2M3, E3M2 or padded E2M1).
    constexpr bool kFp8 = KIND == kE4m3 && !kPair, kFp4 = KIND == kE2m1 && !kPair, kFp6 = padded_kind(KIND);
    constexpr bool kMx = kFp8 || kFp4 || kFp6 || kPair;
    // E4M3 and padded 6-bit operands share the byte layout (128 values per
    // 128-byte row step) and the split-row fragments
    constexpr bool kByteRows = kFp8 || kFp6;
    // split-row fragments on A's and on B's side (row16<true>): the output
    // rows and columns follow them
    constexpr bool kRowsA = kPair ? kPairB : kByteRows, kRowsB = kPair ? kPairA : kByteRows;
    static_assert(!kMx || MF16, "block-scaled kinds are built for the 16x16 MFMA");
    // 16-element scale blocks: a lane's 32 values of a 32-block are two
    // 16-element halves (one 16-byte chunk of a padded kind, or the two 8-byte
    // halves of a dense E2M1 chunk), so each 16x16 block takes two MFMAs, each
    // with one half (the other zero) and that half's scales
    constexpr bool kV16 = SV == 16;
    static_assert(SV == 32 || (kV16 && (kFp4 || kFp6) && !kMixed), "16-element blocks: E2M1 and padded kinds");
    // one step moves 128 bytes of every tile row: 64 16-bit, 128 E4M3 or 256
    // E2M1 (packed two per byte) K elements
    // (with kPair the E4M3 operand's 128; the E2M1 operand's 128-byte rows
    // then hold two steps)
    constexpr int kStepK = kPair ? 128 : kFp4 ? 256 : kByteRows ? 128 : 64;
    constexpr int kStepA = kPairA ? 256 : kStepK, kStepB = kPairB ? 256 : kStepK;

    // the grouped scale copies (below) with 32-element blocks, for one kind
    // on both sides (with MN-major scales, whose kernels have one loop, for
    // every byte-row kind, mix and D): their stages hold 32 bytes per row (2 x 64 KiB of
    // operand stages + 2 x 16 KiB).  (With two different kinds the wide loop
    // left the kernels short of registers, up to 21 spilled and reloaded
    // every step; an E4M3 A (alone or with a 6-bit or padded 4-bit B) fits
    // with fp32 D under the scheduling strategy of its units,
    // gemm256_e4m3_f32.hip and gemm256_mixed_e4m3_f32.hip, and keeps the
    // 16-byte groups otherwise.)
    constexpr bool kWideStage =
        ((kByteRows && (!kMixed || KIND == kE4m3 || SM) && (KIND != kE4m3 || OUT == kOutF32 || SM)) || kFp4) && !kV16 && !SB;
    static_assert(!SM || kWideStage || (kPair && !WO), "MN-major scales: the wide scale stage (pairs: per step)");
    // only the 32-K-block loop (K % 2048 == 0, checked by the host): without
    // the fallback loops the kernels keep more registers for the K loop
    constexpr bool kWideOnly = WO;
    static_assert(!kWideOnly || kWideStage, "wide-only kernels: the wide scale stage");
    // MN-major scales for other K: the per-step loop alone, each step's
    // scales of 256 rows copied as one (E2M1: two) 1 KiB instruction per
    // operand into the wide stage's first K blocks
    constexpr bool kMnStep = SM && !WO;
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage];
    __shared__ __attribute__((aligned(256))) uint8_t scl0[!kMx ? 4 : kWideStage || SM ? kScaleStageWide : kScaleStage];
    __shared__ __attribute__((aligned(256))) uint8_t scl1[!kMx ? 4 : kWideStage || SM ? kScaleStageWide : kScaleStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, lh = lane >> 5;
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int wm = (wave / kWavesN) * 128, wn = (wave % kWavesN) * (32 * TN);
    // bytes from one K-major operand row to the next (lda, ldb are in elements)
    const uint32_t a_row_bytes = uint32_t(lda) * 128 / kStepA, b_row_bytes = uint32_t(ldb) * 128 / kStepB;
    const int KT = K / kStepK;
    // M and N need not be multiples of 256: a tail tile reads zeros (K-major
    // rows beyond the operand, through the buffer range) or values that only
    // reach outputs beyond M or N (MN-major), and the epilogue stores only
    // outputs inside D
    const int rows_a = min(kBM, M - m0), rows_b = min(kBN, N - n0);

    // ---- operand copies ---------------------------------------------------------
    // K-major operands are copied straight into the K-major LDS tile;
    // MN-major operands straight into an MN-major LDS tile, read back with
    // transposing LDS reads.
    constexpr bool kDmaA = !A_MN, kDmaB = !B_MN;
    constexpr bool kTrA = A_MN, kTrB = B_MN;
    DmaOperand<W> da, db;
    if constexpr (kDmaA)
        da.init(A, m0, rows_a, a_row_bytes, wave, lane, 0);
    if constexpr (kDmaB)
        db.init(B, n0, rows_b, b_row_bytes, wave, lane, kATile);
    DmaMnOperand<W> dma_mna, dma_mnb;
    if constexpr (kTrA)
        dma_mna.init(A, M, lda, m0, K, wave, lane, 0);
    if constexpr (kTrB)
        dma_mnb.init(B, N, ldb, n0, K, wave, lane, kATile);

    // ---- scale copies (MX): 64-row group g = 0..7 (A rows for g < 4, B rows
    // for g >= 4) is copied by wave g % W.  Per K step (kScaleGroups false):
    // lane l copies the step's 32-bit scale word of row 64*(g%4) + l into
    // scale-stage word 64*g + l.  Per group of four K steps (kScaleGroups, the
    // 16x16 path with eight waves and K a multiple of 1024): lane l copies the
    // 16 scale bytes of the four steps of row 64*(g%4) + sf_slot_row(l) into
    // stage bytes 16*(64g + l) .. +15 (the slot order makes a fragment
    // block's 16 rows consecutive slots, whose byte reads conflict two-way and
    // no more).  A row's scales for one step are only 4 bytes and consecutive rows
    // are K/32 bytes apart, so a per-step copy touches one cache line per lane
    // for 4 useful bytes; fetching four steps at once cuts those line accesses
    // fourfold, and they cost as much address-unit time as the operand copies.
    constexpr bool kScaleGroups = kByteRows && !kV16 && !SB && !kPair;   // E4M3 and the padded kinds, 32-element blocks
    // dense E2M1 with 32-element blocks: the same 16-byte copies per row,
    // which hold two of its K steps (two scale words per row per step), in
    // natural row order
    constexpr bool kFp4Groups = kFp4 && !kV16 && !SB;
    constexpr int kSfInstr = 8 / W;
    const uint32_t sf_row = uint32_t(K) / SV;
    __amdgpu_buffer_rsrc_t sf_rsrc[kSfInstr];
    uint32_t sf_voff = 0;
    if constexpr (kMx) {
#pragma unroll
        for (int q = 0; q < kSfInstr; ++q) {
            const int g = wave + W * q;
            const bool is_b = g >= 4;
            if constexpr (SM)
                // [K block][row] with M (N) bytes per K block: from the tile's
                // first row to the end of the array.  Rows beyond M or N read
                // the next K block's first rows (or zeros past the end), which
                // only reach outputs that are not stored.
                sf_rsrc[q] = make_rsrc((is_b ? SFB : SFA) + (is_b ? n0 : m0),
                                       sf_row * uint32_t(is_b ? N : M) - uint32_t(is_b ? n0 : m0));
            else
                sf_rsrc[q] = make_rsrc((is_b ? SFB : SFA) + size_t(is_b ? n0 : m0) * sf_row,
                                       uint32_t(is_b ? rows_b : rows_a) * sf_row);
        }
        // with kScaleGroups lane l copies row sf_slot_row(l) of its group
        sf_voff = uint32_t(64 * (wave & 3) + (kScaleGroups ? sf_slot_row(lane) : lane)) * sf_row;
    }
    // Wide groups (kWideStage: one block-scaled kind on both sides, K a
    // multiple of 2048): 32 bytes per row and group (eight E4M3 or padded or
    // four E2M1 steps), two copies per wave and group.
    // Copy q of wave g fetches rows of slots 32q .. 32q+31 of its 64-row group
    // (slot order as above), lane l the half l/32 of slot 32q + l%32, so both
    // halves of a row come from one cache line in one instruction, and
    // writes 1 KiB of consecutive LDS (sf_wide_offset).  A grouped copy of 16
    // bytes per row touches a cache line per lane for 16 useful bytes; per K
    // step the wide copies make half as many line requests, which are what
    // the copy path's time is spent on.
    // (sf_slot_row keeps bit 5, so copy 1's rows are copy 0's plus 32: one
    // per-lane offset, the second copy 32 rows further through the scalar
    // offset)
    // With MN-major scales (SM) copy q of wave w is instruction i = 2 (w%4) + q
    // of its operand's stage half: K blocks 4i .. 4i+3 of the group, all 256
    // rows, lane l the chunk of sf_mn_copy_block / sf_mn_copy_row (a per-lane
    // offset; the instruction's K blocks through the scalar offset).
    uint32_t sf_voff_w = 0;
    const uint32_t sf_pitch = SM ? uint32_t(wave < 4 ? M : N) : 0u;   // bytes per K block (SM)
    if constexpr (kWideStage || SM) {
        static_assert(kSfInstr == 1, "one 64-row scale group per wave");
        static_assert(sf_slot_row(32 + 5) == 32 + sf_slot_row(5), "slot order keeps bit 5");
        const int slot = lane & 31;
        if constexpr (SM)
            sf_voff_w = sf_mn_copy_block(0, lane) * sf_pitch + sf_mn_copy_row(lane);
        else
            sf_voff_w = uint32_t(64 * (wave & 3) + (kScaleGroups ? sf_slot_row(slot) : slot)) * sf_row +
                        16u * uint32_t(lane >> 5);
    }
    // kPair with grouped scale copies: the E4M3 operand's rows in the slot
    // order of sf_slot_row, the E2M1 operand's in natural order
    uint32_t sf_voff_grp = 0;
    if constexpr (kPair) {
        const bool split = wave < 4 ? kRowsA : kRowsB;
        sf_voff_grp = uint32_t(64 * (wave & 3) + (split ? sf_slot_row(lane) : lane)) * sf_row;
    }
    static_assert(!SB || (kMx && W == 8), "register-assembled scales: block-scaled kinds, eight waves");
    // scale words per row per step: one (E4M3 and padded kinds, four
    // 32-element blocks), two (E2M1, eight blocks), twice that with
    // 16-element blocks; word w of 64-row group g sits at stage byte
    // 2048w + 256g + 4*(row in group)
    constexpr int kWords = (kFp4 ? 2 : 1) * (kV16 ? 2 : 1);
    // SB (K not a multiple of the K step): a row's K/SV scale bytes are then
    // not a whole number of 4-byte words, so the words cannot be copied
    // straight into LDS.  Each step, lane l of wave g loads the step's scale
    // bytes of row 64*(g%4) + l of its group one by one (range-checked: rows
    // beyond the operand read zero), assembles the words in registers and
    // stores them into the scale stage in the layout above.  A block at or
    // beyond K gets the byte 127 (2^0): its values are zeros, and no byte of
    // a neighbouring row (255 would be NaN) is read for it.
    uint32_t sbyte[SB ? 4 * kWords : 1];
    const uint32_t sf_range = kMx ? uint32_t(wave < 4 ? rows_a : rows_b) * sf_row : 0;
    auto load_scale_bytes = [&](int kt) {
        if constexpr (SB) {
#pragma unroll
            for (int w = 0; w < kWords; ++w)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t j = 4u * uint32_t(kWords * kt + w) + uint32_t(b);   // block index in the row
                    const uint32_t off = j < sf_row ? sf_voff + j : sf_range;
                    sbyte[4 * w + b] = j < sf_row ? uint32_t(__builtin_amdgcn_raw_buffer_load_b8(sf_rsrc[0], off, 0, 0))
                                                  : 127u;
                }
        }
    };
    auto put_scales = [&](uint8_t *sstage) {
        if constexpr (SB) {
            sched_fence();   // after the step's MFMAs: the loads' wait must not block them
#pragma unroll
            for (int w = 0; w < kWords; ++w) {
                const uint32_t word = sbyte[4 * w] | (sbyte[4 * w + 1] << 8) | (sbyte[4 * w + 2] << 16) |
                                      (sbyte[4 * w + 3] << 24);
                *reinterpret_cast<uint32_t *>(sstage + 2048 * w + 256 * wave + 4 * lane) = word;
            }
        }
    };

    // per-step MN-major scale copies (kMnStep): kMnInstr 1 KiB instructions
    // per operand and step, issued by waves 0.. and 4..; the others' offset
    // lies beyond the buffer range (below 2^31 bytes, checked by the host)
    constexpr int kMnInstr = kFp4 ? 2 : 1, kMnBlocks = 4 * kMnInstr;
    const bool mn_active = (wave & 3) < kMnInstr;
    const uint32_t sf_voff_step = mn_active ? sf_voff_w : 0x80000000u;
    auto issue_step = [&](uint8_t *stage, uint8_t *sstage, int kt) {
        if constexpr (kDmaA)
            da.issue(stage, kt);
        if constexpr (kTrA)
            dma_mna.issue(stage, kt);
        if constexpr (kTrB)
            dma_mnb.issue(stage, kt);
        if constexpr (kDmaB)
            db.issue(stage, kt);
        if constexpr (SB) {
            load_scale_bytes(kt);
        } else if constexpr (kMnStep) {
            // instruction i = wave % 4 of the operand's step: K blocks
            // kMnBlocks kt + 4i .. +3 of all 256 rows (sf_mn_offset); the
            // other waves issue theirs out of the buffer's range (no memory
            // access) into stage bytes that no read touches, so that every
            // wave runs the same code (a branch here split the loop's
            // schedule and spilled 115-135 registers)
            buffer_load_lds16(sf_rsrc[0], sstage + (wave >> 2) * kSfMnB + 1024 * (wave & 3), sf_voff_step,
                              mn_active ? uint32_t(kMnBlocks * kt + 4 * (wave & 3)) * sf_pitch : 0u);
        } else if constexpr (kMx) {
#pragma unroll
            for (int q = 0; q < kSfInstr; ++q)
#pragma unroll
                for (int w = 0; w < kWords; ++w)
                    buffer_load_lds4(sf_rsrc[q], sstage + 2048 * w + 256 * (wave + W * q), sf_voff,
                                     4u * uint32_t(kWords * kt + w));
        }
    };
    // the operand copies of one step without its scale words (grouped scales)
    auto issue_ab = [&](uint8_t *stage, int kt) {
        if constexpr (kDmaA)
            da.issue(stage, kt);
        if constexpr (kDmaB)
            db.issue(stage, kt);
    };
    // scale group `grp` (K steps 4grp .. 4grp+3; E2M1: 2grp, 2grp+1),
    // kScaleGroups and kFp4Groups only
    auto issue_scales = [&](uint8_t *sstage, int grp) {
        if constexpr (kScaleGroups || kFp4Groups)
            buffer_load_lds16(sf_rsrc[0], sstage + 1024 * wave, sf_voff, 16u * uint32_t(grp));
    };
    // wide group `grp` (K steps 8grp .. 8grp+7; E2M1: 4grp .. 4grp+3)
    auto issue_scales_wide = [&](uint8_t *sstage, int grp) {
        if constexpr (kWideStage) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
                buffer_load_lds16(sf_rsrc[0], sstage + 2048 * wave + 1024 * q, sf_voff_w,
                                  SM ? uint32_t(32 * grp + 4 * (2 * (wave & 3) + q)) * sf_pitch
                                     : 32u * uint32_t(grp) + uint32_t(32 * q) * sf_row);
        }
    };

    // ---- MFMA operand read addresses -------------------------------------------
    // Block row `row` of a fragment, 16-byte chunk c, sits at
    // row*128 + ((c ^ key(row)) << 4).  For sub-step ks the chunk is
    // 2ks ^ lh (16-bit) or 4ks ^ lh and 4ks ^ 2 ^ lh (8-bit), so every address
    // is one per-fragment base XOR a constant.
    // In an MN-major tile read with transposing reads (kTrA / kTrB) the base
    // is mn_frag_base and sub-step ks, half e sits (16ks + 4e) K rows further.
    uint32_t abase[TM], bbase[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const uint32_t row = wm + 32 * i + lr;
        abase[i] = kTrA ? mn_frag_base(0, wm + 32 * i, lane)
                        : row * kTileRowBytes + ((lh ^ tile_key(row)) << 4);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const uint32_t row = wn + 32 * j + lr;
        bbase[j] = kTrB ? mn_frag_base(kATile, wn + 32 * j, lane)
                        : kATile + row * kTileRowBytes + ((lh ^ tile_key(row)) << 4);
    }

    // 16x16 MFMAs (MF16): the same wave tile as 2TM x 2TN blocks of
    // 16 x 16.  16-bit: fragment rows l % 16, 16-byte chunk 4s + kblk16(l/16)
    // for the 32-wide sub-step s, i.e. base XOR (s << 6).  E4M3: one 16x16x128
    // MFMA per K step, chunks mx_chunk16(l/16) and that + 4 (base XOR 64).
    constexpr bool kMf16 = MF16;
    // Epilogue through LDS with non-temporal 256-byte row pieces (see the
    // epilogue), except where it made the compiler spill inside the main loop
    // (it shares the register allocation): dense E2M1 with 16-element scale
    // blocks, E4M3 A with 6-bit B, padded E2M1 A with another kind of B, and
    // the 16-bit kernel with both operands MN-major.  Kernels with an E4M3
    // operand make room for it by reading fragments one MFMA ahead.
    constexpr bool kStagedEpi = kMf16 && OUT == kOutF32 && !(A_MN && B_MN) && !(kFp4 && kV16) &&
                                !(KIND == kE4m3 && (kKindB == kE2m3 || kKindB == kE3m2)) &&
                                !(KIND == kE2m1p && kKindB != kE2m1p);
    constexpr int TM16 = kMf16 ? 2 * TM : 1, TN16 = kMf16 ? 2 * TN : 1;
    uint32_t abase16[TM16], bbase16[TN16];
    if constexpr (kMf16) {
        const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
        for (int i = 0; i < TM16; ++i) {
            const int c = kPair ? (kPairB ? pair_chunk16(g) : kblk16(g))
                          : kFp6 ? fp6_chunk16(g) : kFp8 ? (kMixed ? mx_chunk16_mixed(g) : mx_chunk16(g)) : kblk16(g);
            abase16[i] = kTrA ? mn_frag_base16(0, wm + 16 * i, lane) : kfrag_base<kRowsA>(0, wm, i, c, lane);
        }
#pragma unroll
        for (int j = 0; j < TN16; ++j) {
            const int c = kPair ? (kPairA ? pair_chunk16(g) : kblk16(g))
                          : kMixed ? (kFp6B ? fp6_chunk16(g) : mx_chunk16_mixed(g))
                                   : kFp6 ? fp6_chunk16(g) : kFp8 ? mx_chunk16(g) : kblk16(g);
            bbase16[j] = kTrB ? mn_frag_base16(kATile, wn + 16 * j, lane) : kfrag_base<kRowsB>(kATile, wn, j, c, lane);
        }
    }

    f32x16 acc[kMf16 ? 1 : TN][kMf16 ? 1 : TM];
    f32x4 acc4[TN16][TM16];
    if constexpr (kMf16) {
#pragma unroll
        for (int j = 0; j < TN16; ++j)
#pragma unroll
            for (int i = 0; i < TM16; ++i)
                acc4[j][i] = f32x4{};
    } else {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[j][i] = f32x16{};
    }

    auto compute16 = [&](const uint8_t *s) {
        uint32_t ab[TM], bb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            ab[i] = opaque(abase[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            bb[j] = opaque(bbase[j]);
        u32x4 af[2][TM], bf[2][TN];
        auto frag = [&](uint32_t base, int ks, bool tr) {
            if (!tr)
                return lds_read16(s, base ^ (ks << 5));
            const uint32_t b = base ^ ((ks & 1) << 5);
            const u32x2 lo = lds_read_tr16(s, b + uint32_t(16 * ks) * kMnRowBytes);
            const u32x2 hi = lds_read_tr16(s, b + uint32_t(16 * ks + 4) * kMnRowBytes);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        auto rd = [&](int ks, u32x4 *a, u32x4 *b) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                a[i] = frag(ab[i], ks, kTrA);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                b[j] = frag(bb[j], ks, kTrB);
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

    auto compute16x16 = [&](const uint8_t *s) {
        uint32_t ab[TM16], bb[TN16];
#pragma unroll
        for (int i = 0; i < TM16; ++i)
            ab[i] = opaque(abase16[i]);
#pragma unroll
        for (int j = 0; j < TN16; ++j)
            bb[j] = opaque(bbase16[j]);
        auto frag = [&](uint32_t base, int ks, bool tr) {
            if (!tr)
                return lds_read16(s, base ^ (ks << 6));
            const u32x2 lo = lds_read_tr16(s, base + uint32_t(32 * ks) * kMnRowBytes);
            const u32x2 hi = lds_read_tr16(s, base + uint32_t(32 * ks + 4) * kMnRowBytes);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            u32x4 af[TM16], bf[TN16];
#pragma unroll
            for (int i = 0; i < TM16; ++i)
                af[i] = frag(ab[i], ks, kTrA);
#pragma unroll
            for (int j = 0; j < TN16; ++j)
                bf[j] = frag(bb[j], ks, kTrB);
#pragma unroll
            for (int j = 0; j < TN16; ++j)
#pragma unroll
                for (int i = 0; i < TM16; ++i)
                    acc4[j][i] = mfma_16x16x32<KIND == kBf16>(bf[j], af[i], acc4[j][i]);
        }
    };

    // sf_stride: scale-stage bytes per row (4: one step's word; 16: a group of
    // four steps); widx: which of the row's words (the step inside its group)
    // wide: the scale stage of the wide groups (32 bytes per row; widx 0..7)
    auto compute_mx16 = [&](const uint8_t *s, const uint8_t *ss, int sf_stride, int widx, auto wide) {
        constexpr bool WD = decltype(wide)::value;
        uint32_t ab[TM16], bb[TN16];
#pragma unroll
        for (int i = 0; i < TM16; ++i)
            ab[i] = opaque(abase16[i]);
#pragma unroll
        for (int j = 0; j < TN16; ++j)
            bb[j] = opaque(bbase16[j]);
        // lane l supplies the scale of K block l/16 of row l % 16: byte l/16 of
        // the row's scale word, read as one byte (a word and a per-lane shift
        // would keep one more register live through the loop)
        // (row16(b, x) = row16(0, x) + 32*(b/2) + 8*(b%2): one per-lane base
        // and constant offsets, kept opaque so that they are not hoisted).
        // With kScaleGroups the rows sit in the slot order of sf_slot_row
        // (both the per-step words and the 16-byte groups): block b of row x
        // is slot (wave's first row) + 16 * b + x.
        const int r16 = lane & 15;
        static_assert(!kScaleGroups || (32 * TN) % 64 == 0, "wave rows start 64-row groups");
        // (wide stage: sf_wide_read with the step's half widx/4 and byte
        // 4 (widx%4) + block, split into lane, block and step parts)
        // (MN-major scales: sf_mn_offset of K block 4 widx + l/16 and the
        // lane's tile row, B's stage half 8 KiB further, split likewise)
        constexpr bool MN = WD && SM;
        const uint32_t sfa = opaque(MN   ? sf_mn_offset(uint32_t(lane >> 4), uint32_t(wm + row16<true>(0, r16)))
                                    : WD ? sf_wide_read(wm, 0, 0, lane >> 4, lane)
                                         : uint32_t(sf_stride * (wm + (kScaleGroups ? r16 : row16<true>(0, r16))) + (lane >> 4)));
        const uint32_t sfb = opaque(MN   ? kSfMnB + sf_mn_offset(uint32_t(lane >> 4), uint32_t(wn + row16<true>(0, r16)))
                                    : WD ? sf_wide_read(kBM + wn, 0, 0, lane >> 4, lane)
                                         : uint32_t(sf_stride * (kBM + wn + (kScaleGroups ? r16 : row16<true>(0, r16))) + (lane >> 4)));
        auto sf_off = [&](int b) {
            return MN   ? int(sf_mn_offset(0, uint32_t(row16<true>(b, 0))))
                   : WD ? int(sf_wide_read(0, b, 0, 0, 0)) : sf_stride * (kScaleGroups ? 16 * b : 32 * (b >> 1) + 8 * (b & 1));
        };
        const int sstep = MN ? int(sf_mn_offset(uint32_t(4 * widx), 0)) : WD ? int(sf_wide_offset(0, widx >> 2)) + 4 * (widx & 3) : 4 * widx;
        // E4M3: chunks c and c + 4.  Padded kinds: chunks c and c ^ 1, of
        // which the first twelve (6-bit) or eight (4-bit) bytes each form
        // registers 0..2 and 3..5 (0..1 and 2..3)
        auto frag_of = [&](uint32_t base, auto kind) {
            constexpr int k = decltype(kind)::value;
            const u32x4 lo = lds_read16(s, base);
            const u32x4 hi = lds_read16(s, base ^ (padded_kind(k) ? 16u : 64u));
            if constexpr (k == kE2m1p)
                return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 4, 5, 2, 3, 6, 7));
            else if constexpr (padded_kind(k))
                return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 4, 5, 6, 3, 7));
            else
                return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        auto frag = [&](uint32_t base) { return frag_of(base, std::integral_constant<int, KIND>{}); };
        auto frag_b = [&](uint32_t base) { return frag_of(base, std::integral_constant<int, kKindB>{}); };
        // MFMA m = TN16 * i + j; each block's fragment and scale are read two
        // MFMAs ahead of first use, in that order (FragSchedule), so that a
        // wave's first MFMA waits for a few reads rather than for the whole
        // step's B fragments and scales, which all eight waves request at once
        // after the barrier.  With an E4M3 operand and the staged epilogue one
        // MFMA ahead: that frees the registers the epilogue needs (with two,
        // the compiler spilled inside the loop); the loop alone is 1.4 %
        // slower, the kernel with the staged epilogue 4 % faster (8192^3
        // MX-fp8).  With the wide loop alone (kWideOnly) the kernels have the
        // registers for two (8192^3, row-major scales: E4M3 -1.9 %, E4M3 with
        // padded E2M1 -3.2 %; MN-major: -1.7 % and -2.2 %, with E2M3 level).
        constexpr int kAhead = kStagedEpi && (KIND == kE4m3 || kKindB == kE4m3) && !kWideOnly ? 1 : 2;
        using Sched = FragSchedule<TM16, TN16, kAhead>;
        uint32_t sa[TM16], sb[TN16];
        i32x8 bf[TN16], af[TM16];
        static_for<0, TM16 * TN16>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            constexpr int c0 = m == 0 ? 0 : Sched::issued(m - 1), c1 = Sched::issued(m);
            static_for<c0, c1>([&](auto rc) {
                constexpr int it = Sched::item(decltype(rc)::value);
                if constexpr (it > 0) {
                    sa[it - 1] = ss[sfa + sf_off(it - 1) + sstep];
                    af[it - 1] = frag(ab[it - 1]);
                } else {
                    sb[-it - 1] = ss[sfb + sf_off(-it - 1) + sstep];
                    bf[-it - 1] = frag_b(bb[-it - 1]);
                }
            });
            if constexpr (c1 > c0)
                __builtin_amdgcn_sched_group_barrier(0x100, 3 * (c1 - c0), 0);   // DS reads
            constexpr int i = m / TN16, j = m % TN16;
            acc4[j][i] = mfma_scale_16x16x128_fmt<mx_format<kKindB>(), mx_format<KIND>()>(bf[j], af[i], acc4[j][i],
                                                                                          sb[j], sa[i]);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                     // MFMA
        });
    };

    // E2M1: two 128-element sub-steps per step; lane (r, g) reads chunk
    // 4ks + kblk16(g) of its row (one 32-element scale block, 16 bytes) into
    // the low half of the operand and supplies that block's scale: byte
    // kblk16(g) of the row's scale word ks.
    // sf_stride: scale-stage bytes per row (4: per-step words, the second
    // 2048 bytes further; 16: a group of two steps, eight bytes each); widx:
    // the step inside its group
    // wide: the scale stage of the wide groups (32 bytes per row, four steps;
    // widx 0..3)
    auto compute_fp4 = [&](const uint8_t *s, const uint8_t *ss, int sf_stride, int widx, auto wide) {
        constexpr bool WD = decltype(wide)::value;
        uint32_t ab[TM16], bb[TN16];
#pragma unroll
        for (int i = 0; i < TM16; ++i)
            ab[i] = opaque(abase16[i]);
#pragma unroll
        for (int j = 0; j < TN16; ++j)
            bb[j] = opaque(bbase16[j]);
        // lane group g supplies the scale of block kblk16(g): that byte of its
        // row's scale word, read as one byte.  With 16-element blocks the
        // chunk's two halves are 16-blocks 2c and 2c + 1 of the step (c =
        // 4ks + kblk16(g)): word 2ks + kblk16(g)/2, bytes 2 (kblk16(g) % 2) and
        // that + 1.
        const int r16 = lane & 15, kb = kblk16(lane >> 4);
        const uint32_t sb16 = kV16 ? uint32_t(2048 * (kb >> 1) + 2 * (kb & 1)) : uint32_t(kb);
        // (wide stage: rows in natural order, read as in compute_mx16 with
        // the step's half widx/2 and byte 8 (widx%2) + 4 ks + block)
        // (MN-major scales: sf_mn_offset of K block 4 (2 widx + ks) + kblk16
        // and the lane's tile row)
        constexpr bool MN = WD && SM;
        const uint32_t sfa = opaque(MN   ? sf_mn_offset(uint32_t(kb), uint32_t(wm + r16))
                                    : WD ? sf_wide_read(wm, 0, 0, sb16, lane) : uint32_t(sf_stride * (wm + r16)) + sb16);
        const uint32_t sfb = opaque(MN   ? kSfMnB + sf_mn_offset(uint32_t(kb), uint32_t(wn + r16))
                                    : WD ? sf_wide_read(kBM + wn, 0, 0, sb16, lane)
                                         : uint32_t(sf_stride * (kBM + wn + r16)) + sb16);
        const uint32_t sf_blk = 16u * uint32_t(sf_stride);   // 16 rows further
        auto blk_off = [&](int b) {
            return MN ? sf_mn_offset(0, uint32_t(16 * b)) : WD ? sf_wide_read(0, b, 0, 0, 0) : sf_blk * uint32_t(b);
        };
        const u32x4 zero = {0, 0, 0, 0};
        // sub-step u: K elements 128 u' .. of the step (u' = ks), and with
        // 16-element blocks each chunk in two halves h
        auto frag = [&](uint32_t base, int ks, int h) {
            if constexpr (kV16) {
                // registers 0..1 the half, 2..3 zero, 4..7 not read by the FP4 MFMA
                const u32x2 d = lds_read8(s, (base ^ uint32_t(ks << 6)) + 8u * uint32_t(h));
                const u32x2 z = {0, 0};
                return __builtin_bit_cast(i32x8, __builtin_shufflevector(d, z, 0, 1, 2, 3, -1, -1, -1, -1));
            } else {
                const u32x4 v = lds_read16(s, base ^ uint32_t(ks << 6));
                return __builtin_bit_cast(i32x8, __builtin_shufflevector(v, zero, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        };
        // reads three MFMAs ahead of first use (two with 16-element blocks,
        // whose kernels have no registers to spare), as in compute_mx16; three
        // ran 8192^3 MX-fp4 1.6 % faster than two
        using Sched = FragSchedule<TM16, TN16, kV16 ? 2 : 3>;
        static_for<0, kV16 ? 4 : 2>([&](auto uc) {
            constexpr int u = decltype(uc)::value;
            constexpr int ks = kV16 ? u >> 1 : u, h = kV16 ? u & 1 : 0;
            // scale byte offset of the sub-step
            const int sw = kV16 ? 2048 * 2 * ks + h
                           : MN ? int(sf_mn_offset(uint32_t(4 * (2 * widx + ks)), 0))
                           : WD ? int(sf_wide_offset(0, widx >> 1)) + 8 * (widx & 1) + 4 * ks
                                : sf_stride == 16 ? 8 * widx + 4 * ks : 2048 * ks;
            uint32_t sa[TM16], sb[TN16];
            i32x8 bf[TN16], af[TM16];
            static_for<0, TM16 * TN16>([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                constexpr int c0 = m == 0 ? 0 : Sched::issued(m - 1), c1 = Sched::issued(m);
                static_for<c0, c1>([&](auto rc) {
                    constexpr int it = Sched::item(decltype(rc)::value);
                    if constexpr (it > 0) {
                        sa[it - 1] = ss[sw + sfa + blk_off(it - 1)];
                        af[it - 1] = frag(ab[it - 1], ks, h);
                    } else {
                        sb[-it - 1] = ss[sw + sfb + blk_off(-it - 1)];
                        bf[-it - 1] = frag(bb[-it - 1], ks, h);
                    }
                });
                if constexpr (c1 > c0)
                    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (c1 - c0), 0);   // DS reads
                constexpr int i = m / TN16, j = m % TN16;
                acc4[j][i] = mfma_scale_16x16x128_e2m1(bf[j], af[i], acc4[j][i], sb[j], sa[i]);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                     // MFMA
            });
        });
    };

    // Padded kinds with 16-element scale blocks: lane group g's two chunks
    // (fp6_chunk16(g) and that ^ 1) are one 16-block each, taken one per
    // sub-step h into the low registers (twelve bytes for 6-bit, eight for
    // 4-bit values; the rest zero).  Chunk c of the step is 16-block c: word
    // c / 4 = g / 2 of the row's two per-step words, byte c % 4.
    auto compute_pad16 = [&](const uint8_t *s, const uint8_t *ss) {
        uint32_t ab[TM16], bb[TN16];
#pragma unroll
        for (int i = 0; i < TM16; ++i)
            ab[i] = opaque(abase16[i]);
#pragma unroll
        for (int j = 0; j < TN16; ++j)
            bb[j] = opaque(bbase16[j]);
        const int r16 = lane & 15, g = lane >> 4;
        const uint32_t sg = uint32_t(2048 * (g >> 1) + (fp6_chunk16(g) & 3));
        const uint32_t sfa = opaque(uint32_t(4 * (wm + row16<true>(0, r16))) + sg);
        const uint32_t sfb = opaque(uint32_t(4 * (kBM + wn + row16<true>(0, r16))) + sg);
        auto sf_off = [&](int b) { return 4 * (32 * (b >> 1) + 8 * (b & 1)); };
        auto frag = [&](uint32_t base, int h) {
            const uint32_t a = base ^ uint32_t(16 * h);
            // the half in the low registers, zeros for the other half, the
            // registers the format does not read left undefined
            if constexpr (KIND == kE2m1p) {
                const u32x2 d = lds_read8(s, a);
                const u32x2 z = {0, 0};
                return __builtin_bit_cast(i32x8, __builtin_shufflevector(d, z, 0, 1, 2, 3, -1, -1, -1, -1));
            } else {
                const u32x4 d = lds_read16(s, a);            // the last word is padding
                const u32x4 z = {0, 0, 0, 0};
                return __builtin_bit_cast(i32x8, __builtin_shufflevector(d, z, 0, 1, 2, 4, 5, 6, -1, -1));
            }
        };
        using Sched = FragSchedule<TM16, TN16, 2>;
        static_for<0, 2>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            // the two halves' fragments are not interleaved (register pressure)
            if constexpr (h == 1)
                __builtin_amdgcn_sched_barrier(0);
            uint32_t sa[TM16], sb[TN16];
            i32x8 bf[TN16], af[TM16];
            static_for<0, TM16 * TN16>([&](auto mc) {
                constexpr int m = decltype(mc)::value;
                constexpr int c0 = m == 0 ? 0 : Sched::issued(m - 1), c1 = Sched::issued(m);
                static_for<c0, c1>([&](auto rc) {
                    constexpr int it = Sched::item(decltype(rc)::value);
                    if constexpr (it > 0) {
                        sa[it - 1] = ss[(sfa ^ uint32_t(h)) + sf_off(it - 1)];
                        af[it - 1] = frag(ab[it - 1], h);
                    } else {
                        sb[-it - 1] = ss[(sfb ^ uint32_t(h)) + sf_off(-it - 1)];
                        bf[-it - 1] = frag(bb[-it - 1], h);
                    }
                });
                if constexpr (c1 > c0)
                    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (c1 - c0), 0);   // DS reads
                constexpr int i = m / TN16, j = m % TN16;
                acc4[j][i] = mfma_scale_16x16x128_fmt<mx_format<KIND>(), mx_format<KIND>()>(bf[j], af[i], acc4[j][i],
                                                                                            sb[j], sa[i]);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                     // MFMA
            });
        });
    };

    // E4M3 paired with dense E2M1 (kPair), one 128-element K step: the E4M3
    // operand's tile in stage s8 (its split-row fragments, chunks
    // pair_chunk16(g) and that ^ 2), the E2M1 operand's in stage s4 (its
    // 128-byte rows hold two steps; half h = the step's parity: contiguous
    // fragment rows, chunk 4h + kblk16(g), one 32-element block per lane in
    // the low four registers).  Both sides' lane group g supplies the scale
    // of memory block kblk16(g) of the step: that byte of the row's per-step
    // scale word (rows in natural order, 4 bytes apart).
    // sf_stride 4: per-step words (rows in natural order); 16: a group of
    // four steps per row slot (slot 16b + x holds fragment row x of block b
    // on either side), widx the step inside the group
    auto compute_pair = [&](const uint8_t *s8, const uint8_t *s4, int h, const uint8_t *ss, int sf_stride, int widx) {
        uint32_t ab[TM16], bb[TN16];
#pragma unroll
        for (int i = 0; i < TM16; ++i)
            ab[i] = opaque(abase16[i]);
#pragma unroll
        for (int j = 0; j < TN16; ++j)
            bb[j] = opaque(bbase16[j]);
        const int r16 = lane & 15, kb = kblk16(lane >> 4);
        const bool grp = sf_stride == 16;
        // (MN-major scales, SM: the per-step stage, sf_mn_offset of K block
        // kb and the lane's tile row on each side, B's half 8 KiB further)
        const uint32_t sfa = opaque(SM ? sf_mn_offset(uint32_t(kb), uint32_t(wm + row16<kRowsA>(0, r16)))
                                       : uint32_t(sf_stride * (wm + (kRowsA && !grp ? row16<true>(0, r16) : r16)) + kb +
                                                  4 * widx));
        const uint32_t sfb = opaque(SM ? kSfMnB + sf_mn_offset(uint32_t(kb), uint32_t(wn + row16<kRowsB>(0, r16)))
                                       : uint32_t(sf_stride * (kBM + wn + (kRowsB && !grp ? row16<true>(0, r16) : r16)) +
                                                  kb + 4 * widx));
        auto sf_off = [&](bool split, int b) {
            if constexpr (SM)
                return int(split ? sf_mn_offset(0, uint32_t(row16<true>(b, 0))) : sf_mn_offset(0, uint32_t(16 * b)));
            else
                return sf_stride * (split && !grp ? 32 * (b >> 1) + 8 * (b & 1) : 16 * b);
        };
        const u32x4 zero = {0, 0, 0, 0};
        auto frag8 = [&](uint32_t base) {
            const u32x4 lo = lds_read16(s8, base), hi = lds_read16(s8, base ^ 32u);
            return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        auto frag4 = [&](uint32_t base) {
            const u32x4 v = lds_read16(s4, base ^ uint32_t(h << 6));
            return __builtin_bit_cast(i32x8, __builtin_shufflevector(v, zero, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // reads (fragment and scale) per A and per B item of the schedule
        constexpr int kReadsA = kRowsA ? 3 : 2, kReadsB = kRowsB ? 3 : 2;
        using Sched = FragSchedule<TM16, TN16, 2>;
        uint32_t sa[TM16], sb[TN16];
        i32x8 bf[TN16], af[TM16];
        static_for<0, TM16 * TN16>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            constexpr int c0 = m == 0 ? 0 : Sched::issued(m - 1), c1 = Sched::issued(m);
            constexpr int reads = [] {
                int r = 0;
                for (int c = c0; c < c1; ++c)
                    r += Sched::item(c) > 0 ? kReadsA : kReadsB;
                return r;
            }();
            static_for<c0, c1>([&](auto rc) {
                constexpr int it = Sched::item(decltype(rc)::value);
                if constexpr (it > 0) {
                    sa[it - 1] = ss[sfa + sf_off(kRowsA, it - 1)];
                    af[it - 1] = kRowsA ? frag8(ab[it - 1]) : frag4(ab[it - 1]);
                } else {
                    sb[-it - 1] = ss[sfb + sf_off(kRowsB, -it - 1)];
                    bf[-it - 1] = kRowsB ? frag8(bb[-it - 1]) : frag4(bb[-it - 1]);
                }
            });
            if constexpr (c1 > c0)
                __builtin_amdgcn_sched_group_barrier(0x100, reads, 0);   // DS reads
            constexpr int i = m / TN16, j = m % TN16;
            acc4[j][i] = mfma_scale_16x16x128_fmt<mx_format<kKindB>(), mx_format<KIND>()>(bf[j], af[i], acc4[j][i],
                                                                                          sb[j], sa[i]);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                     // MFMA
        });
    };

    auto compute = [&](const uint8_t *s, const uint8_t *ss) {
        if constexpr (kMnStep && kFp4)
            compute_fp4(s, ss, 16, 0, std::true_type{});     // MN-major stage, first K blocks
        else if constexpr (kMnStep)
            compute_mx16(s, ss, 16, 0, std::true_type{});
        else if constexpr (kFp4)
            compute_fp4(s, ss, 4, 0, std::false_type{});
        else if constexpr (kFp6 && kV16)
            compute_pad16(s, ss);
        else if constexpr (kMx)
            compute_mx16(s, ss, 4, 0, std::false_type{});
        else if constexpr (kMf16)
            compute16x16(s);
        else
            compute16(s);
    };

    // ---- main loop: two K steps per iteration, one stage array each; an odd
    // final step (already in lds0) is computed after the loop.  The loop body
    // has no branches: in the last pair of an even step count the copy into
    // lds0 repeats step KT-1 into a stage nobody reads again, which keeps the
    // compiler from draining the copies in flight at a control-flow merge. ------
    if constexpr (kPair) {
        // E4M3 with dense E2M1 (K a multiple of 256; the host launches no
        // other): four K steps per iteration, then the last pair of steps
        // when their number is not a multiple of four.  The E4M3 operand's stages
        // alternate lds0 / lds1 every step; the E2M1 operand's 128-byte tile
        // rows hold two steps, so its tile for steps 2p and 2p+1 sits in its
        // part of stage p % 2 and is copied half during each of the two steps
        // before, into a stage whose last reader ended at the barrier before
        // them.  Scale words go per step into scl0 / scl1.  Copies beyond the
        // end repeat the last step or pair into a stage nobody reads again, so
        // the loop has no branches.
        DmaOperand<W> &d8 = kPairB ? da : db;
        DmaOperand<W> &d4 = kPairB ? db : da;
        const int NP = KT / 2;
        auto issue_sf = [&](uint8_t *sstage, int kt) {
            if constexpr (SM)   // K blocks 4kt .. 4kt+3 of 256 rows per operand (as issue_step)
                buffer_load_lds16(sf_rsrc[0], sstage + (wave >> 2) * kSfMnB + 1024 * (wave & 3), sf_voff_step,
                                  mn_active ? uint32_t(4 * kt) * sf_pitch : 0u);
            else
                buffer_load_lds4(sf_rsrc[0], sstage + 256 * wave, sf_voff, 4u * uint32_t(kt));
        };
        static_assert(kSfInstr == 1 && kWords == 1, "one per-step scale word per row, one copy per wave");
        if (!SM && KT % 8 == 0) {
            // K a multiple of 1024: scale words copied per group of four
            // steps (16 bytes per row, as for E4M3 alone), into scl0 / scl1
            // alternating every four steps, each as the last copy of the third
            // step of the group before and left in flight by that step's
            // barrier; eight steps per iteration
            const int NG = KT / 4;
            auto issue_grp = [&](uint8_t *sstage, int grp) {
                buffer_load_lds16(sf_rsrc[0], sstage + 1024 * wave, sf_voff_grp, 16u * uint32_t(grp));
            };
            auto step_end = [] {
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier_keep_vm<0>();
                __builtin_amdgcn_sched_barrier(0);
            };
            auto step_end_keep1 = [] {
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier_keep_vm<1>();
                __builtin_amdgcn_sched_barrier(0);
            };
            issue_grp(scl0, 0);
            d8.issue(lds0, 0);
            d4.issue(lds0, 0);
            __syncthreads();
            for (int kt = 0; kt < KT; kt += 8) {
                const int g = kt / 4, p = kt / 2;
                d8.issue(lds1, kt + 1);
                d4.issue_half(lds1, p + 1, 0);
                compute_pair(lds0, lds0, 0, scl0, 16, 0);
                step_end();
                d8.issue(lds0, kt + 2);
                d4.issue_half(lds1, p + 1, 1);
                compute_pair(lds1, lds0, 1, scl0, 16, 1);
                step_end();
                d8.issue(lds1, kt + 3);
                d4.issue_half(lds0, p + 2, 0);
                issue_grp(scl1, g + 1);
                compute_pair(lds0, lds1, 0, scl0, 16, 2);
                step_end_keep1();
                d8.issue(lds0, kt + 4);
                d4.issue_half(lds0, p + 2, 1);
                compute_pair(lds1, lds1, 1, scl0, 16, 3);
                step_end();
                d8.issue(lds1, kt + 5);
                d4.issue_half(lds1, p + 3, 0);
                compute_pair(lds0, lds0, 0, scl1, 16, 0);
                step_end();
                d8.issue(lds0, kt + 6);
                d4.issue_half(lds1, p + 3, 1);
                compute_pair(lds1, lds0, 1, scl1, 16, 1);
                step_end();
                d8.issue(lds1, kt + 7);
                d4.issue_half(lds0, min(p + 4, NP - 1), 0);
                issue_grp(scl0, min(g + 2, NG - 1));
                compute_pair(lds0, lds1, 0, scl1, 16, 2);
                step_end_keep1();
                d8.issue(lds0, min(kt + 8, KT - 1));
                d4.issue_half(lds0, min(p + 4, NP - 1), 1);
                compute_pair(lds1, lds1, 1, scl1, 16, 3);
                step_end();
            }
            __syncthreads();   // no copy may still be writing LDS when the workgroup ends
            goto epilogue;
        }
        d8.issue(lds0, 0);
        d4.issue(lds0, 0);
        issue_sf(scl0, 0);
        __syncthreads();
        int kt = 0;
        for (; kt + 4 <= KT; kt += 4) {
            const int p = kt / 2;
            d8.issue(lds1, kt + 1);
            d4.issue_half(lds1, min(p + 1, NP - 1), 0);
            issue_sf(scl1, kt + 1);
            compute_pair(lds0, lds0, 0, scl0, 4, 0);
            lds_barrier_keep_vm<0>();
            d8.issue(lds0, min(kt + 2, KT - 1));
            d4.issue_half(lds1, min(p + 1, NP - 1), 1);
            issue_sf(scl0, min(kt + 2, KT - 1));
            compute_pair(lds1, lds0, 1, scl1, 4, 0);
            lds_barrier_keep_vm<0>();
            d8.issue(lds1, min(kt + 3, KT - 1));
            d4.issue_half(lds0, min(p + 2, NP - 1), 0);
            issue_sf(scl1, min(kt + 3, KT - 1));
            compute_pair(lds0, lds1, 0, scl0, 4, 0);
            lds_barrier_keep_vm<0>();
            d8.issue(lds0, min(kt + 4, KT - 1));
            d4.issue_half(lds0, min(p + 2, NP - 1), 1);
            issue_sf(scl0, min(kt + 4, KT - 1));
            compute_pair(lds1, lds1, 1, scl1, 4, 0);
            lds_barrier_keep_vm<0>();
        }
        if (kt < KT) {
            // steps KT-2 and KT-1: their E2M1 pair, E4M3 step KT-2 and its
            // scale words are in lds0 / scl0 (the loop's last copies, or the
            // prologue's)
            d8.issue(lds1, KT - 1);
            issue_sf(scl1, KT - 1);
            compute_pair(lds0, lds0, 0, scl0, 4, 0);
            lds_barrier_keep_vm<0>();
            compute_pair(lds1, lds0, 1, scl1, 4, 0);
        }
        __syncthreads();   // no copy may still be writing LDS when the workgroup ends
        goto epilogue;
    }
    if constexpr (kFp4Groups && !kMnStep) {
        if (KT % 8 == 0) {
            // Dense E2M1, K a multiple of 2048: eight K steps per iteration,
            // wide scale groups of four steps (scl0 for the first four, scl1
            // for the next).  A group's scales (two copies per wave) are
            // copied during the third step of the group before it, as that
            // step's last copies, which its barrier leaves in flight; the
            // stage they overwrite was last read three steps earlier.  Copies
            // beyond the end repeat the last step or group into a stage nobody
            // reads again, so the loop has no branches.
            const int NG = KT / 4;
            auto step_end = [] {
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier_keep_vm<0>();
                __builtin_amdgcn_sched_barrier(0);
            };
            auto step_end_keep2 = [] {
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier_keep_vm<2>();
                __builtin_amdgcn_sched_barrier(0);
            };
            using wide = std::true_type;
            issue_scales_wide(scl0, 0);
            issue_ab(lds0, 0);
            __syncthreads();
            for (int kt = 0; kt < KT; kt += 8) {
                const int g = kt / 4;
                issue_ab(lds1, kt + 1);
                compute_fp4(lds0, scl0, 16, 0, wide{});
                step_end();
                issue_ab(lds0, kt + 2);
                compute_fp4(lds1, scl0, 16, 1, wide{});
                step_end();
                issue_ab(lds1, kt + 3);
                issue_scales_wide(scl1, g + 1);
                compute_fp4(lds0, scl0, 16, 2, wide{});
                step_end_keep2();
                issue_ab(lds0, kt + 4);
                compute_fp4(lds1, scl0, 16, 3, wide{});
                step_end();
                issue_ab(lds1, kt + 5);
                compute_fp4(lds0, scl1, 16, 0, wide{});
                step_end();
                issue_ab(lds0, kt + 6);
                compute_fp4(lds1, scl1, 16, 1, wide{});
                step_end();
                issue_ab(lds1, kt + 7);
                issue_scales_wide(scl0, min(g + 2, NG - 1));
                compute_fp4(lds0, scl1, 16, 2, wide{});
                step_end_keep2();
                issue_ab(lds0, min(kt + 8, KT - 1));
                compute_fp4(lds1, scl1, 16, 3, wide{});
                step_end();
            }
            __syncthreads();   // no copy may still be writing LDS when the workgroup ends
            goto epilogue;
        }
        if constexpr (kWideOnly)
            goto epilogue;   // K is a multiple of 2048 (checked by the host)
        if (KT % 4 == 0) {
            // Dense E2M1, four K steps per iteration: operand stages alternate
            // lds0 / lds1, scale groups (two steps each) scl0 / scl1.  A
            // group's scales are copied during the first step of the group
            // before it, as that step's last copy, which the step's barrier
            // leaves in flight (completions are counted in order); the stage
            // they overwrite was last read a step earlier.  Copies beyond
            // the last step or group repeat the last one into a stage nobody
            // reads again, so the loop has no branches.
            const int NG = KT / 2;
            auto step_end = [] {
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier_keep_vm<0>();
                __builtin_amdgcn_sched_barrier(0);
            };
            auto step_end_keep1 = [] {
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier_keep_vm<1>();
                __builtin_amdgcn_sched_barrier(0);
            };
            issue_scales(scl0, 0);
            issue_ab(lds0, 0);
            __syncthreads();
            for (int kt = 0; kt < KT; kt += 4) {
                const int g = kt / 2;
                issue_ab(lds1, kt + 1);
                issue_scales(scl1, g + 1);
                compute_fp4(lds0, scl0, 16, 0, std::false_type{});
                step_end_keep1();
                issue_ab(lds0, kt + 2);
                compute_fp4(lds1, scl0, 16, 1, std::false_type{});
                step_end();
                issue_ab(lds1, kt + 3);
                issue_scales(scl0, min(g + 2, NG - 1));
                compute_fp4(lds0, scl1, 16, 0, std::false_type{});
                step_end_keep1();
                issue_ab(lds0, min(kt + 4, KT - 1));
                compute_fp4(lds1, scl1, 16, 1, std::false_type{});
                step_end();
            }
            __syncthreads();   // no copy may still be writing LDS when the workgroup ends
            goto epilogue;
        }
    }
    if constexpr (kScaleGroups && kWideStage && !kMnStep) {
        if (KT % 16 == 0) {
            // K a multiple of 2048: sixteen K steps per iteration, wide scale
            // groups of eight steps (scl0 for the first eight, scl1 for the
            // next), copied during the seventh step of the group before them
            // as that step's last copies (two per wave), which its barrier
            // leaves in flight; the stage they overwrite was last read seven
            // steps earlier.  Copies beyond the end repeat the last step or
            // group into a stage nobody reads again: no branches.
            const int NG = KT / 8;
            auto step_end = [] {
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier_keep_vm<0>();
                __builtin_amdgcn_sched_barrier(0);
            };
            auto step_end_keep2 = [] {
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier_keep_vm<2>();
                __builtin_amdgcn_sched_barrier(0);
            };
            using wide = std::true_type;
            issue_scales_wide(scl0, 0);
            issue_ab(lds0, 0);
            __syncthreads();
            for (int kt = 0; kt < KT; kt += 16) {
                const int g = kt / 8;
                issue_ab(lds1, kt + 1);
                compute_mx16(lds0, scl0, 16, 0, wide{});
                step_end();
                issue_ab(lds0, kt + 2);
                compute_mx16(lds1, scl0, 16, 1, wide{});
                step_end();
                issue_ab(lds1, kt + 3);
                compute_mx16(lds0, scl0, 16, 2, wide{});
                step_end();
                issue_ab(lds0, kt + 4);
                compute_mx16(lds1, scl0, 16, 3, wide{});
                step_end();
                issue_ab(lds1, kt + 5);
                compute_mx16(lds0, scl0, 16, 4, wide{});
                step_end();
                issue_ab(lds0, kt + 6);
                compute_mx16(lds1, scl0, 16, 5, wide{});
                step_end();
                issue_ab(lds1, kt + 7);
                issue_scales_wide(scl1, g + 1);
                compute_mx16(lds0, scl0, 16, 6, wide{});
                step_end_keep2();
                issue_ab(lds0, kt + 8);
                compute_mx16(lds1, scl0, 16, 7, wide{});
                step_end();
                issue_ab(lds1, kt + 9);
                compute_mx16(lds0, scl1, 16, 0, wide{});
                step_end();
                issue_ab(lds0, kt + 10);
                compute_mx16(lds1, scl1, 16, 1, wide{});
                step_end();
                issue_ab(lds1, kt + 11);
                compute_mx16(lds0, scl1, 16, 2, wide{});
                step_end();
                issue_ab(lds0, kt + 12);
                compute_mx16(lds1, scl1, 16, 3, wide{});
                step_end();
                issue_ab(lds1, kt + 13);
                compute_mx16(lds0, scl1, 16, 4, wide{});
                step_end();
                issue_ab(lds0, kt + 14);
                compute_mx16(lds1, scl1, 16, 5, wide{});
                step_end();
                issue_ab(lds1, kt + 15);
                issue_scales_wide(scl0, min(g + 2, NG - 1));
                compute_mx16(lds0, scl1, 16, 6, wide{});
                step_end_keep2();
                issue_ab(lds0, min(kt + 16, KT - 1));
                compute_mx16(lds1, scl1, 16, 7, wide{});
                step_end();
            }
            __syncthreads();   // no copy may still be writing LDS when the workgroup ends
            goto epilogue;
        }
        if constexpr (kWideOnly)
            goto epilogue;   // K is a multiple of 2048 (checked by the host)
    }
    if constexpr (kScaleGroups && !kMnStep) {
        if (KT % 8 == 0) {
            // Eight K steps per iteration: operand stages alternate lds0 /
            // lds1, scale groups alternate scl0 / scl1 every four steps.  A
            // group's scales are copied during the third step of the group
            // before it, as that step's last copy, and that step's barrier
            // leaves this one copy in flight (vector-memory completions are
            // counted in order, so it cannot hold up the step's operand
            // copies): the scattered scale reads get two steps to land, and
            // the stage they overwrite was last read four steps earlier.
            // Copies beyond the last step or group repeat the last one into a
            // stage nobody reads again, so the loop has no branches.
            const int NG = KT / 4;
            // a step's work is not moved across its closing barrier, which
            // keeps the eight unrolled steps from overlapping in registers
            auto step_end = [] {
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier_keep_vm<0>();
                __builtin_amdgcn_sched_barrier(0);
            };
            auto step_end_keep1 = [] {
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier_keep_vm<1>();
                __builtin_amdgcn_sched_barrier(0);
            };
            issue_scales(scl0, 0);
            issue_ab(lds0, 0);
            __syncthreads();
            for (int kt = 0; kt < KT; kt += 8) {
                const int g = kt / 4;
                issue_ab(lds1, kt + 1);
                compute_mx16(lds0, scl0, 16, 0, std::false_type{});
                step_end();
                issue_ab(lds0, kt + 2);
                compute_mx16(lds1, scl0, 16, 1, std::false_type{});
                step_end();
                issue_ab(lds1, kt + 3);
                issue_scales(scl1, g + 1);
                compute_mx16(lds0, scl0, 16, 2, std::false_type{});
                step_end_keep1();
                issue_ab(lds0, kt + 4);
                compute_mx16(lds1, scl0, 16, 3, std::false_type{});
                step_end();
                issue_ab(lds1, kt + 5);
                compute_mx16(lds0, scl1, 16, 0, std::false_type{});
                step_end();
                issue_ab(lds0, kt + 6);
                compute_mx16(lds1, scl1, 16, 1, std::false_type{});
                step_end();
                issue_ab(lds1, kt + 7);
                issue_scales(scl0, min(g + 2, NG - 1));
                compute_mx16(lds0, scl1, 16, 2, std::false_type{});
                step_end_keep1();
                issue_ab(lds0, min(kt + 8, KT - 1));
                compute_mx16(lds1, scl1, 16, 3, std::false_type{});
                step_end();
            }
            __syncthreads();   // no copy may still be writing LDS when the workgroup ends
            goto epilogue;
        }
    }
    if constexpr (!kPair) {
    if (KT > 0) {
    issue_step(lds0, scl0, 0);
    put_scales(scl0);
    __syncthreads();

    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
        issue_step(lds1, scl1, kt + 1);
        compute(lds0, scl0);
        put_scales(scl1);
        lds_barrier_keep_vm<0>();
        issue_step(lds0, scl0, min(kt + 2, KT - 1));
        compute(lds1, scl1);
        put_scales(scl0);
        lds_barrier_keep_vm<0>();
    }
    if (kt < KT)
        compute(lds0, scl0);
    __syncthreads();   // no copy may still be writing LDS when the workgroup ends
    }
    }
    // K not a multiple of the step (operands copied straight into LDS, and
    // for block-scaled kinds the SB scale path; the host launches no other
    // configuration for it): one more step after the loop whose K values
    // beyond K are copied as zeros into both operands, so they add nothing.
    if constexpr (!kMx || SB) {
        if (K % kStepK) {
            lds_barrier_keep_vm<0>();   // every copy landed, every wave done reading lds0
            // bytes of each K-major row's step slice inside K (whole 16-byte chunks)
            const uint32_t lim = uint32_t(K % kStepK) * 128 / kStepK;
            if constexpr (kDmaA)
                da.issue_tail(lds0, KT, lim, wave, lane);
            if constexpr (kTrA)
                dma_mna.issue_tail(lds0, KT, K, wave, lane);
            if constexpr (kDmaB)
                db.issue_tail(lds0, KT, lim, wave, lane);
            if constexpr (kTrB)
                dma_mnb.issue_tail(lds0, KT, K, wave, lane);
            load_scale_bytes(KT);
            put_scales(scl0);
            lds_barrier_keep_vm<0>();
            compute(lds0, scl0);
        }
    }

    // ---- epilogue -------------------------------------------------------------
epilogue:
    const bool opts_on = opts.neg || opts.row_mask || opts.col_zero;
    if constexpr (kStagedEpi) {
        // Byte-row blocks give each row's lanes two runs of 8 columns, too
        // small a piece for non-temporal stores, and the other blocks 16
        // columns (64 bytes), so the tile goes through
        // the (now idle) operand stages: each wave writes a quarter of its
        // 128 x 64 tile (32 rows, fragment blocks 2q and 2q+1) into its own
        // 32-row area (waves 0-3 in lds0, 4-7 in lds1; 16-byte chunks
        // XOR-keyed by row so that writes and reads hit distinct banks), reads
        // it back as 4 rows x 256 bytes per instruction and stores those
        // non-temporally.  The lanes of one wave exchange values through
        // its area, so each quarter's writes and reads are separated by a
        // wave-level LDS fence (wave_lds_sync); the workgroup barrier keeps
        // the last K step's reads of the stages before the first write.
        __syncthreads();
        static_assert(4 * 32 * kEpiPitch <= uint32_t(kStage), "four 32-row areas per stage");
        uint8_t *area = (wave < 4 ? lds0 : lds1) + (wave & 3) * 32 * kEpiPitch;
        const int rd_row = lane >> 4, rd_col = 4 * (lane & 15);
        // With beta = 1 the quarter's eight pieces of the old D are loaded
        // before its LDS round trip, all at once: loaded one by one next to
        // their stores, each load's whole memory latency was waited for in
        // turn (8192^3 fp16 with beta: 899.5 -> 884.6 us).  Outputs beyond M
        // or N load D[0] instead (always inside D) and store nothing.
        auto piece = [&](int q, int k) {
            const int m = m0 + wm + 32 * q + 4 * k + rd_row, n = n0 + wn + rd_col;
            return m < M && n < N ? size_t(m) * ldd + n : ~size_t(0);
        };
        // (The K-tail kernels (SB), short of registers, load each piece with
        // its store.  Issuing quarter q + 1's loads before quarter q's round
        // trip measured 0.6 % slower than this on 8192^3 fp16 with beta.)
        constexpr bool kBatchOld = BETA && !SB;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4 old[kBatchOld ? 8 : 1];
            if constexpr (kBatchOld) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const size_t idx = piece(q, k);
                    old[k] = load_d4<OUT>(D, idx == ~size_t(0) ? 0 : idx);
                }
            }
#pragma unroll
            for (int j = 0; j < TN16; ++j)
#pragma unroll
                for (int ii = 0; ii < 2; ++ii)
                    *reinterpret_cast<f32x4 *>(area + epi_write_offset<kRowsA, kRowsB>(q, ii, j, lane)) = acc4[j][2 * q + ii];
            wave_lds_sync();
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                f32x4 v = *reinterpret_cast<const f32x4 *>(area + epi_read_offset(k, lane));
                const size_t idx = piece(q, k);
                if (idx == ~size_t(0))
                    continue;
                const int m = m0 + wm + 32 * q + 4 * k + rd_row, n = n0 + wn + rd_col;
                if (opts_on && !apply_opts(opts, m, n, v))
                    continue;
                if constexpr (kBatchOld)
                    v += old[k];
                store_d4<OUT, BETA && !kBatchOld, true>(D, idx, v, opts.sat);
            }
            wave_lds_sync();   // the next quarter's writes come after these reads
        }
        return;
    }
    if constexpr (kMf16) {
        // 16x16 block (j, i): lane l holds fragment row l % 16 of A block i
        // and fragment rows 4(l/16) .. +3 of B block j
        // (with beta = 1 a block row's old D is loaded before its stores, as
        // in the staged epilogue; outputs beyond M or N load D[0] and store
        // nothing)
        constexpr bool kBatchOld = BETA && !SB;
#pragma unroll
        for (int j = 0; j < TN16; ++j) {
            f32x4 old[kBatchOld ? TM16 : 1];
            if constexpr (kBatchOld) {
#pragma unroll
                for (int i = 0; i < TM16; ++i) {
                    const int m = m0 + wm + row16<kRowsA>(i, lane & 15);
                    const int n = n0 + wn + row16<kRowsB>(j, 4 * (lane >> 4));
                    old[i] = load_d4<OUT>(D, m < M && n < N ? size_t(m) * ldd + n : 0);
                }
            }
#pragma unroll
            for (int i = 0; i < TM16; ++i) {
                const int m = m0 + wm + row16<kRowsA>(i, lane & 15);
                const int n = n0 + wn + row16<kRowsB>(j, 4 * (lane >> 4));
                if (m >= M || n >= N)
                    continue;
                f32x4 v = acc4[j][i];
                if (opts_on && !apply_opts(opts, m, n, v))
                    continue;
                if constexpr (kBatchOld)
                    v += old[i];
                // 16-bit and E2M1 blocks: the four lanes of a row hold 16
                // consecutive columns (64 bytes of fp32 D); byte-row blocks:
                // two runs of 8, and 16-bit D halves the piece
                store_d4<OUT, BETA && !kBatchOld, !(kRowsA || kRowsB) && OUT == kOutF32>(D, size_t(m) * ldd + n, v,
                                                                                         opts.sat);
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = m0 + wm + 32 * i + lr;
            f32x4 old[BETA ? 4 : 1];
            if constexpr (BETA) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n0 + wn + 32 * j + 8 * q + 4 * lh;
                    old[q] = load_d4<OUT>(D, m < M && n < N ? size_t(m) * ldd + n : 0);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn + 32 * j + 8 * q + 4 * lh;
                if (m >= M || n >= N)
                    continue;
                f32x4 v = {acc[j][i][4 * q + 0], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                           acc[j][i][4 * q + 3]};
                if (opts_on && !apply_opts(opts, m, n, v))
                    continue;
                if constexpr (BETA)
                    v += old[q];
                store_d4<OUT, false>(D, size_t(m) * ldd + n, v, opts.sat);
            }
        }
}

// 16x16 MFMAs for every operand kind, except 16-bit operands that are both
// MN-major, which take 32x32x16 (their 16x16 fragment reads would need more
// than 256 VGPRs).
template <int KIND, bool A_MN, bool B_MN, int OUT = kOutF32, int KB = -1, int SV = 32, bool SB = false,
          bool SM = false, bool WO = false>
hipError_t launch_kind(const MxArgs &a, hipStream_t stream)
{
    constexpr bool kMf16 = !(A_MN && B_MN);
    const int tiles_m = (a.M + kBM - 1) / kBM, tiles_n = (a.N + kBN - 1) / kBN;
    const int blocks = tiles_m * tiles_n;
    const uint8_t *A = static_cast<const uint8_t *>(a.A);
    const uint8_t *B = static_cast<const uint8_t *>(a.B);
    if (a.beta)
        hipLaunchKernelGGL((gemm256_kernel<KIND, A_MN, B_MN, true, kMf16, OUT, KB, SV, SB, SM, WO>), dim3(blocks), dim3(64 * W),
                           0, stream, A, B, a.SFA, a.SFB, a.D, a.M, a.N, a.K, a.lda, a.ldb, a.ldd, tiles_m,
                           tiles_n, a.group_m, a.opts);
    else
        hipLaunchKernelGGL((gemm256_kernel<KIND, A_MN, B_MN, false, kMf16, OUT, KB, SV, SB, SM, WO>), dim3(blocks), dim3(64 * W),
                           0, stream, A, B, a.SFA, a.SFB, a.D, a.M, a.N, a.K, a.lda, a.ldb, a.ldd, tiles_m,
                           tiles_n, a.group_m, a.opts);
    return hipGetLastError();
}

// D's element kind chosen at run time
template <int KIND, bool A_MN, bool B_MN, int KB = -1, int SV = 32, bool SB = false, bool SM = false,
          bool WO = false>
hipError_t launch_out(const MxArgs &a, hipStream_t stream)
{
    switch (a.out) {
    case kOutBf16: return launch_kind<KIND, A_MN, B_MN, kOutBf16, KB, SV, SB, SM, WO>(a, stream);
    case kOutF16: return launch_kind<KIND, A_MN, B_MN, kOutF16, KB, SV, SB, SM, WO>(a, stream);
    default: return launch_kind<KIND, A_MN, B_MN, kOutF32, KB, SV, SB, SM, WO>(a, stream);
    }
}

// Block-scaled kinds with a K that is not a multiple of their K step take
// the SB variant (scale words assembled in registers).
template <int KIND, bool A_MN, bool B_MN, int KB = -1, int SV = 32>
hipError_t launch_cfg(const MxArgs &a, hipStream_t stream)
{
    // E4M3 with dense E2M1: K is a multiple of 256 (no SB variant)
    constexpr bool kPairKinds = (KIND == kE4m3 && KB == kE2m1) || (KIND == kE2m1 && KB == kE4m3);
    if constexpr (KIND != kBf16 && KIND != kF16 && !kPairKinds) {
        constexpr int kStep = KIND == kE2m1 ? 256 : 128;
        if (a.K % kStep != 0)
            return launch_out<KIND, A_MN, B_MN, KB, SV, true>(a, stream);
    }
    return launch_out<KIND, A_MN, B_MN, KB, SV, false>(a, stream);
}

}  // namespace
}  // namespace mswz
