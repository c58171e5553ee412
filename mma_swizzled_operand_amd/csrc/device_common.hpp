// device_common.hpp — vector types, MFMA wrappers and the workgroup -> tile
// mapping shared by the gfx950 GEMM kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.hpp"

namespace mswz {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// 32x32x16 MFMA on 16-bit operands, fp32 accumulate.  Operand lane l holds
// 8 consecutive K elements of row l % 32 (K half l / 32); both operands use
// the same lane -> K assignment, so any K order inside the instruction gives
// the same sum of products.
template <bool BF16>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c)
{
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// 16x16x32 MFMA on 16-bit operands, fp32 accumulate.  Operand lane l holds 8
// consecutive K elements of row l % 16 (K group l / 16); the 16x16 result
// sits in 4 registers per lane: register r of lane l is row 4*(l/16) + r of
// the first operand's rows, column l % 16 of the second's.
template <bool BF16>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Block-scaled 32x32x64 MFMA on OCP E4M3 operands (format code 0 for both).
// Lane l holds K elements 16h..16h+15 and 32+16h..32+16h+15 (h = l / 32) of
// row l % 32; the scale of K block h of that row is byte SEL of lane l's
// 32-bit scale operand.
template <int SEL>
__device__ __forceinline__ f32x16 mfma_scale_32x32x64_e4m3(i32x8 a, i32x8 b, f32x16 c,
                                                          int scale_a, int scale_b)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SEL, scale_a, SEL, scale_b);
}

// Block-scaled 16x16x128 MFMA, scale byte 0 of each scale register, the
// first and second operands in formats F1 and F2 (E4M3 0, E2M3 2, E3M2 3,
// E2M1 4).  Lane images (each pinned by a one-wave probe):
//   E4M3: lane l holds 32 bytes of row l % 16: bytes 0..15 lie in 32-wide
//         scale block (l/16)/2 and bytes 16..31 in block 2 + (l/16)/2;
//   E2M3 / E3M2: 32 values of row l % 16, value j in bits 6j .. 6j+5 of
//         registers 0..5, all in scale block l/16;
//   E2M1: 32 values, value j in bits 4j .. 4j+3 of registers 0..3, all in
//         scale block l/16;
// and in every case lane i + 16b supplies row i's scale for block b.  Across
// formats, values meet by an internal K index: 32g + j for value j of lane
// group g of a 6- or 4-bit operand, 32(g/2) + 16(g%2) + j (plus 64 for bytes
// 16..31) for byte j of an E4M3 lane.
template <int F1, int F2>
__device__ __forceinline__ f32x4 mfma_scale_16x16x128_fmt(i32x8 a, i32x8 b, f32x4 c, int scale_a, int scale_b)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, F1, F2, 0, scale_a, 0, scale_b);
}

// The same MFMA with OCP E2M1 (FP4) operands (format code 4): lane l holds
// 32 elements (16 bytes, low nibble first) of row l % 16 in the low four
// registers of each operand, all in scale block l/16, and lane i + 16b
// supplies row i's scale for block b.
__device__ __forceinline__ f32x4 mfma_scale_16x16x128_e2m1(i32x8 a, i32x8 b, f32x4 c, int scale_a,
                                                           int scale_b)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, scale_a, 0, scale_b);
}

// Workgroup -> output tile.  The hardware hands consecutive workgroups to the
// eight XCDs in turn (workgroup b runs on XCD b % 8), and each XCD has its own
// L2.  Tile ids are therefore re-ordered so that each XCD receives one
// contiguous run of ids, and ids are rastered in groups of `group_m` tile rows
// (column by column inside a group) so that the workgroups resident on one XCD
// at the same time share a few A row panels and B column panels.
//
// group_m < 0 selects a two-dimensional split instead: the tile grid is cut
// into a 2 x 4 grid of regions (when both counts divide), XCD x takes region
// (x / 4, x % 4), and inside a region tiles are rastered in groups of
// -group_m tile rows.  Then each A row panel is fetched by 4 XCDs and each B
// column panel by 2, instead of 1 and 8.
__host__ __device__ __forceinline__ void tile_of_block(int b, int tiles_m, int tiles_n, int group_m,
                                                       int &tm, int &tn)
{
    const int T = tiles_m * tiles_n;
    if (group_m < 0 && (tiles_m & 1) == 0 && (tiles_n & 3) == 0) {
        const int rm = tiles_m >> 1, rn = tiles_n >> 2;   // region size in tiles
        const int x = b & 7, t = b >> 3;                 // XCD, index inside its region
        const int g = -group_m;
        const int per_group = g * rn;
        const int gi = t / per_group;
        const int first = gi * g;
        const int gm = rm - first < g ? rm - first : g;
        const int r = t - gi * per_group;
        tm = (x >> 2) * rm + first + r % gm;
        tn = (x & 3) * rn + r / gm;
        return;
    }
    group_m = group_m < 0 ? -group_m : group_m;
    int t = b;
    if ((T & 7) == 0)
        t = (b & 7) * (T >> 3) + (b >> 3);
    const int per_group = group_m * tiles_n;
    const int g = t / per_group;
    const int first_m = g * group_m;
    const int gm = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    const int r = t - g * per_group;
    tm = first_m + r % gm;
    tn = r / gm;
}

// Buffer resource for raw (unstructured) buffer loads: base address, no
// stride, `bytes` valid bytes (reads beyond it return zero), gfx9-family
// word 3 (32-bit data format, raw addressing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane l writes LDS bytes
// [lds + 16*l, +16) (lds is wave-uniform); the source is base + voffset + soffset.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, uint8_t *lds,
                                                  uint32_t voffset, uint32_t soffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                             voffset, soffset, 0, 0);
}

// 4 bytes per lane from a buffer straight into LDS: lane l writes LDS bytes
// [lds + 4*l, +4).
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t r, uint8_t *lds,
                                                 uint32_t voffset, uint32_t soffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4,
                                             voffset, soffset, 0, 0);
}

// Workgroup barrier for LDS pipelines: waits until at most `VM` of this
// wave's vector-memory loads (the most recently issued ones) are still in
// flight and all its LDS operations are done, then joins the barrier.  The
// memory clobber keeps the compiler from moving memory operations across it.
// The wait is the s_waitcnt builtin, which the compiler's own wait-count
// tracking sees, so it does not wait for the same loads again later.
// Encoding (gfx9 family): vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
template <int VM>
__device__ __forceinline__ void lds_barrier_keep_vm()
{
    static_assert(VM >= 0 && VM < 64, "vmcnt is 6 bits");
    constexpr int kEnc = (VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (0 << 8);
    __builtin_amdgcn_s_waitcnt(kEnc);
    asm volatile("s_barrier" ::: "memory");
}

// Orders one wave's LDS accesses across its lanes: every lane's LDS writes
// before the call are visible to every lane's LDS reads after it (and reads
// before it are done before writes after it).  Needed where lanes of one wave
// exchange data through LDS, since from one lane's point of view its own
// accesses to different addresses are independent and could be reordered.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Scheduling fence: no instruction is moved across it by the compiler.
__device__ __forceinline__ void sched_fence()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                               uint32_t soffset)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, 0));
}

__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                                 uint32_t soffset)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, voffset, soffset, 0);
}

// Make a value opaque to the optimiser for one use site, so that values
// derived from it (per sub-step LDS addresses) are recomputed where they are
// used instead of being hoisted out of the K loop and held in registers.
template <typename T>
__device__ __forceinline__ T opaque(T v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// 16-byte LDS read / write.
__device__ __forceinline__ u32x4 lds_read16(const uint8_t *lds, uint32_t off)
{
    return *reinterpret_cast<const u32x4 *>(lds + off);
}
__device__ __forceinline__ void lds_write16(uint8_t *lds, uint32_t off, u32x4 v)
{
    *reinterpret_cast<u32x4 *>(lds + off) = v;
}
// Transposing 8-byte LDS read of 16-bit values (ds_read_b64_tr_b16).  In
// each group of 16 lanes, lanes 4j .. 4j+3 name four 8-byte pieces, i.e. 16
// values v_j[0..15] in lane order; lane t of the group receives
// (v_0[t], v_1[t], v_2[t], v_3[t]).  So four lanes per row pointing at 16
// consecutive values of rows r0 .. r0+3 give lane t the column t of that 4x16
// block.
__device__ __forceinline__ u32x2 lds_read8(const uint8_t *lds, uint32_t off)
{
    return *reinterpret_cast<const u32x2 *>(lds + off);
}
__device__ __forceinline__ u32x3 lds_read12(const uint8_t *lds, uint32_t off)
{
    return *reinterpret_cast<const u32x3 *>(lds + off);
}
__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t *lds, uint32_t off)
{
    auto *p = (__attribute__((address_space(3))) i16x4 *)(lds + off);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
}

__device__ __forceinline__ u32x4 global_read16(const uint8_t *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

// Transpose an 8x8 block of 16-bit values held as eight 16-byte rows:
// out[i] element j = in[j] element i.
__device__ __forceinline__ void transpose8x8_b16(const u32x4 in[8], u32x4 out[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t lo = in[2 * p][i >> 1];
            const uint32_t hi = in[2 * p + 1][i >> 1];
            out[i][p] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                : ((lo & 0xffffu) | (hi << 16));
        }
    }
}

}  // namespace mswz
