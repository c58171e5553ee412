// layout.hpp — operand address functions shared by the gfx950 kernels and the
// host-side checks.  Everything here is constexpr and usable on host and device.
//
// Two families live here:
//
// 1. The shared-descriptor byte walk and its swizzle modes as the pages define
//    them (tcgen05.cp page, "Shared descriptor address walk"; tcgen05.mma
//    page, "Shared descriptors are byte-stride contracts").  Before swizzling,
//    row r of a descriptor starts at (r / 8) * group_stride + (r % 8) * (16 << s)
//    bytes; an unswizzled walk adds (w / 4) * chunk_stride + (w % 4) * 4 for
//    32-bit word w, a swizzled walk adds 4 * w.  K-major and MN-major swizzled
//    descriptors use SDO as the row-group stride and LDO as the chunk stride;
//    MN-major unswizzled swaps the two.  Mode 4 (32-bit MN-major) groups four
//    128-byte K rows per SDO and steps LDO per 128-byte M/N chunk.  The final
//    address is the swizzle of origin + walk.
//    Swizzle modes: 0 identity; 1/2/3 move 16-byte chunk c of row j inside a
//    256/512/1024-byte period to c ^ (j >> (3 - s)) (only the periods are
//    printed on the pages; this is the reading that keeps 16-byte atoms whole
//    with exactly those periods); mode 4 is the printed
//    offset ^ ((offset >> 2) & 96) with a 512-byte period.
//
// 2. The LDS operand-tile layout the kernels stage A and B tiles in.  A tile
//    row holds 128 bytes of one M/N row (64 16-bit or 128 8-bit K elements) —
//    the mode-3 geometry: 128-byte rows, 8-row groups 1024 bytes apart, rows
//    contiguous.  The 16-byte chunk c of row r sits at chunk c ^ key(r) with
//    key(r) = (r ^ (r >> 3)) & 7: the row-in-group index of mode 3 further
//    XORed with the group index.  That extension keeps the wave-wide 16-byte
//    MFMA operand reads (32 consecutive rows, one chunk per half-wave) and the
//    staging writes free of bank conflicts under both 32-bank/8-lane and
//    64-bank/16-lane cycle models, and makes the transposed MN-major staging
//    writes conflict free under the first.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define MSWZ_HD __host__ __device__ __forceinline__
#else
#define MSWZ_HD inline
#endif

namespace mswz {

// ---- pages' descriptor walk --------------------------------------------------

enum : int { kMajorK = 0, kMajorMN = 1 };

MSWZ_HD constexpr int64_t swizzle_period(int mode)
{
    return mode == 1 ? 256 : mode == 2 ? 512 : mode == 3 ? 1024 : mode == 4 ? 512 : 16;
}

MSWZ_HD constexpr int64_t swizzle(int mode, int64_t off)
{
    switch (mode) {
    case 1: return off ^ ((off >> 3) & 0x10);
    case 2: return off ^ ((off >> 3) & 0x30);
    case 3: return off ^ ((off >> 3) & 0x70);
    case 4: return off ^ ((off >> 2) & 0x60);
    default: return off;
    }
}

// Byte address of 32-bit word w of descriptor row r.
MSWZ_HD constexpr int64_t desc_address(int64_t r, int64_t w, int64_t ldo, int64_t sdo,
                                       int mode, int major, int64_t origin)
{
    const bool swap = (major == kMajorMN) && (mode == 0);
    const int64_t group_stride = swap ? ldo : sdo;
    const int64_t chunk_stride = swap ? sdo : ldo;
    int64_t pre;
    if (mode == 4) {
        pre = (r >> 2) * group_stride + (r & 3) * 128 + (w >> 5) * chunk_stride + (w & 31) * 4;
    } else {
        pre = (r >> 3) * group_stride + (r & 7) * (int64_t(16) << mode);
        pre += (mode == 0) ? (w >> 2) * chunk_stride + (w & 3) * 4 : 4 * w;
    }
    return swizzle(mode, origin + pre);
}

// Descriptor field checks (tcgen05.cp page, same section; tcgen05.mma page,
// same section): strides are nonnegative 16-byte multiples below 2^18,
// origins 16-byte aligned, swizzled origins aligned to the full period.
// Returns 0 when valid, otherwise the number of the first failed rule.
MSWZ_HD constexpr int desc_check(int64_t ldo, int64_t sdo, int mode, int64_t origin)
{
    if (mode < 0 || mode > 4) return 1;
    if (ldo < 0 || sdo < 0 || (ldo & 15) || (sdo & 15)) return 2;
    if (ldo >= (int64_t(1) << 18) || sdo >= (int64_t(1) << 18)) return 3;
    if (origin < 0 || (origin & 15)) return 4;
    if (mode != 0 && (origin % swizzle_period(mode)) != 0) return 5;
    return 0;
}

// ---- kernels' LDS operand tile -------------------------------------------------

constexpr uint32_t kTileRowBytes = 128;

MSWZ_HD constexpr uint32_t tile_key(uint32_t row) { return (row ^ (row >> 3)) & 7u; }

// Byte offset of 16-byte chunk `chunk` (0..7) of tile row `row`.
MSWZ_HD constexpr uint32_t tile_offset(uint32_t row, uint32_t chunk)
{
    return row * kTileRowBytes + ((chunk ^ tile_key(row)) << 4);
}

}  // namespace mswz
