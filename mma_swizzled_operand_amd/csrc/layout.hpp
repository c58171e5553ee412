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

// Direct global -> LDS copy of a K-major tile: wave instruction q (of any
// wave) fills LDS bytes [1024 q, 1024 q + 1024) contiguously, lane l writing
// 16 bytes at 1024 q + 16 l, i.e. position l % 8 of tile row 8 q + l / 8.
// The lane therefore fetches the source chunk that the layout puts there
// (the permutation is its own inverse).
MSWZ_HD constexpr uint32_t dma_row(int q, int lane) { return uint32_t(8 * q + (lane >> 3)); }
MSWZ_HD constexpr uint32_t dma_chunk(int q, int lane) { return uint32_t((lane & 7) ^ (((lane >> 3) ^ q) & 7)); }

// ---- MN-major operand tile ([K][R] storage, R = M or N) ----------------------
// One K step is 64 K rows of 512 bytes (256 16-bit values); 16-byte chunk c of
// K row k (values 8c .. 8c+7) sits at position c ^ mn_key(k).  A wave
// instruction fills two K rows (1 KiB) contiguously: instruction q, lane l
// writes position l % 32 of K row 2q + l / 32.
constexpr uint32_t kMnRowBytes = 512;
MSWZ_HD constexpr uint32_t mn_key(uint32_t k) { return (4u * (k & 3u)) ^ (2u * ((k >> 4) & 1u)); }
MSWZ_HD constexpr uint32_t mn_tile_offset(uint32_t k, uint32_t chunk)
{
    return k * kMnRowBytes + ((chunk ^ mn_key(k)) << 4);
}
MSWZ_HD constexpr uint32_t dma_mn_krow(int q, int lane) { return uint32_t(2 * q + (lane >> 5)); }
MSWZ_HD constexpr uint32_t dma_mn_chunk(int q, int lane)
{
    return uint32_t(lane & 31) ^ mn_key(dma_mn_krow(q, lane));
}

// ---- MFMA fragment maps of the 256x256 kernel ----------------------------------
// K-block order of the 16x16x32 fragments: lane group g = l/16 of that MFMA
// supplies 8 K values of its row, the 8-value block kblk16(g) = 2*(g%2) + g/2
// of the 32-wide sub-step, the same for A and B (a sum over K does not depend
// on the order of its terms).  With the natural order the 16-byte reads of
// lanes 8p .. 8p+7 and 32+8p .. 32+8p+7, which are served together, would hit
// the same banks; with this order the two chunks differ in their lowest bit.
MSWZ_HD constexpr int kblk16(int g) { return 2 * (g & 1) + (g >> 1); }

// First-half chunk of lane group g for the block-scaled 16x16x128 MFMA on
// E4M3 (second half: chunk + 4).  The chunk must lie in scale block g/2, so
// groups 0 and 1 (2 and 3) read chunks that differ only in their lowest bit;
// E4M3 fragments therefore take their 16 rows from two runs of 8 rows 16
// apart (row16) and groups g and g + 2 take chunks of different parity.
MSWZ_HD constexpr int mx_chunk16(int g) { return 2 * (g >> 1) + ((g & 1) ^ (g >> 1)); }

// First chunk of lane group g for the block-scaled MFMA on the padded kinds
// (sixteen values per 16-byte chunk; the second chunk is this one ^ 1): lane
// (row i, group g) holds the 32 values of scale block g, chunks 2g and 2g+1,
// taken in the other order for g = 0 and 2, which keeps the reads of the
// split-row fragments free of bank conflicts.
MSWZ_HD constexpr int fp6_chunk16(int g) { return 2 * g + ((g & 1) ^ 1); }

// First-half chunk of lane group g of an E4M3 operand paired with a padded
// kind (second half: chunk + 4).  Values meet by an internal K index: 32g + j
// for value j of lane group g of a 6- or 4-bit operand, 32(g/2) + 16(g%2) + j
// for byte j < 16 of an E4M3 lane (64 more for bytes 16..31); with the padded
// operand in fp6_chunk16 order this order makes partners share their memory
// K position, and is free of bank conflicts with the split-row fragments.
MSWZ_HD constexpr int mx_chunk16_mixed(int g) { return (g >> 1) ? g : g ^ 1; }

// First-half chunk of lane group g of an E4M3 operand paired with dense
// E2M1 (second half: chunk ^ 2).  The E2M1 operand's lane group g holds the
// 32 values of its step block kblk16(g) (one 16-byte chunk) at internal K
// index 32g + j; the E4M3 lanes' internal indices (32(g/2) + 16(g%2) + j,
// plus 64 for bytes 16..31) then name memory K 16 * pair_chunk16(g) + j and,
// for the second half, that + 32: groups (0, 1, 2, 3) read chunks
// (0, 1, 4, 5) and (2, 3, 6, 7).
MSWZ_HD constexpr int pair_chunk16(int g) { return (g & 1) + 4 * (g >> 1); }

// Tile row (relative to the wave's first row) of row x (0..15) of 16-row
// fragment block b: 16-bit operands use 16 consecutive rows; the byte-row
// (E4M3 and padded) operands rows 32*(b/2) + 8*(b%2) + {0..7, 16..23}.  Runs
// of 4 consecutive x stay consecutive rows, so the epilogue still stores 16
// bytes per lane.
template <bool MX>
MSWZ_HD constexpr int row16(int b, int x)
{
    return MX ? 32 * (b >> 1) + 8 * (b & 1) + (x & 7) + 16 * (x >> 3) : 16 * b + x;
}

// Scale-stage slot of row l of a 64-row group when each row's scales take 16
// bytes (four K steps): l with bits 3 and 4 swapped (an involution).  A scale
// read of 16-row fragment block b touches rows row16<true>(b, x), x = 0..15:
// bits 0-2 and 4 from x, bits 3 and 5 from b; in this order they are the 16
// consecutive slots 16 b + x.
MSWZ_HD constexpr int sf_slot_row(int l) { return (l & ~24) | ((l & 8) << 1) | ((l & 16) >> 1); }

// Scale stage with 32 bytes per row (eight E4M3 / padded K steps, or four
// E2M1 steps), in two 16-byte halves h: byte offset of slot `slot` (0..511),
// half h.  Each 32-slot block holds the first halves of its slots, then the
// second halves, so that one 16-byte copy instruction fetches both halves of
// 32 rows (two lanes per row, in one cache line) and writes them to 1 KiB of
// consecutive LDS; within a half, slots sit 16 bytes apart as in the
// 16-byte stage.
MSWZ_HD constexpr uint32_t sf_wide_offset(uint32_t slot, uint32_t h)
{
    return (slot >> 5) * 1024u + h * 512u + (slot & 31u) * 16u;
}

// The byte lane l reads from a wide stage for fragment block b of the
// 16-row blocks that start at slot slot0 (a multiple of 32): slot
// slot0 + 16b + l%16, at byte `byte` of the slot's half h.  For such slot0
// the offset splits into a per-lane part (b = 0, h = 0, byte 0), a per-block
// part (slot0 = 0, lane 0) and the half and byte, which the kernels add as
// immediates.
MSWZ_HD constexpr uint32_t sf_wide_read(uint32_t slot0, int b, uint32_t h, uint32_t byte, int lane)
{
    return sf_wide_offset(slot0 + 16u * uint32_t(b) + uint32_t(lane & 15), h) + byte;
}
static_assert(sf_wide_read(96, 5, 1, 7, 13) ==
                  sf_wide_read(96, 0, 0, 0, 13) + sf_wide_read(0, 5, 0, 0, 0) + sf_wide_offset(0, 1) + 7,
              "wide scale reads split into lane, block and half parts");

// Scale stage for scales stored MN-major, [K block][row] (the pages'
// canonical SFA / SFB order, tcgen05.mma page, "Operands and repeat axes":
// the K-repeat axis outside the rows): per operand 32 K blocks (eight E4M3 /
// padded K steps, four E2M1 steps) of 256 rows, 8 KiB.  A 16-byte chunk holds
// the scales of 16 consecutive rows for one K block; K block g, rows
// 16r .. 16r+15 sit at chunk 64 (g/4) + 4r + g%4, so the chunks of four
// consecutive K blocks and one 16-row run are consecutive.  One 16-byte copy
// instruction (sf_mn_copy_block, sf_mn_copy_row) fetches four K blocks of all
// 256 rows, i.e. four 256-byte runs of memory (8 cache lines, against 32 for
// the row-major wide stage), and writes 1 KiB of consecutive LDS.  A byte read
// for four K blocks of 16 rows lands in distinct bank groups (the K block
// picks the chunk's position among four, and a split 16-row block's two runs
// are four chunks apart), so it is free of conflicts under the byte model.
MSWZ_HD constexpr uint32_t sf_mn_offset(uint32_t g, uint32_t row)
{
    return (g >> 2) * 1024u + (row >> 4) * 64u + (g & 3u) * 16u + (row & 15u);
}
// lane l of copy instruction i (K blocks 4i .. 4i+3 of the stage): K block
// and first row of its 16-byte chunk
MSWZ_HD constexpr uint32_t sf_mn_copy_block(int i, int l) { return 4u * uint32_t(i) + uint32_t(l & 3); }
MSWZ_HD constexpr uint32_t sf_mn_copy_row(int l) { return 16u * uint32_t(l >> 2); }
static_assert(sf_mn_offset(sf_mn_copy_block(5, 39), sf_mn_copy_row(39)) == 1024u * 5 + 16u * 39,
              "copy lane l of instruction i writes LDS bytes 1024 i + 16 l");
// The reads add a per-lane part (K block within the group of four, first row
// of the lane), a per-fragment-block part and a per-step part: no carries
// between them for the fragments' rows (row16) and steps.
template <bool MX>
MSWZ_HD constexpr bool sf_mn_reads_split()
{
    for (uint32_t wm = 0; wm < 256; wm += 64)
        for (int b = 0; b < (MX ? 8 : 4); ++b)
            for (int x = 0; x < 16; ++x)
                for (uint32_t q = 0; q < 4; ++q)
                    for (uint32_t t = 0; t < 8; ++t)
                        if (sf_mn_offset(4 * t + q, wm + uint32_t(row16<MX>(b, x))) !=
                            sf_mn_offset(q, wm + uint32_t(row16<MX>(0, x))) + sf_mn_offset(0, uint32_t(row16<MX>(b, 0))) +
                                sf_mn_offset(4 * t, 0))
                            return false;
    return true;
}
static_assert(sf_mn_reads_split<true>() && sf_mn_reads_split<false>(),
              "MN-major scale reads split into lane, block and step parts");

// LDS byte offset, at sub-step 0 and first half, of this lane's piece of the
// 32-row 32x32x16 MFMA fragment whose tile rows start at rbase (a multiple of
// 32) in an MN-major tile, read with ds_read_b64_tr_b16.  The operand wants,
// in lane l, row l % 32 and K values 8*(l/32) .. +7.  With lane t = l % 16 =
// 4j + a of its group, the lane points at K row 8*(l/32) + j, values
// rbase + 16*((l/16) % 2) + 4a .. +3; the transposing read then hands lane l
// row rbase + l % 32 and K values 8*(l/32) .. +3.  The second half (K + 4)
// is 4 rows further, sub-step ks 16*ks rows further and, as bit 4 of its K
// rows is ks % 2, with its chunk XOR 2 (byte offset XOR 32) for odd ks.
MSWZ_HD constexpr uint32_t mn_frag_base(uint32_t tile_off, int rbase, int lane)
{
    const int t = lane & 15, j = t >> 2, a = t & 3, g1 = (lane >> 4) & 1, h = lane >> 5;
    const int chunk = rbase / 8 + 2 * g1 + (a >> 1);
    return tile_off + uint32_t(8 * h + j) * kMnRowBytes + (uint32_t(chunk ^ (4 * j)) << 4) + 8 * (a & 1);
}

// The same for the 16-row fragment of the 16x16x32 MFMA in an MN-major tile:
// lane t = l % 16 = 4j + a of group g points at K row 8*kblk16(g) + j (bit 4
// of which is g % 2), values rbase + 4a .. +3; the second half is 4 K rows
// further, sub-step s 32*s rows further.
MSWZ_HD constexpr uint32_t mn_frag_base16(uint32_t tile_off, int rbase, int lane)
{
    const int t = lane & 15, j = t >> 2, a = t & 3, g = lane >> 4;
    const int chunk = (rbase / 8 + (a >> 1)) ^ (4 * j) ^ (2 * (g & 1));
    return tile_off + uint32_t(8 * kblk16(g) + j) * kMnRowBytes + (uint32_t(chunk) << 4) + 8 * (a & 1);
}

// K-major fragment read base of 16x16 block b: tile rows rbase +
// row16<MX>(b, l % 16), 16-byte chunk `chunk` (the lane group's, see the
// chunk orders above).  Sub-steps and second halves are this base XOR a
// constant: 16-bit and E2M1 sub-step s: ^ (s << 6); E4M3 second half: ^ 64;
// padded kinds' second chunk: ^ 16.
template <bool MX>
MSWZ_HD constexpr uint32_t kfrag_base(uint32_t tile_off, int rbase, int b, int chunk, int lane)
{
    return tile_off + tile_offset(uint32_t(rbase + row16<MX>(b, lane & 15)), uint32_t(chunk));
}

// ---- staged epilogue ------------------------------------------------------------
// Each wave writes a quarter q of its 128 x 64 fp32 tile (32 rows) into its
// own 8 KiB area, rows kEpiPitch = 256 bytes apart, then reads it back as 4
// rows x 256 bytes per instruction.  16-byte chunk c of row r sits at chunk
// c ^ epi_key(r), epi_key(r) = row bits 0 and 1 swapped, bit 2 kept.
// Measured bank behaviour (SQ_LDS_BANK_CONFLICT on two layouts of this
// epilogue, together with the calibrated read model): a 16-byte write is
// served 8 consecutive lanes at a time, a 16-byte read 16 lanes at a time,
// the lanes that agree in lane bits 1 and 5.  A write's 8 lanes hold rows
// that differ in bits 0..2 and one chunk, so the key's bijection on those
// bits puts them in 8 distinct 4-bank groups; a read's 16 lanes hold rows
// that differ in bit 0 and chunks that differ in bits 0, 2 and 3, and the
// key moves row bit 0 to chunk bit 1.
constexpr uint32_t kEpiPitch = 256;
MSWZ_HD constexpr uint32_t epi_key(uint32_t row)
{
    return ((row & 1u) << 1) | ((row >> 1) & 1u) | (row & 4u);
}
// the 16 bytes (4 columns) of 16x16 block (i = 2q + ii, j) that lane l holds;
// MXM / MXN: split-row fragments on the M (A) / N (B) side
template <bool MXM, bool MXN = MXM>
MSWZ_HD constexpr uint32_t epi_write_offset(int q, int ii, int j, int lane)
{
    const uint32_t row = uint32_t(row16<MXM>(2 * q + ii, lane & 15) - 32 * q);
    const uint32_t chunk = uint32_t(row16<MXN>(j, 4 * (lane >> 4))) / 4;
    return row * kEpiPitch + ((chunk ^ epi_key(row)) << 4);
}
// read-back instruction k: lane l reads row 4k + l/16, columns 4(l%16) .. +3
MSWZ_HD constexpr uint32_t epi_read_offset(int k, int lane)
{
    const uint32_t row = uint32_t(4 * k + (lane >> 4));
    return row * kEpiPitch + ((uint32_t(lane & 15) ^ epi_key(row)) << 4);
}

}  // namespace mswz
