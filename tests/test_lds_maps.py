"""The 256x256 kernel's LDS layouts and fragment maps, checked on the CPU bit
for bit (no GPU).

mswz.lds_lanes returns the per-lane LDS addresses of each wave-wide access
the kernel issues, computed by the same address functions the kernel calls
(csrc/layout.hpp).  Each test simulates the data movement: a step's operand
slice is copied into LDS by the copy instructions' (destination, source)
pairs, then read back by the fragment reads, and every lane must receive
exactly the rows and K values that its MFMA operand image requires (the
images are the ones pinned on the GPU by one-wave probes and stated in
csrc/device_common.hpp).  The tile layouts on the LDS side are enumerated
independently by oracle/walk.py.

Bank model (measured with SQ_LDS_BANK_CONFLICT on five read patterns): a
16-byte-per-lane access is served in four passes of 16 lanes, each pass the
lanes that agree in lane bits 1 and 5, over 64 banks of 4 bytes; an access
is conflict-free when, within every pass, distinct words fall in distinct
banks (identical words broadcast).  16-byte writes are served 8 consecutive
lanes at a time: with that, and a cost of (degree - 1) cycles per pass, the
model reproduces exactly the counts measured for two earlier layouts of the
staged epilogue (test_write_model_reproduces_measured_epilogue_conflicts).  Byte reads are modelled as served 32
banks at a time for all 64 lanes (this fits the measured conflicts of the
E4M3 scale reads and their absence for the dense E2M1 ones).  Transposing
8-byte reads are modelled as two passes of 32 lanes (half waves) over 64
banks; this model is not calibrated.
"""
import itertools

import numpy as np
import pytest

import mma_swizzled_operand_amd as mswz
from oracle import walk

KTILE = walk.lds_tile_bruteforce(256)          # [row][chunk] -> byte offset (K-major tile)
MNTILE = walk.mn_tile_bruteforce()             # [k][chunk] -> byte offset (MN-major tile)
K_INV = {int(KTILE[r, c]): (r, c) for r in range(256) for c in range(8)}
MN_INV = {int(MNTILE[k, c]): (k, c) for k in range(64) for c in range(32)}


def kblk(g):
    """K-block order of the 16x16x32 fragments stated in layout.hpp."""
    return 2 * (g & 1) + (g >> 1)


def conflicts(addrs, width, passes):
    """Worst number of distinct words in one bank within a pass."""
    worst = 1
    for lanes in passes:
        banks = {}
        for l in lanes:
            for w in range(max(width // 4, 1)):
                word = addrs[l] // 4 + w
                banks.setdefault(word % 64 if width >= 4 else word % 32, set()).add(word)
        worst = max(worst, max(len(s) for s in banks.values()))
    return worst


def extra_cycles(addrs, width, passes):
    """Modelled conflict cycles of one access: sum over passes of (degree - 1)."""
    return sum(conflicts(addrs, width, [p]) - 1 for p in passes)


PASSES_16 = [[l for l in range(64) if ((l >> 1) & 1) == b1 and (l >> 5) == b5] for b1 in (0, 1) for b5 in (0, 1)]
PASSES_W16 = [list(range(8 * p, 8 * p + 8)) for p in range(8)]
PASSES_8 = [list(range(32)), list(range(32, 64))]
PASSES_1 = [list(range(64))]


def pairs(pattern, p0, p1=0):
    v = mswz.lds_lanes(pattern, p0, p1)
    return v[0::2], v[1::2]


# ---- copies ----------------------------------------------------------------------

def test_kmajor_copies_fill_the_tile_once_with_the_layouts_chunks():
    seen = set()
    for q in range(32):
        dst, src = pairs("dma_k", q)
        assert dst == [1024 * q + 16 * l for l in range(64)]          # 1 KiB contiguous per instruction
        for d, s in zip(dst, src):
            row, chunk = s // 128, (s % 128) // 16
            assert KTILE[row, chunk] == d                              # the chunk the layout puts there
            seen.add(d)
    assert seen == set(range(0, 256 * 128, 16))


def test_mn_major_copies_fill_the_tile_once_with_the_layouts_chunks():
    seen = set()
    for q in range(32):
        dst, src = pairs("dma_mn", q)
        assert dst == [1024 * q + 16 * l for l in range(64)]
        for d, s in zip(dst, src):
            k, chunk = s // 512, (s % 512) // 16
            assert MNTILE[k, chunk] == d
            seen.add(d)
    assert seen == set(range(0, 64 * 512, 16))


# ---- fragment reads -----------------------------------------------------------------

@pytest.mark.parametrize("b", range(16))
def test_16bit_kmajor_fragments(b):
    """16x16x32 operand: lane (r, g) holds row 16b + r and 8 consecutive K
    values; the K block depends on g and the sub-step only (so A and B, read
    the same way, meet), and the four groups and two sub-steps cover the 64 K
    values of the step once."""
    ks_of = {}
    for ks in range(2):
        addrs = mswz.lds_lanes("frag_k16", b, ks)
        assert conflicts(addrs, 16, PASSES_16) == 1
        for l, a in enumerate(addrs):
            row, chunk = K_INV[a]
            assert row == 16 * b + l % 16
            ks_of.setdefault((ks, l >> 4), set()).add(chunk)
    assert all(len(v) == 1 for v in ks_of.values())
    assert sorted(c for v in ks_of.values() for c in v) == list(range(8))
    assert all(ks_of[(ks, g)] == {4 * ks + kblk(g)} for ks in range(2) for g in range(4))


def transposed_read(addrs):
    """ds_read_b64_tr_b16 as pinned by the probe: in each 16-lane group,
    lanes 4j .. 4j+3 name four 8-byte pieces (16 values v_j); lane t of the
    group receives (v_0[t], v_1[t], v_2[t], v_3[t]).  Values are returned as
    (K row, M column) of the MN-major tile."""
    def values(a):
        k, chunk = MN_INV[a - a % 16]
        first = 8 * chunk + (a % 16) // 2
        return [(k, first + e) for e in range(4)]
    out = []
    for l in range(64):
        grp, t = l & ~15, l & 15
        out.append([(values(addrs[grp + 4 * j + t // 4]))[t % 4] for j in range(4)])
    return out


@pytest.mark.parametrize("b", range(16))
def test_16bit_mn_major_fragments_through_transposing_reads(b):
    """MN-major operand read with two transposing reads: lane (r, g) holds M
    row 16b + r and K rows 32 ks + 8 kblk(g) + 0..7 (the same K order as the
    K-major operand, so a K-major partner meets it)."""
    for ks in range(2):
        v = mswz.lds_lanes("frag_mn16", b, ks)
        first, second = v[0::2], v[1::2]
        assert conflicts(first, 8, PASSES_8) == 1 and conflicts(second, 8, PASSES_8) == 1
        got = [x + y for x, y in zip(transposed_read(first), transposed_read(second))]
        for l, vals in enumerate(got):
            g = l >> 4
            assert [m for _, m in vals] == [16 * b + l % 16] * 8
            assert [k for k, _ in vals] == [32 * ks + 8 * kblk(g) + e for e in range(8)]


def e4m3_image_ok(reads, b):
    """E4M3 16x16x128 operand image: lane (r, g) holds row row16(b, r) (two
    runs of 8 rows 16 apart), bytes 0..15 in 32-element scale block g/2 and
    bytes 16..31 in block 2 + g/2; over the four groups every chunk of the
    128-byte step is read once per row."""
    first, second = reads[0::2], reads[1::2]
    per_row = {}
    for l in range(64):
        r, g = l & 15, l >> 4
        row_a, c_a = K_INV[first[l]]
        row_b, c_b = K_INV[second[l]]
        want_row = 32 * (b >> 1) + 8 * (b & 1) + (r & 7) + 16 * (r >> 3)
        assert row_a == want_row and row_b == want_row
        assert c_a // 2 == g // 2 and c_b // 2 == 2 + g // 2
        per_row.setdefault(row_a, []).extend([c_a, c_b])
    assert all(sorted(v) == list(range(8)) for v in per_row.values())
    return first, second


@pytest.mark.parametrize("b", range(16))
def test_e4m3_fragments(b):
    first, second = e4m3_image_ok(mswz.lds_lanes("frag_e4m3", b), b)
    assert conflicts(first, 16, PASSES_16) == 1 and conflicts(second, 16, PASSES_16) == 1


@pytest.mark.parametrize("b", range(16))
def test_padded_fragments(b):
    """Padded 6- and 4-bit operand image: lane (r, g) holds the 32 values of
    scale block g, chunks 2g and 2g + 1 of its row (sixteen values each)."""
    v = mswz.lds_lanes("frag_pad", b)
    first, second = v[0::2], v[1::2]
    assert conflicts(first, 16, PASSES_16) == 1 and conflicts(second, 16, PASSES_16) == 1
    for l in range(64):
        r, g = l & 15, l >> 4
        (ra, ca), (rb, cb) = K_INV[first[l]], K_INV[second[l]]
        assert ra == rb == 32 * (b >> 1) + 8 * (b & 1) + (r & 7) + 16 * (r >> 3)
        assert {ca, cb} == {2 * g, 2 * g + 1}


@pytest.mark.parametrize("b", range(16))
def test_mixed_e4m3_fragments_meet_their_padded_partners(b):
    """E4M3 paired with a padded kind: values meet by the MFMA's internal K
    index (32 g + j for value j of padded lane group g; 32 (g/2) + 16 (g%2) + j,
    plus 64 for bytes 16..31, for byte j of an E4M3 lane), so every internal
    index must name the same memory K on both sides."""
    e = mswz.lds_lanes("frag_e4m3_mixed", b)
    p = mswz.lds_lanes("frag_pad", b)
    assert conflicts(e[0::2], 16, PASSES_16) == 1 and conflicts(e[1::2], 16, PASSES_16) == 1
    for r in range(16):
        mem_e, mem_p = {}, {}
        for g in range(4):
            l = 16 * g + r
            for half, a in enumerate(e[2 * l:2 * l + 2]):
                _, c = K_INV[a]
                for j in range(16):
                    mem_e[32 * (g >> 1) + 16 * (g & 1) + 64 * half + j] = 16 * c + j
            for half, a in enumerate(p[2 * l:2 * l + 2]):
                _, c = K_INV[a]
                for j in range(16):
                    mem_p[32 * g + 16 * half + j] = 16 * c + j
        assert mem_e == mem_p and sorted(mem_e.values()) == list(range(128))


@pytest.mark.parametrize("b", range(16))
def test_e4m3_fragments_meet_their_dense_e2m1_partners(b):
    """E4M3 paired with dense E2M1: the E2M1 tile row (128 bytes) holds two
    E4M3 steps, read in halves h.  E2M1 lane (r, g) holds internal K 32g + j,
    j < 32, in one 16-byte chunk; E4M3 byte j of lane (r, g) internal K
    32(g/2) + 16(g%2) + j, plus 64 for the second read.  Every internal K
    must name the same step-local memory K on both sides, the E2M1 chunk must
    lie in half h, and both reads must be conflict-free."""
    e = mswz.lds_lanes("frag_e4m3_fp4", b)
    assert conflicts(e[0::2], 16, PASSES_16) == 1 and conflicts(e[1::2], 16, PASSES_16) == 1
    for h in range(2):
        f = mswz.lds_lanes("frag_e2m1", b, h)
        assert conflicts(f, 16, PASSES_16) == 1
        for r in range(16):
            mem_e, mem_f = {}, {}
            for g in range(4):
                l = 16 * g + r
                for half, a in enumerate(e[2 * l:2 * l + 2]):
                    row, c = K_INV[a]
                    assert row == 32 * (b >> 1) + 8 * (b & 1) + (r & 7) + 16 * (r >> 3)
                    for j in range(16):
                        mem_e[32 * (g >> 1) + 16 * (g & 1) + 64 * half + j] = 16 * c + j
                row, c = K_INV[f[l]]
                assert row == 16 * b + r and c // 4 == h
                for j in range(32):
                    mem_f[32 * g + j] = 32 * c + j - 128 * h
            assert mem_e == mem_f and sorted(mem_e.values()) == list(range(128))


@pytest.mark.parametrize("b", range(16))
def test_e2m1_fragments(b):
    """Dense E2M1: lane (r, g) holds one 16-byte chunk = one 32-element scale
    block of row 16b + r; groups and sub-steps cover the step's 8 blocks once."""
    blocks = set()
    for ks in range(2):
        addrs = mswz.lds_lanes("frag_e2m1", b, ks)
        assert conflicts(addrs, 16, PASSES_16) == 1
        for l, a in enumerate(addrs):
            row, c = K_INV[a]
            assert row == 16 * b + l % 16
            if l % 16 == 0:
                blocks.add(c)
    assert blocks == set(range(8))


# ---- scales --------------------------------------------------------------------------

def test_grouped_scale_slots_put_each_fragment_rows_scales_where_they_are_read():
    """Grouped scale stage (16 bytes per row: four K steps of four blocks):
    wave w copies row sf_slot_row(l) of 64-row group w into slot l; a lane of
    fragment block b, row x, reads slot 16 b + x.  The slot must hold that
    fragment row's scales, byte g + 4 s its block g of step s."""
    holder = {}
    for w in range(8):
        dst, rows = pairs("scale_dma", w)
        for d, r in zip(dst, rows):
            holder[d // 16] = 64 * (w & 3) + r + (256 if w >= 4 else 0)   # stage slot -> operand row
    assert sorted(holder) == list(range(512))
    for b in range(8):
        for s in range(4):
            addrs = mswz.lds_lanes("scale_grp", b, s)
            for l, a in enumerate(addrs):
                x, g = l & 15, l >> 4
                assert holder[a // 16] == 32 * (b >> 1) + 8 * (b & 1) + (x & 7) + 16 * (x >> 3)
                assert a % 16 == g + 4 * s


def test_grouped_scale_reads_conflict_two_ways_under_the_byte_model():
    """The 16 rows of a fragment block sit in 16-byte slots, 4 words apart:
    under the byte model (32 banks) rows x and x + 8 share a bank.  This is
    the measured source of the E4M3 kernels' LDS bank-conflict cycles."""
    for b in range(8):
        assert conflicts(mswz.lds_lanes("scale_grp", b, 0), 1, PASSES_1) == 2


def _wide_holder(pattern):
    """Stage byte -> (operand row, scale byte) after the wide copies of one
    group: copy q of wave w writes 1 KiB; lane l's 16 bytes are half h of a
    row's 32 scale bytes (eight E4M3 / padded steps, four E2M1 steps)."""
    holder = {}
    for w in range(8):
        for q in range(2):
            dst, src = pairs(pattern, w, q)
            assert dst == [2048 * w + 1024 * q + 16 * l for l in range(64)]   # 1 KiB contiguous
            rows = {r // 2 for r in src}
            assert len(rows) == 32                       # 32 rows, both halves of each: one line per row
            for d, r in zip(dst, src):
                row, h = r // 2, r % 2
                for byte in range(16):
                    holder[d + byte] = (64 * (w & 3) + row + (256 if w >= 4 else 0), 16 * h + byte)
    assert sorted(holder) == list(range(512 * 32))
    return holder


def test_wide_scale_slots_put_each_fragment_rows_scales_where_they_are_read():
    """32-byte-per-row stage of the 6-bit kinds (slot order of sf_slot_row):
    every byte that lane (x, g) of fragment block b reads at step s of its
    group of eight is byte 4 s + g of that fragment row's 32 scale bytes."""
    holder = _wide_holder("scale_dma_wide")
    for b in range(8):
        for st in range(8):
            for l, a in enumerate(mswz.lds_lanes("scale_grp_wide", b, st)):
                x, g = l & 15, l >> 4
                assert holder[a] == (32 * (b >> 1) + 8 * (b & 1) + (x & 7) + 16 * (x >> 3), 4 * st + g)


def test_wide_fp4_scale_slots_put_each_fragment_rows_scales_where_they_are_read():
    """Dense E2M1 (rows in order): the byte lane (x, g) of block b reads at
    step s of its group of four, sub-step u, is byte 8 s + 4 u + kblk16(g) of
    row 16 b + x's 32 scale bytes (a step's eight 32-element blocks)."""
    holder = _wide_holder("scale_dma_wide_nat")
    for b in range(8):
        for st in range(4):
            for u in range(2):
                for l, a in enumerate(mswz.lds_lanes("scale_fp4_wide", b, 2 * st + u)):
                    x, g = l & 15, l >> 4
                    assert holder[a] == (16 * b + x, 8 * st + 4 * u + kblk(g))


def test_wide_scale_reads_conflict_two_ways_under_the_byte_model():
    """Within a half the slots sit 16 bytes apart as in the 16-byte stage, so
    the reads keep its two-way conflict and no more."""
    for b in range(8):
        for st in (0, 5):
            assert conflicts(mswz.lds_lanes("scale_grp_wide", b, st), 1, PASSES_1) == 2
            assert conflicts(mswz.lds_lanes("scale_fp4_wide", b, st), 1, PASSES_1) == 2


def _mn_holder():
    """Stage byte -> (operand row, K block of the 32-block group) after the
    MN-major scale copies of one group (scales stored [K block][row]): copy q
    of wave w writes 1 KiB; lane l's 16 bytes are one K block's scales of 16
    consecutive rows."""
    holder = {}
    for w in range(8):
        for q in range(2):
            dst, src = pairs("scale_dma_mn", w, q)
            assert dst == [2048 * w + 1024 * q + 16 * l for l in range(64)]   # 1 KiB contiguous
            blocks = {}
            for r in src:
                blocks.setdefault(r // 256, set()).add(r % 256)
            # four K blocks, each all 256 rows: four 256-byte runs of memory
            assert len(blocks) == 4 and all(v == set(range(0, 256, 16)) for v in blocks.values())
            for d, r in zip(dst, src):
                for byte in range(16):
                    holder[d + byte] = (r % 256 + byte + (256 if w >= 4 else 0), r // 256)
    assert sorted(holder) == list(range(512 * 32))
    assert sorted(set(holder.values())) == [(row, g) for row in range(512) for g in range(32)]
    return holder


def test_mn_scale_copies_put_each_fragment_rows_scales_where_they_are_read():
    """MN-major scales, E4M3 and padded kinds (split-row fragments): the byte
    lane (x, g) of fragment block b reads at step s of its group of eight is
    K block 4 s + g of that fragment row."""
    holder = _mn_holder()
    for b in range(8):
        for st in range(8):
            for l, a in enumerate(mswz.lds_lanes("scale_grp_mn", b, st)):
                x, g = l & 15, l >> 4
                assert holder[a] == (32 * (b >> 1) + 8 * (b & 1) + (x & 7) + 16 * (x >> 3), 4 * st + g)


def test_mn_fp4_scale_copies_put_each_fragment_rows_scales_where_they_are_read():
    """MN-major scales, dense E2M1 (rows in order): lane (x, g) of block b at
    step s of its group of four, sub-step u, reads K block 8 s + 4 u +
    kblk16(g) of row 16 b + x."""
    holder = _mn_holder()
    for b in range(8):
        for st in range(4):
            for u in range(2):
                for l, a in enumerate(mswz.lds_lanes("scale_fp4_mn", b, 2 * st + u)):
                    x, g = l & 15, l >> 4
                    assert holder[a] == (16 * b + x, 8 * st + 4 * u + kblk(g))


def test_mn_scale_reads_are_conflict_free_under_the_byte_model():
    """The four K blocks of one read sit in four consecutive chunks (and a
    split block's second run four chunks further), so the 64 byte reads
    touch distinct banks or share a word."""
    for b in range(8):
        for st in range(8):
            assert conflicts(mswz.lds_lanes("scale_grp_mn", b, st), 1, PASSES_1) == 1
            assert conflicts(mswz.lds_lanes("scale_fp4_mn", b, st), 1, PASSES_1) == 1


def test_mn_scale_patterns_reject_out_of_range_arguments():
    for pat, p0, p1 in (("scale_dma_mn", 8, 0), ("scale_dma_mn", 0, 2), ("scale_grp_mn", 8, 0),
                        ("scale_grp_mn", 0, 8), ("scale_fp4_mn", -1, 0)):
        with pytest.raises(mswz.MswzError):
            mswz.lds_lanes(pat, p0, p1)


# ---- staged epilogue -------------------------------------------------------------------

@pytest.mark.parametrize("rows", [0, 1, 2, 3])
def test_staged_epilogue_writes_every_output_of_a_quarter_once_where_it_is_read(rows):
    """Register r of 16x16 block (i, j) in lane l is output row row16(i, l % 16),
    column row16(j, 4 (l/16)) + r of the wave's tile (the MFMA output image,
    B first operand), row16 split or contiguous on each side (rows: 0 both
    contiguous, 1 both split, 2 split M only, 3 split N only).  A quarter q's 32 x 64 outputs are written once into the
    wave's area and the read-back instructions return each (row, 4 columns)
    piece to the lane that stores row 4k + l/16, columns 4 (l%16) .. +3.
    Writes and reads are conflict-free under the 16-byte models."""
    split_m, split_n = rows in (1, 2), rows in (1, 3)

    def r16(split, b, x):
        return 32 * (b >> 1) + 8 * (b & 1) + (x & 7) + 16 * (x >> 3) if split else 16 * b + x
    for q in range(4):
        where = {}
        for ii, j in itertools.product(range(2), range(4)):
            addrs = mswz.lds_lanes("epi_write", q, 16 * rows + 4 * ii + j)
            assert conflicts(addrs, 16, PASSES_W16) == 1
            for l, a in enumerate(addrs):
                m = r16(split_m, 2 * q + ii, l % 16) - 32 * q
                n = r16(split_n, j, 4 * (l >> 4))
                for reg in range(4):
                    assert (a + 4 * reg) not in where
                    where[a + 4 * reg] = (m, n + reg)
        assert sorted(where.values()) == [(m, n) for m in range(32) for n in range(64)]
        for k in range(8):
            addrs = mswz.lds_lanes("epi_read", k)
            assert conflicts(addrs, 16, PASSES_16) == 1
            for l, a in enumerate(addrs):
                assert [where[a + 4 * e] for e in range(4)] == [(4 * k + l // 16, 4 * (l % 16) + e) for e in range(4)]


def _epilogue_cycles(pitch, key):
    """Modelled conflict cycles of one wave's staged epilogue (16-bit blocks:
    4 quarters x 8 writes, then 8 reads each) for a row pitch in bytes and a
    chunk key of the row."""
    total = 0
    for q in range(4):
        for ii, j in itertools.product(range(2), range(4)):
            w = []
            for l in range(64):
                row, chunk = 16 * ii + l % 16, 4 * j + (l >> 4)
                w.append(row * pitch + 16 * (chunk ^ key(row)))
            total += extra_cycles(w, 16, PASSES_W16)
        for k in range(8):
            r = []
            for l in range(64):
                row = 4 * k + (l >> 4)
                r.append(row * pitch + 16 * ((l & 15) ^ key(row)))
            total += extra_cycles(r, 16, PASSES_16)
    return total


def test_write_model_reproduces_measured_epilogue_conflicts():
    """SQ_LDS_BANK_CONFLICT per dispatch of bf16 8192^3 (1024 tiles of 8
    waves; the K loop's reads are modelled conflict-free) measured 1048576
    with rows 272 bytes apart and no key, and 2097152 with 256-byte rows and
    the key 2 r0 + 4 r2 + 8 (r3 ^ r4) (r_i: bit i of the row).  Reads alone
    (16-lane passes) explain the first; writes served 8 consecutive lanes at
    a time explain the second, while 16-lane passes by lane bits 1 and 5 for
    writes would predict 0 for it."""
    per_dispatch = 1024 * 8
    assert _epilogue_cycles(272, lambda r: 0) * per_dispatch == 1048576
    old_key = lambda r: 2 * (r & 1) + 4 * ((r >> 2) & 1) + 8 * (((r >> 3) ^ (r >> 4)) & 1)
    assert _epilogue_cycles(256, old_key) * per_dispatch == 2097152
    lib_key = lambda r: ((r & 1) << 1) | ((r >> 1) & 1) | (r & 4)
    assert _epilogue_cycles(256, lib_key) == 0


def test_lane_map_export_rejects_bad_arguments():
    with pytest.raises(mswz.MswzError):
        mswz.lds_lanes("dma_k", 32)
    with pytest.raises(mswz.MswzError):
        mswz.lds_lanes("frag_k16", 0, 2)
    lib = mswz.load()
    assert lib.mswz_lds_lanes(99, 0, 0, None, 0) == -1
