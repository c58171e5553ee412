"""Address-walk and swizzle pins (CPU only).

Part 1 pins the oracle's brute-force enumerators (oracle/walk.py) to what the
pages print: the tcgen05.cp page's example descriptor, the tcgen05.mma page's
example descriptors and its printed mode-4 permutation, and the stated
periods and 16-byte atoms.

Part 2 (further down) checks the GPU library's own address functions, which
the kernels use, bit for bit against those enumerators.
"""
import itertools

import numpy as np
import pytest

from oracle import walk


# ---- part 1: brute force vs the pages ---------------------------------------

def test_cp_page_example_descriptor_is_plain_16_byte_rows():
    """tcgen05.cp page example: a (128,4) uint32 image in the default layout
    copied with ldo=16, sdo=128, swizzle=0 — the walk is byte 16*r + 4*w."""
    addr = walk.desc_walk_bruteforce(128, 4, ldo=16, sdo=128, mode=0)
    r, w = np.meshgrid(np.arange(128), np.arange(4), indexing="ij")
    assert np.array_equal(addr, 16 * r + 4 * w)


def test_mma_page_example_descriptor_rows_are_128_bytes_before_swizzle():
    """tcgen05.mma page example: (128,64) and (64,64) fp16 K-major tiles with
    descriptor (16, 1024, 3): before the swizzle, row r starts at 128*r and its
    64 halves (32 words) are contiguous."""
    for rows in (128, 64):
        # swizzled modes add 4*w per word, so the pre-swizzle walk is contiguous
        sw = np.array([[(r // 8) * 1024 + (r % 8) * 128 + 4 * w for w in range(32)] for r in range(rows)])
        assert np.array_equal(np.sort(sw.ravel()), np.arange(rows * 32) * 4)
        phys = walk.desc_walk_bruteforce(rows, 32, ldo=16, sdo=1024, mode=3, major="k")
        # swizzle keeps each row inside its own 128-byte line and 16-byte chunks whole
        assert np.array_equal(phys // 128, sw // 128)
        assert np.array_equal(phys % 16, sw % 16)
        assert len(set(phys.ravel().tolist())) == rows * 32


def test_mode4_table_equals_printed_formula():
    """tcgen05.mma page: mode 4 permutes offset -> offset ^ ((offset >> 2) & 96)."""
    for off in range(4096):
        assert walk.swizzle_bruteforce(4, off) == off ^ ((off >> 2) & 96)


@pytest.mark.parametrize("mode", [1, 2, 3, 4])
def test_swizzle_is_periodic_bijective_involutive_and_keeps_atoms(mode):
    P = walk.PERIOD[mode]
    atom = 32 if mode == 4 else 16
    img = [walk.swizzle_bruteforce(mode, x) for x in range(4 * P)]
    assert sorted(img) == list(range(4 * P))                       # bijection
    for x in range(4 * P):
        assert walk.swizzle_bruteforce(mode, img[x]) == x            # involution
        assert img[x] % atom == x % atom                             # atom kept
        assert img[x] // P == x // P                                 # stays in its period
        if x + P < 4 * P:
            assert img[x + P] == img[x] + P                          # periodicity
    # the period is the smallest one (the permutation is not the identity)
    assert img[:P] != list(range(P))


def test_mode0_is_identity():
    assert all(walk.swizzle_bruteforce(0, x) == x for x in range(4096))


def test_stride_roles_table():
    """tcgen05.mma page stride-role table."""
    assert walk.stride_roles("k", 0) == ("sdo", "ldo")
    assert walk.stride_roles("k", 3) == ("sdo", "ldo")
    assert walk.stride_roles("mn", 2) == ("sdo", "ldo")
    assert walk.stride_roles("mn", 0) == ("ldo", "sdo")


def test_mn_major_unswizzled_swaps_roles():
    a = walk.desc_walk_bruteforce(16, 8, ldo=512, sdo=64, mode=0, major="mn")
    # row group stride is LDO (512), chunk stride is SDO (64)
    assert a[8, 0] - a[0, 0] == 512
    assert a[0, 4] - a[0, 0] == 64
    b = walk.desc_walk_bruteforce(16, 8, ldo=512, sdo=64, mode=0, major="k")
    assert b[8, 0] - b[0, 0] == 64
    assert b[0, 4] - b[0, 0] == 512


def test_lds_tile_layout_bruteforce_properties():
    t = walk.lds_tile_bruteforce(256)
    assert sorted(t.ravel().tolist()) == list(range(0, 256 * 128, 16))   # bijection onto the tile
    assert np.array_equal(t // 128, np.arange(256)[:, None].repeat(8, 1))  # rows stay in place
    # for rows < 8 the key is the row index: the page's mode-3 geometry
    assert [walk.lds_tile_key_table()[r] for r in range(8)] == list(range(8))


@pytest.mark.parametrize("banks,group", [(32, 8), (64, 16)])
def test_lds_tile_layout_conflict_free_for_kernel_accesses(banks, group):
    """Modelled bank conflicts of the kernels' wave-wide 16-byte LDS accesses
    under the two candidate bank models (32 banks / 8 lanes per cycle, 64
    banks / 16 lanes per cycle): MFMA operand reads (lane l reads row l%32,
    chunk c0 + l//32) and staging writes (lane l writes row l//8, chunk l%8)."""
    t = walk.lds_tile_bruteforce(256)
    for r0, c0 in itertools.product(range(0, 256, 32), range(0, 8, 2)):
        addrs = [t[r0 + l % 32, c0 + l // 32] for l in range(64)]
        assert walk.bank_conflict_degree(addrs, 16, banks, group) == 1
    for r0 in range(0, 256, 8):
        addrs = [t[r0 + l // 8, l % 8] for l in range(64)]
        assert walk.bank_conflict_degree(addrs, 16, banks, group) == 1
