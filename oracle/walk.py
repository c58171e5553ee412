"""Brute-force address-walk enumerators — TEST INFRASTRUCTURE ONLY (oracle side).

Everything here is built from the textual definitions with explicit loops and
explicit per-period permutation tables.  Nothing here uses the shift-and-mask
form the GPU library uses, so a wrong shift, mask or stride role in the GPU
library's address functions shows up as a mismatch.

Sources
-------
* tcgen05.cp page, "Shared descriptor address walk": before swizzling, row r
  starts at (r div 8)*SDO + (r mod 8)*(16 << s) bytes; without swizzle word w
  adds (w div 4)*LDO + (w mod 4)*4, with swizzle it adds 4*w (LDO unused);
  swizzle periods are 256/512/1024 bytes for modes 1/2/3.
* tcgen05.mma page, "Shared descriptors are byte-stride contracts": the
  row-group / contiguous-chunk stride roles per major (K-major: SDO/LDO;
  MN-major swizzled: SDO/LDO; MN-major unswizzled: LDO/SDO); mode 4 groups
  four 128-byte K rows per SDO, takes LDO to the next 128-byte M/N chunk and
  permutes 32-byte atoms with a 512-byte period, printed as a formula.

Reading taken for modes 1..3 (the page prints only their periods): within one
period the 16-byte chunk c of row j (j = 0..7 inside the period) moves to
chunk c XOR (j div 2^(3-s)).  That keeps 16-byte atoms whole and has exactly
the stated periods.  Parity of modes 1..3 beyond those two properties is
unpinned.

The GPU kernels' own LDS tile layout (rows of 128 bytes, eight 16-byte chunks
per row, one chunk permutation per row) is enumerated by ``lds_tile_bruteforce``.
"""
from __future__ import annotations

import numpy as np

ROW_BYTES = {0: 16, 1: 32, 2: 64, 3: 128}   # 16 << s for modes 0..3
PERIOD = {1: 256, 2: 512, 3: 1024, 4: 512}   # swizzle periods


def _chunk_perm_table(mode: int) -> list[list[int]]:
    """perm[j][c]: destination 16-byte chunk of chunk c in row j of a period
    (modes 1..3), built row by row."""
    rows_per_period = 8
    chunks_per_row = ROW_BYTES[mode] // 16
    step = 2 ** (3 - mode)          # rows that share one XOR key
    table = []
    for j in range(rows_per_period):
        key = j // step
        table.append([c ^ key for c in range(chunks_per_row)])
    return table


def _atom_perm_table_mode4() -> list[list[int]]:
    """Mode 4: a 512-byte period holds four 128-byte rows of four 32-byte
    atoms; atom a of row j moves to atom a XOR j."""
    return [[a ^ j for a in range(4)] for j in range(4)]


def swizzle_bruteforce(mode: int, offset: int) -> int:
    """Physical byte offset of a pre-swizzle byte offset, by table lookup."""
    if mode == 0:
        return offset
    base = (offset // PERIOD[mode]) * PERIOD[mode]
    inner = offset - base
    if mode == 4:
        row, rest = divmod(inner, 128)
        atom, byte = divmod(rest, 32)
        return base + row * 128 + _atom_perm_table_mode4()[row][atom] * 32 + byte
    row, rest = divmod(inner, ROW_BYTES[mode])
    chunk, byte = divmod(rest, 16)
    return base + row * ROW_BYTES[mode] + _chunk_perm_table(mode)[row][chunk] * 16 + byte


def stride_roles(major: str, mode: int) -> tuple[str, str]:
    """(row-group stride, contiguous-chunk stride) field names per the page's table."""
    if major == "k":
        return ("sdo", "ldo")
    if mode == 0:
        return ("ldo", "sdo")
    return ("sdo", "ldo")


def desc_walk_bruteforce(rows: int, words: int, ldo: int, sdo: int, mode: int,
                         major: str = "k", origin: int = 0) -> np.ndarray:
    """Physical byte address of b32 word (r, w) for every r < rows, w < words.

    Modes 0..3 follow the cp page's row/word walk, with the row-group and
    chunk strides assigned by major per the mma page's table; mode 4 follows
    the mma page's four-rows-per-SDO, 128-byte-chunk-per-LDO walk.  ``origin``
    is the (already inverse-swizzled) descriptor origin added before the
    swizzle, so the final address is swizzle(origin + walk).
    """
    group_field, chunk_field = stride_roles(major, mode)
    strides = {"ldo": ldo, "sdo": sdo}
    group_stride = strides[group_field]
    chunk_stride = strides[chunk_field]
    out = np.zeros((rows, words), dtype=np.int64)
    for r in range(rows):
        for w in range(words):
            if mode == 4:
                pre = (r // 4) * group_stride + (r % 4) * 128
                pre += (w // 32) * chunk_stride + (w % 32) * 4
            else:
                pre = (r // 8) * group_stride + (r % 8) * ROW_BYTES[mode]
                if mode == 0:
                    pre += (w // 4) * chunk_stride + (w % 4) * 4
                else:
                    pre += 4 * w
            out[r, w] = swizzle_bruteforce(mode, origin + pre)
    return out


# ---- the GPU kernels' LDS operand-tile layout ---------------------------------

def lds_tile_key_table() -> list[int]:
    """XOR key of each row inside the 64-row super-period of the kernels'
    tile layout: key(row) = (row mod 8) XOR (row div 8), for row < 64."""
    return [(r % 8) ^ (r // 8) for r in range(64)]


def lds_tile_bruteforce(rows: int) -> np.ndarray:
    """Byte offset of 16-byte chunk (row, c) of a [rows][128 B] operand tile:
    rows are 128 bytes apart; chunk c lands at chunk position c XOR key(row),
    with the key table repeating every 64 rows."""
    keys = lds_tile_key_table()
    out = np.zeros((rows, 8), dtype=np.int64)
    for r in range(rows):
        perm = [c ^ keys[r % 64] for c in range(8)]
        for c in range(8):
            out[r, c] = r * 128 + perm[c] * 16
    return out


def bank_conflict_degree(byte_addrs, access_bytes: int, banks: int, lanes_per_cycle: int) -> int:
    """Worst number of distinct 4-byte words that share one bank within any
    group of ``lanes_per_cycle`` consecutive lanes (identical words broadcast).
    1 means conflict free under the model (``banks`` banks of 4 bytes)."""
    worst = 1
    addrs = list(byte_addrs)
    for g in range(0, len(addrs), lanes_per_cycle):
        per_bank: dict[int, set[int]] = {}
        for a in addrs[g:g + lanes_per_cycle]:
            for w in range(access_bytes // 4):
                word = a // 4 + w
                per_bank.setdefault(word % banks, set()).add(word)
        worst = max(worst, max(len(s) for s in per_bank.values()))
    return worst


def mn_tile_key_table() -> list[int]:
    """Chunk XOR key of each K row of the kernels' MN-major tile (64 K rows of
    32 chunks): 4 x (k mod 4), with the bit of value 2 set for K rows 16..31
    and 48..63 (the half of a 32-row block that the odd sub-step's fragments
    read)."""
    table = []
    for k in range(64):
        key = [0, 4, 8, 12][k % 4]
        if (k // 16) % 2 == 1:
            key ^= 2
        table.append(key)
    return table


def mn_tile_bruteforce() -> np.ndarray:
    """Byte offset of 16-byte chunk (k, c) of an MN-major tile of 64 K rows of
    512 bytes: chunk c lands at chunk position c XOR key(k)."""
    keys = mn_tile_key_table()
    out = np.zeros((64, 32), dtype=np.int64)
    for k in range(64):
        for c in range(32):
            out[k, c] = k * 512 + (c ^ keys[k]) * 16
    return out
