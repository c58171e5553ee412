"""C ABI checks that need no GPU (CPU only).

* libmswz.so loads and exports every function include/mswz_gemm.h declares;
* every rejection gemm_plan_create / gemm_run / gemm_run_blockscaled document
  happens on the host, before any GPU work (fake, never-dereferenced pointer
  values are enough to reach them);
* the library's address functions — the pages' descriptor walk and the
  kernels' LDS tile layout — equal the oracle's brute-force enumerations bit
  for bit (tcgen05.cp page, "Shared descriptor address walk"; tcgen05.mma
  page, "Shared descriptors are byte-stride contracts").
"""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import mma_swizzled_operand_amd as mswz
from oracle import walk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mswz_gemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_abi():
    names = declared_functions()
    for required in ("gemm_plan_create", "gemm_run", "gemm_run_blockscaled", "gemm_plan_destroy",
                     "gemm_status_str", "gemm_plan_describe", "mswz_desc_address",
                     "mswz_desc_check", "mswz_tile_offset"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mswz.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        s = mswz.gemm_status_str(code)
        assert s and s != "unknown status"
    assert mswz.gemm_status_str(7) == "unknown status"


# ---- plan creation ------------------------------------------------------------

def _create(*args):
    lib = mswz.load()
    h = ctypes.c_void_p()
    rc = lib.gemm_plan_create(ctypes.byref(h), *args)
    if rc == 0:
        lib.gemm_plan_destroy(h)
    return rc


F16, BF16, E4M3, F32, E2M1, E2M3, E3M2, E2M1P = 1, 2, 3, 4, 5, 6, 7, 8
K_, MN = 0, 1


@pytest.mark.parametrize("args,expect", [
    ((256, 256, 64, F16, F16, F32, K_, K_, 0), 0),
    ((256, 256, 64, BF16, BF16, F32, MN, K_, 0), 0),
    ((256, 256, 128, E4M3, E4M3, F32, K_, K_, 32), 0),
    ((256, 256, 512, E2M1, E2M1, F32, K_, K_, 32), 0),       # MX-fp4
    ((300, 260, 256, E2M1, E2M1, F32, K_, K_, 32), 0),       # ragged MX-fp4
    ((256, 256, 384, E2M1, E2M1, F32, K_, K_, 32), 0),       # K tail (1.5 steps of 256)
    ((256, 256, 400, E2M1, E2M1, F32, K_, K_, 16), -2),      # rows of K/2 bytes not 16-byte aligned
    ((256, 256, 512, E2M1, E2M1, F32, K_, K_, 0), -2),       # fp4 needs scales
    ((256, 256, 512, E2M1, E2M1, F32, MN, K_, 32), -2),      # MN-major fp4 not built
    ((256, 256, 512, E2M1, E4M3, F32, K_, K_, 32), 0),       # dense fp4 x fp8
    ((256, 256, 1536, E4M3, E2M1, F32, K_, K_, 32), 0),      # fp8 x dense fp4
    ((256, 256, 256, E4M3, E2M1, F32, K_, K_, 32), 0),       # fp8 x dense fp4: one pair of steps
    ((256, 256, 384, E4M3, E2M1, F32, K_, K_, 32), -2),      # fp8 x dense fp4: K % 256
    ((256, 256, 512, E4M3, E2M1, F32, K_, K_, 16), -2),      # fp8 x dense fp4: 32-element blocks only
    ((256, 256, 512, E2M1, E2M3, F32, K_, K_, 32), -2),      # dense fp4 pairs with fp8 only
    ((256, 256, 128, E2M3, E2M3, F32, K_, K_, 32), 0),       # MX-fp6 (padded, sixteen per 16 bytes)
    ((300, 260, 384, E3M2, E3M2, BF16, K_, K_, 32), 0),      # ragged, bf16 output
    ((256, 256, 64, E2M3, E2M3, F32, K_, K_, 32), 0),        # K tail (half a 128-element step)
    ((256, 256, 40, E2M3, E2M3, F32, K_, K_, 32), -2),       # K not a multiple of the scale block
    ((256, 256, 128, E3M2, E3M2, F32, K_, K_, 0), -2),       # fp6 needs scales
    ((256, 256, 128, E2M3, E2M3, F32, K_, MN, 32), -2),      # MN-major fp6 not built
    ((256, 256, 128, E2M3, E3M2, F32, K_, K_, 32), 0),       # mixed 8- and 6-bit kinds
    ((256, 256, 128, E2M3, E4M3, F32, K_, K_, 32), 0),
    ((300, 260, 256, E4M3, E3M2, F16, K_, K_, 32), 0),
    ((256, 256, 256, E2M1, E2M3, F32, K_, K_, 32), -2),      # dense FP4 mixes with E4M3 only
    ((256, 256, 256, E2M3, E2M1, F32, K_, K_, 32), -2),
    ((256, 256, 128, E4M3, BF16, F32, K_, K_, 32), -2),      # dense with block-scaled
    ((256, 256, 128, 9, 9, F32, K_, K_, 32), -1),            # unknown dtype
    ((256, 256, 128, E2M1P, E2M1P, F32, K_, K_, 32), 0),     # padded FP4 (sixteen per 16 bytes)
    ((256, 256, 128, E4M3, E2M1P, F32, K_, K_, 32), 0),      # mixed fp8 x padded fp4
    ((256, 256, 128, E2M1P, E2M1, F32, K_, K_, 32), -2),     # the dense FP4 form does not mix
    ((256, 256, 64, E2M1P, E2M1P, F32, K_, K_, 32), 0),      # K tail: half a 128-element step
    ((256, 256, 48, E2M1P, E2M1P, F32, K_, K_, 32), -2),     # K not a multiple of the scale block
    ((256, 256, 48, E2M1P, E2M1P, F32, K_, K_, 16), 0),      # ... of 16-element blocks it is
    ((256, 256, 48, E2M1, E2M1, F32, K_, K_, 16), -2),       # E2M1 rows of K/2 bytes need K % 32
    ((256, 256, 96, E2M1, E2M1, F32, K_, K_, 16), 0),
    ((256, 256, 160, E4M3, E2M3, F32, K_, K_, 32), 0),       # mixed kinds, K tail
    ((0, 256, 64, F16, F16, F32, K_, K_, 0), -1),            # empty M
    ((256, -1, 64, F16, F16, F32, K_, K_, 0), -1),
    ((256, 256, 0, F16, F16, F32, K_, K_, 0), -1),           # empty K
    ((256, 256, 64, 9, F16, F32, K_, K_, 0), -1),            # unknown dtype
    ((256, 256, 64, F16, F16, F32, 2, K_, 0), -1),           # unknown major
    ((256, 256, 64, F16, F16, F32, K_, K_, -32), -1),
    ((256, 256, 64, F16, BF16, F32, K_, K_, 0), -2),         # mixed 16-bit kinds
    ((256, 256, 64, F16, F16, F16, K_, K_, 0), 0),           # fp16 output (rounded)
    ((256, 256, 64, BF16, BF16, BF16, K_, K_, 0), 0),        # bf16 output
    ((256, 256, 128, E4M3, E4M3, BF16, K_, K_, 32), 0),      # MX with bf16 output
    ((256, 256, 64, F16, F16, E4M3, K_, K_, 0), -2),         # e4m3 output
    ((256, 256, 64, F32, F32, F32, K_, K_, 0), -2),
    ((256, 256, 128, E4M3, E4M3, F32, K_, K_, 0), -2),       # e4m3 needs scales
    ((256, 256, 128, E4M3, E4M3, F32, K_, K_, 16), -2),      # E4M3: only 32-element blocks
    ((256, 256, 256, E2M1, E2M1, F32, K_, K_, 16), 0),       # 16-element blocks (scale_vec::4X)
    ((256, 256, 128, E2M1P, E2M1P, F32, K_, K_, 16), 0),
    ((256, 256, 128, E3M2, E3M2, BF16, K_, K_, 16), 0),
    ((256, 256, 128, E4M3, E2M3, F32, K_, K_, 16), -2),      # not for mixed kinds
    ((256, 256, 256, E2M1, E2M1, F32, K_, K_, 8), -2),
    ((256, 256, 64, F16, F16, F32, K_, K_, 32), -2),         # 16-bit is dense only
    ((256, 256, 64, F16, F16, F32, K_, MN, 0), 0),           # B MN-major (16-bit)
    ((256, 256, 64, BF16, BF16, F32, MN, MN, 0), 0),         # both MN-major
    ((256, 256, 128, E4M3, E4M3, F32, K_, MN, 32), -2),      # MN-major fp8 not built
    ((256, 256, 128, E4M3, E4M3, F32, MN, K_, 32), -2),      # MN-major fp8 not built
    ((256, 256, 96, F16, F16, F32, K_, K_, 0), 0),           # 16-bit K tail: 256 tile, zero-padded step
    ((256, 256, 8, BF16, BF16, F32, K_, MN, 0), 0),          # K below one step
    ((256, 256, 100, F16, F16, F32, K_, K_, 0), -2),         # K-major rows not 16-byte aligned
    ((256, 256, 100, F16, F16, F32, MN, K_, 0), -2),         # (B is K-major)
    ((256, 256, 100, F16, F16, F32, MN, MN, 0), 0),          # both MN-major: any K
    ((256, 256, 1, BF16, BF16, F32, MN, MN, 0), 0),
    ((256, 256, 64, E4M3, E4M3, F32, K_, K_, 32), 0),        # K below one 128-element step
    ((256, 256, 80, E4M3, E4M3, F32, K_, K_, 32), -2),       # K not a multiple of 32
    ((100, 256, 64, F16, F16, F32, K_, K_, 0), 0),           # ragged M: 256 tile, masked stores
    ((256, 96, 64, F16, F16, F32, K_, K_, 0), 0),            # ragged N
    ((100, 260, 128, E4M3, E4M3, F32, K_, K_, 32), 0),       # ragged MX
    ((256, 90, 64, F16, F16, F32, K_, K_, 0), -2),           # N % 4: D rows not 16-byte aligned
    ((100, 256, 64, BF16, BF16, F32, MN, K_, 0), -2),        # MN-major A needs M % 8
    ((104, 256, 64, BF16, BF16, F32, MN, K_, 0), 0),
    ((256, 100, 64, F16, F16, F32, K_, MN, 0), -2),          # MN-major B needs N % 8
    ((1 << 21, 64, 64, F16, F16, F32, K_, K_, 0), -1),       # beyond the size limit
    # MN-major operands must span less than 4 GiB (32-bit offsets)
    ((32768, 256, 65536, F16, F16, F32, MN, K_, 0), -2),     # A [K][M] is exactly 4 GiB
    ((32512, 256, 65536, F16, F16, F32, MN, K_, 0), 0),      # just below
    ((256, 65536, 65536, BF16, BF16, F32, K_, MN, 0), -2),   # B [K][N] is 8 GiB
    ((65536, 65536, 65536, BF16, BF16, F32, K_, K_, 0), 0),  # K-major: no such limit
])
def test_plan_create_rejections(args, expect):
    assert _create(*args) == expect


def test_plan_create_null_out():
    lib = mswz.load()
    assert lib.gemm_plan_create(None, 64, 64, 64, F16, F16, F32, K_, K_, 0) == -1


def test_tail_plans_use_the_256_tile():
    d = mswz.gemm_plan_create(1000, 520, 128, "bf16", "bf16").describe()
    assert (d["tile_m"], d["tile_n"], d["blocks"]) == (256, 256, 4 * 3)
    for K in (72, 4104):   # K tails, including shapes that would otherwise pick a smaller tile or streaming
        for M, N in ((128, 128), (64, 16384), (4096, 4096)):
            d = mswz.gemm_plan_create(M, N, K, "f16", "f16").describe()
            assert (d["tile_m"], d["tile_n"]) == (256, 256), (M, N, K)


@pytest.mark.parametrize("group_m", [-4, -1, 1, 4, 16])
def test_tile_raster_is_a_bijection(group_m):
    """Every workgroup maps to one tile and every tile to one workgroup, for
    grids that are and are not multiples of the XCD region grid."""
    lib = mswz.load()
    tm, tn = ctypes.c_int(), ctypes.c_int()
    for tiles_m, tiles_n in [(1, 1), (2, 4), (3, 5), (4, 4), (16, 16), (32, 32), (7, 12), (13, 1), (1, 9)]:
        seen = set()
        for b in range(tiles_m * tiles_n):
            assert lib.mswz_tile_of_block(b, tiles_m, tiles_n, group_m, ctypes.byref(tm), ctypes.byref(tn)) == 0
            assert 0 <= tm.value < tiles_m and 0 <= tn.value < tiles_n
            seen.add((tm.value, tn.value))
        assert len(seen) == tiles_m * tiles_n
    assert lib.mswz_tile_of_block(4, 2, 2, group_m, ctypes.byref(tm), ctypes.byref(tn)) == -1


def test_tile_choice():
    assert mswz.gemm_plan_create(4096, 4096, 4096, "bf16", "bf16").describe()["tile_m"] == 256
    d = mswz.gemm_plan_create(8192, 8192, 8192, "e4m3", "e4m3", scale_vec_len=32).describe()
    assert (d["tile_m"], d["tile_k"], d["blocks"]) == (256, 128, 1024)
    d = mswz.gemm_plan_create(128, 256, 64, "f16", "f16").describe()
    assert d["tile_m"] * d["tile_n"] * d["blocks"] == 128 * 256
    # weight streaming for any M up to 64 (padded to 32 or 64 rows)
    for M, pad in ((1, 32), (17, 32), (32, 32), (33, 64), (64, 64)):
        d = mswz.gemm_plan_create(M, 2048, 1024, "bf16", "bf16").describe()
        assert (d["variant"], d["tile_m"], d["blocks"]) == (21, pad, 2048 // 64), (M, d)
    assert mswz.gemm_plan_create(65, 2048, 1024, "bf16", "bf16").describe()["variant"] != 21
    assert mswz.gemm_plan_create(16, 2048, 1024, "bf16", "bf16", "bf16").describe()["variant"] != 21


def test_scale_major_switches_plans_of_the_wide_stage_kernels():
    """MN-major scales ([K/V][M], [K/V][N]): the 256x256 tile with the 32-byte
    scale stages (LDS 2 x 64 + 2 x 16 KiB); back to row-major restores the
    variant chosen at creation."""
    wide_lds = 2 * 512 * 128 + 2 * 512 * 32
    for a, b, d, K in (("e4m3", "e4m3", "f32", 8192), ("e4m3", "e2m3", "f32", 2048), ("e4m3", "e2m1p", "f32", 4096),
                       ("e2m3", "e2m3", "bf16", 2048), ("e3m2", "e3m2", "f16", 6144), ("e2m1p", "e2m1p", "f32", 2048),
                       ("e2m1", "e2m1", "f32", 8192), ("e2m1", "e2m1", "bf16", 2048), ("e4m3", "e4m3", "f32", 3072),
                       ("e4m3", "e3m2", "f32", 128), ("e2m3", "e2m3", "f32", 1152), ("e2m1", "e2m1", "f16", 768),
                       ("e4m3", "e4m3", "bf16", 2048), ("e4m3", "e4m3", "f16", 640), ("e4m3", "e2m3", "f16", 2048),
                       ("e4m3", "e2m1p", "bf16", 1024), ("e2m3", "e4m3", "f32", 2048), ("e2m3", "e3m2", "f32", 384),
                       ("e2m1p", "e3m2", "bf16", 4096), ("e4m3", "e2m1", "f32", 2048), ("e4m3", "e2m1", "bf16", 768)):
        p = mswz.gemm_plan_create(4096, 1040, K, a, b, d, scale_vec_len=32)
        before = p.describe()
        mswz.gemm_plan_set_scale_major(p, "mn")
        after = p.describe()
        assert p.sf_major == "mn"
        assert (after["tile_m"], after["tile_n"], after["lds_bytes"]) == (256, 256, wide_lds), (a, b, d, after)
        assert after["blocks"] == 16 * 5
        mswz.gemm_plan_set_scale_major(p, "k")
        assert p.describe() == before and p.sf_major == "k"
    # a grid the creation gives the 128 tile: MN-major scales take the 256 one
    p = mswz.gemm_plan_create(2048, 2048, 2048, "e4m3", "e4m3", scale_vec_len=32)
    assert p.describe()["tile_m"] == 128
    mswz.gemm_plan_set_scale_major(p, "mn")
    assert (p.describe()["tile_m"], p.describe()["blocks"], p.describe()["lds_bytes"]) == (256, 64, wide_lds)
    mswz.gemm_plan_set_scale_major(p, "k")
    assert p.describe()["tile_m"] == 128


@pytest.mark.parametrize("args, expect", [
    ((4096, 4096, 3104, "e4m3", "e4m3", "f32", 32), -2),      # K not a multiple of the K step
    ((4096, 4096, 2048 + 32, "e2m3", "e2m3", "f32", 32), -2),
    ((4096, 4096, 2048 + 128, "e2m1", "e2m1", "f32", 32), -2),
    ((4104, 4096, 2048, "e4m3", "e4m3", "f32", 32), -2),      # M not a multiple of 16
    ((4096, 4100, 2048, "e2m1", "e2m1", "f32", 32), -2),      # N not a multiple of 16
    ((4096, 4096, 2048, "e2m1", "e4m3", "f32", 32), -2),      # dense E2M1 A with E4M3 B
    ((4096, 4096, 2048, "e2m1", "e2m1", "f32", 16), -2),      # 16-element blocks
    ((4096, 4096, 2048, "e2m3", "e2m3", "f32", 16), -2),
    ((4096, 4096, 2048, "bf16", "bf16", "f32", 0), -5),       # dense plan
])
def test_scale_major_rejections_leave_the_plan_unchanged(args, expect):
    M, N, K, a, b, d, v = args
    p = mswz.gemm_plan_create(M, N, K, a, b, d, scale_vec_len=v)
    before = p.describe()
    lib = mswz.load()
    assert lib.gemm_plan_set_scale_major(p.handle, 1) == expect
    assert p.describe() == before
    if expect == -2:
        assert lib.gemm_plan_set_scale_major(p.handle, 0) == 0      # row-major stays available


def test_scale_major_argument_checks():
    lib = mswz.load()
    p = mswz.gemm_plan_create(4096, 4096, 2048, "e4m3", "e4m3", scale_vec_len=32)
    assert lib.gemm_plan_set_scale_major(None, 1) == -1
    assert lib.gemm_plan_set_scale_major(p.handle, 2) == -1
    assert lib.gemm_plan_set_scale_major(p.handle, -1) == -1
    # scale arrays of at most 2^31 bytes: K/V * M <= 2^31
    big = mswz.gemm_plan_create((1 << 19) + 16, 256, 1 << 17, "e2m1", "e2m1", scale_vec_len=32)
    assert lib.gemm_plan_set_scale_major(big.handle, 1) == -2
    ok = mswz.gemm_plan_create(1 << 19, 256, 1 << 17, "e2m1", "e2m1", scale_vec_len=32)
    assert lib.gemm_plan_set_scale_major(ok.handle, 1) == 0
    wide_n = mswz.gemm_plan_create(256, (1 << 19) + 16, 1 << 17, "e2m1", "e2m1", scale_vec_len=32)
    assert lib.gemm_plan_set_scale_major(wide_n.handle, 1) == -2


# ---- run-time rejections (fake pointers: never dereferenced) -------------------

def test_run_rejections_before_gpu_work():
    lib = mswz.load()
    dense = mswz.gemm_plan_create(256, 256, 64, "f16", "f16")
    mx = mswz.gemm_plan_create(256, 256, 128, "e4m3", "e4m3", scale_vec_len=32)
    P = 0x10000
    assert lib.gemm_run(None, P, P, P, 0, None) == -1
    assert lib.gemm_run(dense.handle, None, P, P, 0, None) == -1
    assert lib.gemm_run(dense.handle, P, P, None, 0, None) == -1
    assert lib.gemm_run(dense.handle, P, P, P, 2, None) == -1          # beta not 0/1
    assert lib.gemm_run(dense.handle, P + 8, P, P, 0, None) == -3      # misaligned A
    assert lib.gemm_run(dense.handle, P, P, P + 4, 0, None) == -3      # misaligned D
    assert lib.gemm_run(mx.handle, P, P, P, 0, None) == -5             # wrong kind
    assert lib.gemm_run_blockscaled(dense.handle, P, P, P, P, P, 0, None) == -5
    assert lib.gemm_run_blockscaled(mx.handle, P, P, None, P, P, 0, None) == -1
    assert lib.gemm_run_blockscaled(mx.handle, P, P, P + 1, P, P, 0, None) == -3
    assert lib.gemm_run_blockscaled(mx.handle, P, P, P, P, P, -1, None) == -1


def test_run_opts_rejections_before_gpu_work():
    lib = mswz.load()
    dense = mswz.gemm_plan_create(256, 256, 64, "f16", "f16")
    mx = mswz.gemm_plan_create(256, 256, 128, "e4m3", "e4m3", scale_vec_len=32)
    P = 0x10000
    run = lib.gemm_run_opts

    def opts(**kw):
        o = mswz.GemmOpts(0, 0, 0, None, None, 1)
        for k, v in kw.items():
            setattr(o, k, v)
        return ctypes.byref(o)

    assert run(None, P, P, None, None, P, 0, None, None) == -1
    assert run(dense.handle, P, P, P, P, P, 0, None, None) == -1            # scales on a dense plan
    assert run(mx.handle, P, P, None, P, P, 0, None, None) == -1            # missing SFA
    assert run(dense.handle, P, P, None, None, P, 2, opts(neg_a=1), None) == -1
    assert run(dense.handle, P + 8, P, None, None, P, 0, opts(neg_a=1), None) == -3
    assert run(mx.handle, P, P, P + 1, P, P, 0, opts(sat_d=1), None) == -3
    assert run(dense.handle, P, P, None, None, P, 0, opts(row_mask=P + 2), None) == -3
    assert run(dense.handle, P, P, None, None, P, 0, opts(col_zero=P + 1), None) == -3
    # the checks come before the predicate
    assert run(dense.handle, P + 8, P, None, None, P, 0, opts(pred=0), None) == -3
    assert run(dense.handle, P, P, None, None, P, 2, opts(pred=0), None) == -1
    # pred = 0 with valid arguments enqueues nothing (no GPU needed) and succeeds
    assert run(dense.handle, P, P, None, None, P, 0, opts(pred=0, neg_a=1, row_mask=P), None) == 0
    assert run(mx.handle, P, P, P, P, P, 1, opts(pred=0), None) == 0


def test_workspace_size_query():
    lib = mswz.load()
    assert lib.gemm_plan_workspace_size(None) == -1
    # weight streaming 64 x 16384 x 8192: 64 column blocks x 4 K parts, so 4
    # fp32 partials of 64 x 16384
    assert mswz.gemm_plan_create(64, 16384, 8192, "bf16", "bf16").workspace_bytes() == 4 * 64 * 16384 * 4
    assert mswz.gemm_plan_create(64, 2048, 4096, "f16", "f16").workspace_bytes() == 16 * 64 * 2048 * 4
    assert mswz.gemm_plan_create(32, 16384, 8192, "bf16", "bf16").workspace_bytes() == 4 * 32 * 16384 * 4
    assert mswz.gemm_plan_create(1, 4096, 4096, "bf16", "bf16").workspace_bytes() == 16 * 1 * 4096 * 4
    assert mswz.gemm_plan_create(17, 16384, 8192, "f16", "f16").workspace_bytes() == 4 * 17 * 16384 * 4
    assert mswz.gemm_plan_create(48, 1024 + 64, 8192, "bf16", "bf16").workspace_bytes() == 0   # N % 256
    assert mswz.gemm_plan_create(65, 16384, 8192, "bf16", "bf16").workspace_bytes() == 0       # M > 64
    assert mswz.gemm_plan_create(4096, 4096, 4096, "bf16", "bf16").workspace_bytes() == 0
    assert mswz.gemm_plan_create(256, 256, 128, "e4m3", "e4m3", scale_vec_len=32).workspace_bytes() == 0


def test_run_ws_rejections_before_gpu_work():
    lib = mswz.load()
    sk = mswz.gemm_plan_create(64, 16384, 8192, "bf16", "bf16")
    need = sk.workspace_bytes()
    P = 0x10000
    assert lib.gemm_run_ws(sk.handle, P, P, P, 0, None, need, None) == -1          # no workspace
    assert lib.gemm_run_ws(sk.handle, P, P, P, 0, P, need - 1, None) == -1         # too small
    assert lib.gemm_run_ws(sk.handle, P, P, P, 2, P, need, None) == -1             # beta
    assert lib.gemm_run_ws(sk.handle, P, P, P, 0, P + 8, need, None) == -3         # misaligned
    assert lib.gemm_run_ws(sk.handle, None, P, P, 0, P, need, None) == -1
    # a plan without a workspace path runs as gemm_run (same checks)
    dense = mswz.gemm_plan_create(256, 256, 64, "f16", "f16")
    assert lib.gemm_run_ws(dense.handle, P + 8, P, P, 0, None, 0, None) == -3
    assert lib.gemm_run_ws(None, P, P, P, 0, P, need, None) == -1


def test_binding_checks_buffer_sizes_before_the_library():
    import torch
    plan = mswz.gemm_plan_create(256, 256, 64, "f16", "f16")
    with pytest.raises((ValueError, TypeError)):
        mswz.gemm_run(plan, torch.zeros(10), torch.zeros(10), torch.zeros(10))


# ---- address functions vs brute force -----------------------------------------

@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("major", ["k", "mn"])
def test_desc_address_matches_bruteforce(mode, major):
    rows, words = (16, 64) if mode == 4 else (24, 4 * (1 << mode) * 2)
    for ldo, sdo, origin in [(16, 1024, 0), (256, 128, 0), (2048, 4096, 4096), (64, 512, 1024)]:
        if mode in (1, 2, 3, 4) and origin % walk.PERIOD[mode]:
            continue
        ref = walk.desc_walk_bruteforce(rows, words, ldo, sdo, mode, major, origin)
        got = np.array([[mswz.desc_address(r, w, ldo, sdo, mode, major, origin)
                         for w in range(words)] for r in range(rows)])
        assert np.array_equal(got, ref)


def test_desc_address_page_examples():
    # tcgen05.cp page: (128,4) b32 image, ldo=16, sdo=128, no swizzle -> 16r + 4w
    for r, w in itertools.product(range(128), range(4)):
        assert mswz.desc_address(r, w, 16, 128, 0) == 16 * r + 4 * w
    # tcgen05.mma page mode 4: offset ^ ((offset >> 2) & 96) on a 4-rows-per-SDO walk
    for r, w in itertools.product(range(8), range(32)):
        pre = (r // 4) * 512 + (r % 4) * 128 + 4 * w
        assert mswz.desc_address(r, w, 512, 512, 4, "mn") == pre ^ ((pre >> 2) & 96)


@pytest.mark.parametrize("ldo,sdo,mode,origin,expect_ok", [
    (16, 1024, 3, 0, True), (16, 128, 0, 16, True), (16, 1024, 3, 512, False),
    (8, 1024, 3, 0, False), (16, 1 << 18, 0, 0, False), (16, 256, 1, 256, True),
    (16, 256, 2, 256, False), (16, 512, 4, 512, True), (16, 512, 5, 0, False),
    (-16, 128, 0, 0, False), (16, 128, 0, 8, False),
])
def test_desc_check_rules(ldo, sdo, mode, origin, expect_ok):
    assert (mswz.desc_check(ldo, sdo, mode, origin) == 0) == expect_ok


def test_tile_offset_matches_bruteforce():
    ref = walk.lds_tile_bruteforce(256)
    got = np.array([[mswz.tile_offset(r, c) for c in range(8)] for r in range(256)])
    assert np.array_equal(got, ref)


# ---- row pitches (gemm_plan_create_ld) -----------------------------------------

def _create_ld(*args):
    lib = mswz.load()
    h = ctypes.c_void_p()
    rc = lib.gemm_plan_create_ld(ctypes.byref(h), *args)
    if rc == 0:
        lib.gemm_plan_destroy(h)
    return rc


@pytest.mark.parametrize("args,expect", [
    ((256, 256, 64, BF16, BF16, F32, K_, K_, 0, 0, 0, 0), 0),          # packed
    ((256, 256, 64, BF16, BF16, F32, K_, K_, 0, 64, 64, 256), 0),      # packed, spelled out
    ((256, 256, 64, BF16, BF16, F32, K_, K_, 0, 72, 128, 260), 0),     # views into wider rows
    ((256, 256, 64, BF16, BF16, F32, K_, K_, 0, 60, 0, 0), -1),        # lda < K
    ((256, 256, 64, BF16, BF16, F32, K_, K_, 0, 0, 0, 252), -1),       # ldd < N
    ((256, 256, 64, BF16, BF16, F32, K_, K_, 0, -8, 0, 0), -1),
    ((256, 256, 64, BF16, BF16, F32, K_, K_, 0, 68, 0, 0), -2),        # A rows not 16-byte aligned
    ((256, 256, 64, BF16, BF16, F32, K_, K_, 0, 0, 0, 258), -2),       # D rows: ldd % 4
    ((256, 256, 64, BF16, BF16, F32, K_, K_, 0, 1 << 23, 0, 0), -2),   # beyond the pitch limit
    ((256, 256, 64, BF16, BF16, F32, MN, K_, 0, 200, 0, 0), -1),       # MN-major A: lda >= M
    ((256, 256, 64, BF16, BF16, F32, MN, MN, 0, 264, 272, 0), 0),
    ((256, 256, 64, BF16, BF16, F32, MN, K_, 0, 260, 0, 0), -2),       # lda % 8
    ((256, 256, 128, E4M3, E4M3, F32, K_, K_, 32, 136, 0, 0), -2),     # E4M3 rows: lda % 16
    ((256, 256, 128, E4M3, E4M3, F32, K_, K_, 32, 144, 160, 0), 0),
    ((256, 256, 512, E2M1, E2M1, F32, K_, K_, 32, 528, 0, 0), -2),     # E2M1 rows: lda % 32
    ((256, 256, 512, E2M1, E2M1, F32, K_, K_, 32, 544, 0, 0), 0),
    ((100, 260, 64, F16, F16, BF16, K_, K_, 0, 128, 64, 264), 0),      # ragged, narrow D
    # MN-major spans below 4 GiB, counted with the pitch
    ((16384, 256, 65536, F16, F16, F32, MN, K_, 0, 0, 0, 0), 0),
    ((16384, 256, 65536, F16, F16, F32, MN, K_, 0, 32776, 0, 0), -2),
])
def test_plan_create_ld_rejections(args, expect):
    assert _create_ld(*args) == expect


def test_plan_create_ld_chooses_the_256_tile():
    # strided plans take the 256 tile, also where the packed shape would not
    assert mswz.gemm_plan_create(512, 512, 64, "bf16", "bf16").describe()["tile_m"] == 64
    d = mswz.gemm_plan_create_ld(512, 512, 64, "bf16", "bf16", ldd=520).describe()
    assert d["tile_m"] == 256 and d["blocks"] == 4
    # a weight-streaming shape with a pitch is not routed to the skinny kernels
    sk = mswz.gemm_plan_create(64, 16384, 8192, "bf16", "bf16")
    assert sk.describe()["tile_n"] == 64 and sk.workspace_bytes() > 0
    st = mswz.gemm_plan_create_ld(64, 16384, 8192, "bf16", "bf16", lda=8200)
    assert st.describe()["tile_n"] == 256 and st.workspace_bytes() == 0
    # the pitches the binding will check tensors against
    p = mswz.gemm_plan_create_ld(256, 512, 128, "f16", "f16", "f32", "mn", "k", 0, lda=264)
    assert (p.a_rows, p.a_cols, p.lda) == (128, 256, 264)
    assert (p.b_rows, p.b_cols, p.ldb) == (512, 128, 128)
    assert p.ldd == 512


def test_run_ws_noalloc_rejections_before_gpu_work():
    """Plans whose partials exceed the static scratch are refused with
    MSWZ_ERR_SCRATCH before any HIP call; a NULL plan is invalid."""
    lib = mswz.load()
    assert lib.gemm_noalloc_scratch_bytes() == 16 << 20
    assert mswz.STATUS["scratch"] == -6
    big = mswz.gemm_plan_create(64, 65536, 8192, "bf16", "bf16")      # 2 parts x 64 x 65536 fp32 = 32 MiB
    assert big.workspace_bytes() == 2 * 64 * 65536 * 4
    P = 0x10000
    assert lib.gemm_run_ws_noalloc(big.handle, P, P, P, 0, None) == -6
    assert lib.gemm_run_ws_noalloc(None, P, P, P, 0, None) == -1
    assert "scratch" in mswz.gemm_status_str(-6)
