"""Golden fixtures (tests/golden/), CPU only.

page_walks.json restates address values the pages print (each entry names its
page and section); tensor_mma_example.json holds the fp64 oracle's result on
the tcgen05.mma page's worked example inputs, written by
tests/golden/make_golden.py (which calls only oracle/).  The oracle, the
brute-force walk and the library's own address function are all checked
against them.
"""
import hashlib
import json
import os

import numpy as np

import mma_swizzled_operand_amd as mswz
import oracle
from oracle import walk

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)


def test_cp_example_walk():
    g = load("page_walks.json")["cp_example"]
    bf = walk.desc_walk_bruteforce(g["rows"], g["words"], g["ldo"], g["sdo"], g["mode"])
    for r in range(g["rows"]):
        for w in range(g["words"]):
            assert bf[r, w] == 16 * r + 4 * w
            assert mswz.desc_address(r, w, g["ldo"], g["sdo"], g["mode"]) == 16 * r + 4 * w


def test_mma_example_descriptor():
    g = load("page_walks.json")["mma_example"]
    assert mswz.desc_check(g["ldo"], g["sdo"], g["mode"], 0) == 0
    assert mswz.desc_check(g["ldo"], g["sdo"], g["mode"], g["align"] // 2) != 0   # misaligned origin
    for rows in (128, 64):
        phys = walk.desc_walk_bruteforce(rows, 32, g["ldo"], g["sdo"], g["mode"])
        lib = np.array([[mswz.desc_address(r, w, g["ldo"], g["sdo"], g["mode"]) for w in range(32)]
                        for r in range(rows)])
        assert np.array_equal(phys, lib)
        assert np.array_equal(phys // g["row_bytes"], np.arange(rows)[:, None].repeat(32, 1))


def test_mode4_pairs():
    g = load("page_walks.json")["mode4"]
    for off, expect in g["pairs"]:
        assert walk.swizzle_bruteforce(4, off) == expect


def test_periods():
    g = load("page_walks.json")["periods"]
    for mode in (1, 2, 3):
        assert walk.PERIOD[mode] == g[str(mode)]


def test_tensor_mma_example_oracle():
    g = load("tensor_mma_example.json")
    rng = np.random.default_rng(0)
    a = (rng.integers(-4, 5, (128, 64)) / 4).astype("float16")
    b = (rng.integers(-4, 5, (64, 64)) / 4).astype("float16")
    b2 = (rng.integers(-4, 5, (256, 64)) / 4).astype("float16")
    for name, bb in (("128x64x64", b), ("128x256x64", b2)):
        c = g["cases"][name]
        d = oracle.gemm(128, bb.shape[0], 64, "f16", "k", a.view(np.uint16), "f16", "k", bb.view(np.uint16))
        d32 = d.astype(np.float32)
        assert hashlib.sha256(d32.astype("<f4").tobytes()).hexdigest() == c["sha256_f32_le"]
        assert [float(v) for v in d[0, :8]] == c["row0_first8"]
        assert float(d.sum()) == c["sum"]
        # and the page's own comparison target, fp32 a @ b.T, agrees exactly
        assert np.array_equal(d32, a.astype("float32") @ bb.astype("float32").T)
