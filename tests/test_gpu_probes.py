"""One-wave GPU probes of the instruction lane images the kernels are built
on, checked against the images stated in device_common.hpp and used by
tests/test_lds_maps.py (which moves data through the kernels' LDS maps on
the CPU under exactly these images).  Each probe runs one instruction on
per-lane operands chosen here and compares every lane's result with the
image's prediction; values are small enough that every result is exact.

The probes are tests/probes/probes.hip (built into tests/probes/libprobes.so
by __graft_entry__.build()), which call the library's own instruction
wrappers."""
import ctypes
import os

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "probes", "libprobes.so")


@pytest.fixture(scope="module")
def probes():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: run __graft_entry__.build()")
    h = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    h.probe_mfma16.argtypes = [ctypes.c_int, P, P, P]
    h.probe_mfma_scale16.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, P]
    h.probe_read_tr16.argtypes = [P, ctypes.c_int, P, P]
    return h


def _p(a):
    return ctypes.c_void_p(a.ctypes.data)


# ---- 16x16x32, 16-bit -------------------------------------------------------------

@pytest.mark.parametrize("kind", ["bf16", "f16"])
def test_mfma16_operand_and_output_images(probes, kind):
    """Operand lane l holds 8 K values of row l % 16, K group l / 16 (the same
    K positions in both operands); register r of lane l is D[4 (l/16) + r][l % 16],
    rows from the first operand, columns from the second."""
    rng = np.random.default_rng(11)
    X = rng.integers(-8, 9, (16, 32)).astype(np.float64)   # first operand rows x K
    Y = rng.integers(-8, 9, (16, 32)).astype(np.float64)

    def regs(M):
        bits = np.empty((64, 8), np.uint16)
        for l in range(64):
            vals = M[l % 16, 8 * (l // 16): 8 * (l // 16) + 8]
            if kind == "f16":
                bits[l] = vals.astype(np.float16).view(np.uint16)
            else:
                bits[l] = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        return np.ascontiguousarray(bits).view(np.uint32)

    out = np.zeros((64, 4), np.float32)
    assert probes.probe_mfma16(int(kind == "bf16"), _p(regs(X)), _p(regs(Y)), _p(out)) == 0
    D = X @ Y.T
    want = np.array([[D[4 * (l // 16) + r, l % 16] for r in range(4)] for l in range(64)])
    assert np.array_equal(out.astype(np.float64), want)


# ---- block-scaled 16x16x128 ---------------------------------------------------------

FMT = {"e4m3": 0, "e2m3": 2, "e3m2": 3, "e2m1": 4}


def _codes_by_value(kind):
    """{value: [codes]} for the codes of `kind` whose magnitude is 0, 1, 1.5,
    2 or 3, decoded by the oracle's codecs."""
    if kind == "e4m3":
        codes = np.arange(256)
        vals = oracle.decode("e4m3", codes.astype(np.uint8))
    elif kind == "e2m1":
        codes = np.arange(16)
        vals = oracle.decode("e2m1", (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8))
    else:   # sixteen 6-bit values per padded 16-byte block, value j in bits 6j..6j+5
        codes = np.arange(64)
        blocks = []
        for b in range(4):
            x = sum(int(c) << (6 * j) for j, c in enumerate(codes[16 * b:16 * b + 16]))
            blocks.append(list(x.to_bytes(12, "little")) + [0, 0, 0, 0])
        vals = oracle.decode(kind, np.array(blocks, np.uint8)).ravel()
    table = {}
    for c, v in zip(codes, vals):
        if abs(v) in (0.0, 1.0, 1.5, 2.0, 3.0):
            table.setdefault(float(v), []).append(int(c))
    assert len(table) == 9, (kind, sorted(table))
    return table


def _internal_k(kind, g, j):
    """Internal K index of value j (0..31) of a lane in group g."""
    if kind == "e4m3":
        return 32 * (g // 2) + 16 * (g % 2) + (j % 16) + 64 * (j // 16)
    return 32 * g + j


def _pack(kind, codes, rng):
    """One lane's eight registers from its 32 codes; bits the format does not
    read are random."""
    words = rng.integers(0, 2 ** 32, 8, dtype=np.uint64)
    if kind == "e4m3":
        return np.frombuffer(bytes(int(c) for c in codes), np.uint32).astype(np.uint64)
    width, nregs = (6, 6) if kind in ("e2m3", "e3m2") else (4, 4)
    x = sum(int(c) << (width * j) for j, c in enumerate(codes))
    low = np.frombuffer(x.to_bytes(4 * nregs, "little"), np.uint32).astype(np.uint64)
    words[:nregs] = low
    return words


def _operand(kind, rng):
    """Random operand: the 16 x 128 matrix of values it holds by internal K
    index, and its 64 x 8 registers."""
    table = _codes_by_value(kind)
    values = sorted(table)
    M = np.zeros((16, 128))
    regs = np.zeros((64, 8), np.uint64)
    for l in range(64):
        i, g = l % 16, l // 16
        vals = rng.choice(values, 32)
        codes = [rng.choice(table[v]) for v in vals]
        for j in range(32):
            M[i, _internal_k(kind, g, j)] = vals[j]
        regs[l] = _pack(kind, codes, rng)
    return M, np.ascontiguousarray(regs.astype(np.uint32))


PAIRS = [("e4m3", "e4m3"), ("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e2m1", "e2m1"),
         ("e4m3", "e2m3"), ("e2m3", "e4m3"), ("e4m3", "e3m2"), ("e4m3", "e2m1"),
         ("e2m1", "e4m3"), ("e2m3", "e3m2"), ("e3m2", "e2m1")]


@pytest.mark.parametrize("k1,k2", PAIRS)
def test_mfma_scale16_operand_scale_and_output_images(probes, k1, k2):
    """The images stated for the scaled 16x16x128 MFMA: which (row, internal
    K) every operand byte or value is, lane i + 16 b giving row i's scale for
    32-wide block b from byte 0 of its scale register (the other bytes
    ignored), and the 16x16x32 output image."""
    rng = np.random.default_rng(7 + 13 * FMT[k1] + FMT[k2])
    X, xa = _operand(k1, rng)
    Y, yb = _operand(k2, rng)
    ex = rng.integers(125, 130, 64)
    ey = rng.integers(125, 130, 64)
    sa = (ex | (rng.integers(0, 2 ** 24, 64) << 8)).astype(np.uint32).view(np.int32)
    sb = (ey | (rng.integers(0, 2 ** 24, 64) << 8)).astype(np.uint32).view(np.int32)
    out = np.zeros((64, 4), np.float32)
    assert probes.probe_mfma_scale16(FMT[k1], FMT[k2], _p(xa), _p(yb), _p(sa), _p(sb), _p(out)) == 0
    sX = np.array([[2.0 ** (ex[i + 16 * b] - 127) for b in range(4)] for i in range(16)])
    sY = np.array([[2.0 ** (ey[i + 16 * b] - 127) for b in range(4)] for i in range(16)])
    Xs = X * np.repeat(sX, 32, axis=1)
    Ys = Y * np.repeat(sY, 32, axis=1)
    D = Xs @ Ys.T
    want = np.array([[D[4 * (l // 16) + r, l % 16] for r in range(4)] for l in range(64)])
    assert np.array_equal(out.astype(np.float64), want)


# ---- ds_read_b64_tr_b16 ----------------------------------------------------------------

def _tr_expected(addrs):
    """The stated lane map: in each 16-lane group, lanes 4j .. 4j+3 name 16
    consecutive-by-lane values v_j; lane t of the group receives
    (v_0[t], v_1[t], v_2[t], v_3[t]).  LDS holds u16 value = its index."""
    out = np.zeros((64, 4), np.uint16)
    for l in range(64):
        grp, t = l & ~15, l & 15
        for j in range(4):
            a = addrs[grp + 4 * j + t // 4]
            out[l, j] = a // 2 + t % 4
    return out


def _run_tr(probes, addrs):
    init = np.arange(16384, dtype=np.uint16)
    a = np.ascontiguousarray(np.asarray(addrs, np.uint32))
    out = np.zeros((64, 2), np.uint32)
    assert probes.probe_read_tr16(_p(init), init.size, _p(a), _p(out)) == 0
    return out.view(np.uint16).reshape(64, 4)


def test_read_tr16_lane_map_on_random_addresses(probes):
    rng = np.random.default_rng(5)
    for _ in range(4):
        addrs = 8 * rng.integers(0, 32768 // 8, 64)
        assert np.array_equal(_run_tr(probes, addrs), _tr_expected(addrs))


@pytest.mark.parametrize("b", [0, 5, 15])
def test_read_tr16_on_the_kernels_mn_fragment_addresses(probes, b):
    """The MN-major 16x16x32 fragment reads of the 256x256 kernel, through
    the library's own lane map."""
    import mma_swizzled_operand_amd as mswz
    for ks in range(2):
        v = mswz.lds_lanes("frag_mn16", b, ks)
        for half in (v[0::2], v[1::2]):
            assert np.array_equal(_run_tr(probes, half), _tr_expected(half))
