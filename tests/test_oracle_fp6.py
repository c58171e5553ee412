"""Pins for the oracle's 6-bit element kinds and the padded 4-bit form (CPU only).

The pages name FP6 ("six-bit values") only in the tcgen05.cp page's "Native
FP4/FP6 decompression" section, which fixes the storage: each 16-byte block
holds sixteen packed values followed by four bytes of padding, and the
padding is not part of the data.  The element formats are read as OCP E2M3
and E3M2 (no infinities or NaN) and value j of a block as bits 6j .. 6j+5 of
the block's first twelve bytes taken little-endian.

Pins: every code against the formats' definitions written with exact
rationals, the largest and smallest values, the packing against a bit-by-bit
writer with random padding bytes, the input generator's rounding, and the
GEMM on 6-bit operands against the torch-pinned E4M3 path on the same values
(every E2M3 and E3M2 value is an E4M3 value).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

# (exponent bits, fraction bits, bias)
FORMATS = {"e2m3": (2, 3, 1), "e3m2": (3, 2, 3)}


def exact_value(kind, code):
    """The format definition, in exact rationals: sign, then subnormal
    f / 2^F * 2^(1-bias) for exponent 0, else (1 + f / 2^F) * 2^(e-bias)."""
    E, F, bias = FORMATS[kind]
    s = (code >> (E + F)) & 1
    e = (code >> F) & ((1 << E) - 1)
    f = code & ((1 << F) - 1)
    if e == 0:
        v = Fraction(f, 1 << F) * Fraction(2) ** (1 - bias)
    else:
        v = (1 + Fraction(f, 1 << F)) * Fraction(2) ** (e - bias)
    return -v if s else v


def pack_bitwise(codes: np.ndarray, pad: np.ndarray) -> np.ndarray:
    """Bit-by-bit writer: value j of each 16-value block into bits 6j..6j+5 of
    the block's first twelve bytes (bit b of the payload is bit b % 8 of byte
    b // 8); bytes 12..15 take `pad`."""
    rows, n = codes.shape
    out = np.zeros((rows, n), dtype=np.uint8)
    for r in range(rows):
        for blk in range(n // 16):
            base = 16 * blk
            for j in range(16):
                c = int(codes[r, base + j])
                for t in range(6):
                    if (c >> t) & 1:
                        bit = 6 * j + t
                        out[r, base + bit // 8] |= 1 << (bit % 8)
            out[r, base + 12:base + 16] = pad[r, 4 * blk:4 * blk + 4]
    return out


@pytest.mark.parametrize("kind", list(FORMATS))
def test_every_code_matches_the_definition(kind):
    rng = np.random.default_rng(7)
    codes = np.arange(64, dtype=np.uint8).reshape(4, 16)
    stored = pack_bitwise(codes, rng.integers(0, 256, (4, 4), dtype=np.uint8))
    got = oracle.decode(kind, stored).reshape(-1)
    want = [float(exact_value(kind, c)) for c in range(64)]
    assert list(got) == want
    assert np.signbit(got[32]) and not np.signbit(got[0])   # code 32 is -0


def test_extreme_values():
    e2m3 = oracle.decode("e2m3", pack_bitwise(np.array([[31, 1, 63, 8] + [0] * 12]), np.zeros((1, 4), np.uint8)))
    assert list(e2m3[0, :4]) == [7.5, 0.125, -7.5, 1.0]
    e3m2 = oracle.decode("e3m2", pack_bitwise(np.array([[31, 1, 63, 12] + [0] * 12]), np.zeros((1, 4), np.uint8)))
    assert list(e3m2[0, :4]) == [28.0, 0.0625, -28.0, 1.0]


@pytest.mark.parametrize("kind", list(FORMATS))
def test_packing_and_padding(kind):
    """Random codes packed bit by bit with random padding decode to the codes'
    values in order; changing only the padding changes nothing."""
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 64, (5, 64), dtype=np.uint8)
    stored = pack_bitwise(codes, rng.integers(0, 256, (5, 16), dtype=np.uint8))
    stored2 = pack_bitwise(codes, rng.integers(0, 256, (5, 16), dtype=np.uint8))
    want = np.vectorize(lambda c: float(exact_value(kind, int(c))))(codes)
    assert np.array_equal(oracle.decode(kind, stored), want)
    assert np.array_equal(oracle.decode(kind, stored2), want)


@pytest.mark.parametrize("kind", list(FORMATS))
def test_generator_rounding_and_packing(kind):
    """The input generator: every value round-trips (zero padding), exact
    midpoints go to the even code, magnitudes beyond the largest saturate."""
    # (code 32 is -0: its float keeps the sign)
    vals = np.array([np.copysign(float(exact_value(kind, c)), -1.0 if c >= 32 else 1.0)
                     for c in range(64)]).reshape(4, 16)
    stored = wl.to_stored(vals, kind)
    assert np.array_equal(oracle.decode(kind, stored), vals)
    assert not stored.reshape(-1, 16)[:, 12:].any()
    codes = np.arange(64, dtype=np.uint8).reshape(4, 16)
    assert np.array_equal(stored, pack_bitwise(codes, np.zeros((4, 4), np.uint8)))
    mags = np.array([float(exact_value(kind, c)) for c in range(32)])
    mids = (mags[1:] + mags[:-1]) / 2
    got = oracle.decode(kind, wl.to_stored(np.concatenate([mids, [1e3]])[None, :], kind))[0]
    for i, m in enumerate(mids):          # tie between codes i and i+1: the even one
        assert got[i] == mags[i if i % 2 == 0 else i + 1]
    assert got[31] == mags[31]


def _as_e4m3(kind, stored):
    vals = oracle.decode(kind, stored)
    return torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("kind", list(FORMATS))
@pytest.mark.parametrize("M,N,K", [(3, 5, 64), (16, 9, 256)])
def test_fp6_gemm_equals_e4m3_gemm_of_the_same_values(kind, M, N, K):
    """Packed access and the decoder against the torch-pinned E4M3 path:
    random codes and padding, random block scales, beta = 1."""
    rng = np.random.default_rng(42)
    A = pack_bitwise(rng.integers(0, 64, (M, K), dtype=np.uint8), rng.integers(0, 256, (M, K // 4), dtype=np.uint8))
    B = pack_bitwise(rng.integers(0, 64, (N, K), dtype=np.uint8), rng.integers(0, 256, (N, K // 4), dtype=np.uint8))
    SFA = (127 + rng.integers(-3, 4, (M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(-3, 4, (N, K // 32))).astype(np.uint8)
    D0 = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    got = oracle.gemm(M, N, K, kind, "k", A, kind, "k", B, V=32, SFA=SFA, SFB=SFB, beta=1, D0=D0)
    ref = oracle.gemm(M, N, K, "e4m3", "k", _as_e4m3(kind, A), "e4m3", "k", _as_e4m3(kind, B),
                      V=32, SFA=SFA, SFB=SFB, beta=1, D0=D0)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("kind,one", [("e2m3", 8), ("e3m2", 12)])
def test_fp6_all_ones_closed_form(kind, one):
    """Every element 1.0 with unit scales: every entry is K."""
    M, N, K = 4, 6, 128
    A = pack_bitwise(np.full((M, K), one, np.uint8), np.full((M, K // 4), 0xFF, np.uint8))
    B = pack_bitwise(np.full((N, K), one, np.uint8), np.full((N, K // 4), 0xFF, np.uint8))
    got = oracle.gemm(M, N, K, kind, "k", A, kind, "k", B, V=32, SFA=np.full((M, K // 32), 127, np.uint8),
                      SFB=np.full((N, K // 32), 127, np.uint8))
    assert np.array_equal(got, np.full((M, N), float(K)))


def test_fp6_rows_must_be_whole_blocks():
    with pytest.raises(ValueError):
        oracle.decode("e2m3", np.zeros((2, 24), np.uint8))
    with pytest.raises(ValueError):
        oracle.gemm(2, 2, 24, "e3m2", "k", np.zeros((2, 24), np.uint8), "e3m2", "k",
                    np.zeros((2, 24), np.uint8))


# ---- the padded 4-bit form ("e2m1p": sixteen E2M1 values, then eight bytes
# of padding, per 16-byte block; same section of the tcgen05.cp page) ----------

def pack_e2m1_padded(codes: np.ndarray, pad: np.ndarray) -> np.ndarray:
    """Nibble writer: value j of a block in the low (even j) or high (odd j)
    nibble of byte j // 2; bytes 8..15 take `pad`."""
    rows, n = codes.shape
    out = np.zeros((rows, n), dtype=np.uint8)
    for r in range(rows):
        for blk in range(n // 16):
            for j in range(16):
                out[r, 16 * blk + j // 2] |= int(codes[r, 16 * blk + j]) << (4 * (j % 2))
            out[r, 16 * blk + 8:16 * blk + 16] = pad[r, 8 * blk:8 * blk + 8]
    return out


def test_e2m1_padded_codes_and_padding():
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 16, (4, 64), dtype=np.uint8)
    a = pack_e2m1_padded(codes, rng.integers(0, 256, (4, 32), dtype=np.uint8))
    b = pack_e2m1_padded(codes, rng.integers(0, 256, (4, 32), dtype=np.uint8))
    # the same codes in the dense two-per-byte form (pinned against the format table)
    dense = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    want = oracle.decode("e2m1", dense)
    assert np.array_equal(oracle.decode("e2m1p", a), want)
    assert np.array_equal(oracle.decode("e2m1p", b), want)


def test_e2m1_padded_generator_matches_dense_form():
    rng = np.random.default_rng(13)
    x = rng.normal(0, 2, (3, 64))
    padded = wl.to_stored(x, "e2m1p").reshape(3, 4, 16)
    dense = wl.to_stored(x, "e2m1").reshape(3, 4, 8)
    assert np.array_equal(padded[..., :8], dense) and not padded[..., 8:].any()


@pytest.mark.parametrize("M,N,K", [(3, 5, 64), (16, 9, 256)])
def test_e2m1_padded_gemm_equals_dense_e2m1_gemm(M, N, K):
    rng = np.random.default_rng(14)
    ca = rng.integers(0, 16, (M, K), dtype=np.uint8)
    cb = rng.integers(0, 16, (N, K), dtype=np.uint8)
    A = pack_e2m1_padded(ca, rng.integers(0, 256, (M, K // 2), dtype=np.uint8))
    B = pack_e2m1_padded(cb, rng.integers(0, 256, (N, K // 2), dtype=np.uint8))
    Ad = (ca[:, 0::2] | (ca[:, 1::2] << 4)).astype(np.uint8)
    Bd = (cb[:, 0::2] | (cb[:, 1::2] << 4)).astype(np.uint8)
    SFA = (127 + rng.integers(-3, 4, (M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(-3, 4, (N, K // 32))).astype(np.uint8)
    got = oracle.gemm(M, N, K, "e2m1p", "k", A, "e2m1p", "k", B, V=32, SFA=SFA, SFB=SFB)
    ref = oracle.gemm(M, N, K, "e2m1", "k", Ad, "e2m1", "k", Bd, V=32, SFA=SFA, SFB=SFB)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("ka,kb", [("e4m3", "e2m1p"), ("e2m3", "e3m2"), ("e2m1p", "e2m3")])
def test_mixed_kinds_equal_e4m3_of_the_same_values(ka, kb):
    """Operands of two kinds: the same as both re-encoded as E4M3."""
    M, N, K = 7, 5, 128
    rng = np.random.default_rng(15)
    x = {"A": wl.to_stored(rng.normal(0, 2, (M, K)), ka), "B": wl.to_stored(rng.normal(0, 2, (N, K)), kb)}
    SFA = (127 + rng.integers(-3, 4, (M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(-3, 4, (N, K // 32))).astype(np.uint8)
    got = oracle.gemm(M, N, K, ka, "k", x["A"], kb, "k", x["B"], V=32, SFA=SFA, SFB=SFB)
    ref = oracle.gemm(M, N, K, "e4m3", "k", _as_e4m3(ka, x["A"]), "e4m3", "k", _as_e4m3(kb, x["B"]),
                      V=32, SFA=SFA, SFB=SFB)
    assert np.array_equal(got, ref)
