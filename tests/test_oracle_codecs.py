"""Pins for the oracle's element decoders (CPU only).

Each decoder is checked exhaustively against an independent library routine
(numpy float16, torch bfloat16 / float8_e4m3fn) and against values fixed by
the format definitions.  The 8-bit element format is read as OCP E4M3 and the
scale byte as OCP E8M0 (the tcgen05.mma page's "Weight-stationary and block
scaling" section names block-scaled kinds but no element format).
"""
import numpy as np
import torch

import oracle


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nan = np.isnan(a)
    assert np.array_equal(nan, np.isnan(b))
    assert np.array_equal(a[~nan], b[~nan])
    # signed zeros agree too
    assert np.array_equal(np.signbit(a[~nan]), np.signbit(b[~nan]))


def test_f16_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    _same(oracle.decode("f16", bits), bits.view(np.float16).astype(np.float64))


def test_bf16_all_patterns_match_torch_and_shift():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode("bf16", bits)
    via_torch = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    _same(got, via_torch)
    with np.errstate(invalid="ignore"):
        via_shift = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    _same(got, via_shift)


def test_e4m3_all_patterns_match_torch():
    bits = np.arange(256, dtype=np.uint16).astype(np.uint8)
    got = oracle.decode("e4m3", bits)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    _same(got, ref)


def test_e4m3_definition_spot_values():
    spots = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x00: 0.0,
             0xB8: -1.0, 0x3C: 1.5, 0x07: 7 * 2.0 ** -9}
    bits = np.array(list(spots), dtype=np.uint8)
    got = oracle.decode("e4m3", bits)
    assert list(got) == list(spots.values())
    nan = oracle.decode("e4m3", np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.isnan(nan).all()
    # no infinities in this format
    assert np.isfinite(oracle.decode("e4m3", np.arange(256, dtype=np.uint16).astype(np.uint8))[
        [i for i in range(256) if i & 0x7F != 0x7F]]).all()


def test_f16_bf16_special_values():
    f16 = oracle.decode("f16", np.array([0x3C00, 0x7BFF, 0x0001, 0x0400, 0x7C00, 0xFC00], dtype=np.uint16))
    assert list(f16) == [1.0, 65504.0, 2.0 ** -24, 2.0 ** -14, np.inf, -np.inf]
    bf = oracle.decode("bf16", np.array([0x3F80, 0x0001, 0x0080, 0x7F80, 0xC000], dtype=np.uint16))
    assert list(bf) == [1.0, 2.0 ** -133, 2.0 ** -126, np.inf, -2.0]


def test_e8m0_definition():
    e = np.arange(256, dtype=np.uint16).astype(np.uint8)
    got = oracle.decode_e8m0(e)
    for E in range(255):
        assert got[E] == 2.0 ** (E - 127)
    assert np.isnan(got[255])
    assert got[127] == 1.0


def test_decode_rejects_bad_kind():
    import pytest
    with pytest.raises(ValueError):
        oracle.decode("e4m3", np.zeros(4, dtype=np.uint16))


def test_e2m1_all_patterns_match_the_format_table():
    """OCP E2M1 (FP4): sign, 2 exponent bits (bias 1), 1 fraction bit, no
    infinities or NaN; the format's eight magnitudes, in code order."""
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    codes = np.arange(16, dtype=np.uint8)
    got = oracle.decode("e2m1", codes)[0::2]          # low nibbles carry the codes
    want = np.array(table + [-v for v in table])
    assert np.array_equal(got, want)
    assert np.signbit(got[8]) and not np.signbit(got[0])   # 0x8 is -0


def test_e2m1_nibble_order():
    """Two elements per byte: element 2j in bits 0..3, element 2j+1 in bits 4..7."""
    got = oracle.decode("e2m1", np.array([[0x21, 0xE7]], dtype=np.uint8))
    assert got.shape == (1, 4)
    assert list(got[0]) == [0.5, 1.0, 6.0, -4.0]


def test_generator_e2m1_rounding():
    """Input generation: every E2M1 value round-trips; exact midpoints go to the
    even code; magnitudes beyond 6 saturate (the workload recipe)."""
    import workloads as wl
    vals = oracle.decode("e2m1", np.arange(256, dtype=np.uint8))
    assert np.array_equal(oracle.decode("e2m1", wl.to_stored(vals[None, :], "e2m1"))[0], vals)
    mids = np.array([[0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 9.0]])
    got = oracle.decode("e2m1", wl.to_stored(mids, "e2m1"))[0]
    assert list(got) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0]
