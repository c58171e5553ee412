"""Pins of the oracle's per-call options (oracle.apply_opts) against
formulations that do not use it: the plain oracle GEMM on operands whose sign
bits were flipped or whose rows were zeroed, the format constants from their
bit-field definitions, and a brute-force bit decoder for the masks.

The pages name neg_a, neg_b, sat_d, the output-lane and zero-column masks
and pred (tcgen05.mma page, "Weight-stationary and block scaling") without
defining them; the readings pinned here are the ones oracle.apply_opts states.
"""
import numpy as np
import pytest

import oracle
import workloads as wl

SIGN_BITS = {"f16": 0x8000, "bf16": 0x8000, "e4m3": 0x80, "e2m1": 0x88}   # e2m1: both nibbles


def _gemm(w, x, A=None, B=None, beta=0, D0=None):
    return oracle.gemm(w.M, w.N, w.K, w.kind, w.a_major, x["A"] if A is None else A, w.kind, w.b_major,
                       x["B"] if B is None else B, V=w.V, SFA=x.get("SFA"), SFB=x.get("SFB"), beta=beta,
                       D0=D0)


CASES = [wl.custom(24, 40, 64, "bf16", name="o-bf16"),
         wl.custom(16, 32, 64, "f16", a_major="mn", name="o-f16-amn"),
         wl.custom(16, 24, 128, "e4m3", V=32, name="o-e4m3"),
         wl.custom(8, 16, 256, "e2m1", V=32, name="o-e2m1")]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_negation_equals_flipped_sign_bits(w):
    x = wl.generate(w, seed=3)
    P = _gemm(w, x)
    flipA = x["A"] ^ np.array(SIGN_BITS[w.kind], dtype=x["A"].dtype)
    flipB = x["B"] ^ np.array(SIGN_BITS[w.kind], dtype=x["B"].dtype)
    Db = np.zeros_like(P)
    assert np.array_equal(oracle.apply_opts(P, Db, neg_a=True), _gemm(w, x, A=flipA))
    assert np.array_equal(oracle.apply_opts(P, Db, neg_b=True), _gemm(w, x, B=flipB))
    assert np.array_equal(oracle.apply_opts(P, Db, neg_a=True, neg_b=True), _gemm(w, x, A=flipA, B=flipB))
    assert np.array_equal(oracle.apply_opts(P, Db, neg_a=True, neg_b=True), P)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_zero_columns_equal_zeroed_b_rows(w):
    x = wl.generate(w, seed=4)
    rng = np.random.default_rng(5)
    cols = rng.random(w.N) < 0.4
    words = np.zeros((w.N + 31) // 32, dtype=np.uint32)
    for n in np.flatnonzero(cols):
        words[n // 32] |= np.uint32(1 << (n % 32))
    B = x["B"].copy()
    if w.b_major == "k":
        per = 2 if w.kind == "e2m1" else 1
        B.reshape(w.N, -1)[cols, :] = 0   # stored zero patterns decode to +0 in every format
        assert per in (1, 2)
    else:
        B[:, cols] = 0
    P = _gemm(w, x)
    D0 = rng.standard_normal((w.M, w.N)).astype(np.float32)
    got = oracle.apply_opts(P, D0, beta=1, D0=D0, col_zero=words)
    assert np.array_equal(got, _gemm(w, x, B=B, beta=1, D0=D0))
    assert np.array_equal(got[:, cols], D0[:, cols].astype(np.float64))


def test_row_mask_keeps_rows_and_pred_keeps_everything():
    w = CASES[0]
    x = wl.generate(w, seed=6)
    P = _gemm(w, x)
    Db = np.full(P.shape, np.nan)
    Db[::3] = 7.25
    rows = np.zeros(w.M, dtype=bool)
    rows[[0, 5, 23]] = True
    words = np.zeros(1, dtype=np.uint32)
    for m in np.flatnonzero(rows):
        words[0] |= np.uint32(1 << m)
    got = oracle.apply_opts(P, Db, row_mask=words, neg_a=True)
    assert np.array_equal(got[rows], Db[rows], equal_nan=True)
    assert np.array_equal(got[~rows], -P[~rows])
    assert np.array_equal(oracle.apply_opts(P, Db, pred=False, neg_a=True), Db, equal_nan=True)


def test_saturation_limits_are_the_formats_largest_finite_values():
    # (2 - 2^-mantissa_bits) * 2^max_exponent from each format's bit layout
    assert oracle.D_MAX["f32"] == (2 - 2.0 ** -23) * 2.0 ** 127
    assert oracle.D_MAX["bf16"] == (2 - 2.0 ** -7) * 2.0 ** 127
    assert oracle.D_MAX["f16"] == (2 - 2.0 ** -10) * 2.0 ** 15
    P = np.array([[1e39, -1e39, np.inf, -np.inf], [np.nan, 3.0, -65504.0, 70000.0]])
    Db = np.zeros_like(P)
    got = oracle.apply_opts(P, Db, sat_d=True)
    mx = oracle.D_MAX["f32"]
    assert np.array_equal(got[0], [mx, -mx, mx, -mx])
    assert np.isnan(got[1, 0]) and np.array_equal(got[1, 1:], [3.0, -65504.0, 70000.0])
    g16 = oracle.apply_opts(P, Db, sat_d=True, d_kind="f16")
    assert np.array_equal(g16[1, 1:], [3.0, -65504.0, 65504.0])
    # the clamp acts on beta * D0 + product
    assert oracle.apply_opts(np.array([[60000.0]]), np.array([[60000.0]]), beta=1, sat_d=True,
                             d_kind="f16")[0, 0] == 65504.0


def test_mask_bits_against_brute_force():
    rng = np.random.default_rng(7)
    words = rng.integers(0, 2 ** 32, size=5, dtype=np.uint64).astype(np.uint32)
    n = 150
    want = [bool((int(words[x // 32]) >> (x % 32)) & 1) for x in range(n)]
    assert list(oracle.mask_bits(words, n)) == want
