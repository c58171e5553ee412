"""Pins for the oracle GEMM (CPU only).

The oracle computes D = beta*D0 + A.B^T with B held as (N,K) (tcgen05.mma
page, "Operands and repeat axes" and the 128x64x64 example), reading operands
through their majors ("Shared descriptors are byte-stride contracts": K-major
rows enumerate M/N, MN-major rows enumerate K), with optional per-row block
scales ("Weight-stationary and block scaling").  Each test below fixes its
answer by something other than the oracle itself: closed forms, exact rational
arithmetic, invariants, the page's worked example, or numpy's float64 matmul.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

KINDS = ("f16", "bf16", "e4m3")
ONE = {"f16": 0x3C00, "bf16": 0x3F80, "e4m3": 0x38}


def _stored(kind, x):
    return wl.to_stored(np.asarray(x, dtype=np.float64), kind)


def _store_major(x_logical, major):
    """x_logical is [R][K]; K-major storage is itself, MN-major is [K][R]."""
    return np.ascontiguousarray(x_logical if major == "k" else x_logical.T)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("amaj", ["k", "mn"])
@pytest.mark.parametrize("bmaj", ["k", "mn"])
def test_all_ones_gives_K(kind, amaj, bmaj):
    M, N, K = 7, 5, 96
    dt = np.uint16 if kind != "e4m3" else np.uint8
    A = np.full((M * K,), ONE[kind], dtype=dt)
    B = np.full((N * K,), ONE[kind], dtype=dt)
    D = oracle.gemm(M, N, K, kind, amaj, A, kind, bmaj, B)
    assert (D == K).all()


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("bmaj", ["k", "mn"])
def test_identity_A_gives_B_transposed(kind, bmaj):
    K = N = 24
    rng = np.random.default_rng(3)
    b = rng.uniform(-1, 1, (N, K))
    Bs = _store_major(_stored(kind, b), bmaj)
    A = _stored(kind, np.eye(K))
    D = oracle.gemm(K, N, K, kind, "k", A, kind, bmaj, Bs)
    bval = oracle.decode(kind, _stored(kind, b))          # [N][K]
    assert np.array_equal(D, bval.T)


@pytest.mark.parametrize("amaj", ["k", "mn"])
def test_permutation_A_permutes_rows(amaj):
    kind, K, N = "bf16", 32, 9
    rng = np.random.default_rng(4)
    perm = rng.permutation(K)
    P = np.zeros((K, K))
    P[np.arange(K), perm] = 1.0                          # a(m,k) = [k == perm[m]]
    b = rng.normal(0, 1, (N, K))
    D = oracle.gemm(K, N, K, kind, amaj, _store_major(_stored(kind, P), amaj),
                    kind, "k", _stored(kind, b))
    bval = oracle.decode(kind, _stored(kind, b))
    assert np.array_equal(D, bval[:, perm].T)


def test_zero_A_with_beta_returns_D0_exactly():
    M, N, K = 6, 10, 64
    rng = np.random.default_rng(5)
    D0 = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    A = np.zeros(M * K, dtype=np.uint16)
    B = _stored("f16", rng.uniform(-1, 1, (N, K)))
    D = oracle.gemm(M, N, K, "f16", "k", A, "f16", "k", B, beta=1, D0=D0)
    assert np.array_equal(D, D0.astype(np.float64))


def test_beta_zero_never_reads_D0():
    M, N, K = 4, 4, 8
    A = np.full(M * K, ONE["f16"], dtype=np.uint16)
    B = np.full(N * K, ONE["f16"], dtype=np.uint16)
    D0 = np.full((M, N), np.nan, dtype=np.float32)
    D = oracle.gemm(M, N, K, "f16", "k", A, "f16", "k", B, beta=0, D0=D0)
    assert (D == K).all()


def _exact(kind, a_st, b_st, M, N, K, D0=None, sfa=None, sfb=None, V=0):
    """Exact rational result from the decoded values (brute-force triple loop)."""
    av = oracle.decode(kind, a_st).reshape(M, K)
    bv = oracle.decode(kind, b_st).reshape(N, K)
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                x = Fraction(av[m, k])
                y = Fraction(bv[n, k])
                if V:
                    x *= Fraction(2) ** (int(sfa[m, k // V]) - 127)
                    y *= Fraction(2) ** (int(sfb[n, k // V]) - 127)
                s += x * y
            if D0 is not None:
                s += Fraction(float(D0[m, n]))
            out[m][n] = s
    return out


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 5), (3, 5, 8), (5, 8, 17), (8, 17, 3), (17, 2, 32)])
def test_tiny_shapes_against_exact_rationals(kind, M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    a_st = _stored(kind, rng.uniform(-1, 1, (M, K)))
    b_st = _stored(kind, rng.uniform(-1, 1, (N, K)))
    D0 = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    got, mag = oracle.gemm(M, N, K, kind, "k", a_st, kind, "k", b_st, beta=1, D0=D0, with_mag=True)
    ex = _exact(kind, a_st, b_st, M, N, K, D0=D0)
    for m in range(M):
        for n in range(N):
            err = abs(Fraction(got[m, n]) - ex[m][n])
            # fp64 summation of K exact products plus D0: at most (K+1) roundings
            bound = Fraction((K + 1) * 2.0 ** -53) * (Fraction(mag[m, n]) + abs(Fraction(float(D0[m, n]))))
            assert err <= bound


@pytest.mark.parametrize("kind", KINDS)
def test_exact_small_fp16_e4m3_products_are_bit_exact(kind):
    """fp16 products are multiples of 2^-48 and e4m3 products multiples of
    2^-18, all below 1 in magnitude, so with K <= 32 every fp64 partial sum is
    exact and the oracle must equal the rational result bit for bit."""
    if kind == "bf16":
        pytest.skip("bf16 products can span more than 53 bits of exponent range")
    M, N, K = 5, 7, 32
    rng = np.random.default_rng(11)
    a_st = _stored(kind, rng.uniform(-1, 1, (M, K)))
    b_st = _stored(kind, rng.uniform(-1, 1, (N, K)))
    got = oracle.gemm(M, N, K, kind, "k", a_st, kind, "k", b_st)
    ex = _exact(kind, a_st, b_st, M, N, K)
    for m in range(M):
        for n in range(N):
            assert Fraction(got[m, n]) == ex[m][n]


@pytest.mark.parametrize("kind", KINDS)
def test_majors_are_pure_relabelling(kind):
    M, N, K = 19, 13, 40
    rng = np.random.default_rng(7)
    a = _stored(kind, rng.uniform(-1, 1, (M, K)))
    b = _stored(kind, rng.uniform(-1, 1, (N, K)))
    ref = oracle.gemm(M, N, K, kind, "k", a, kind, "k", b)
    for amaj in ("k", "mn"):
        for bmaj in ("k", "mn"):
            got = oracle.gemm(M, N, K, kind, amaj, _store_major(a, amaj), kind, bmaj, _store_major(b, bmaj))
            assert np.array_equal(got, ref)


def test_page_worked_example_quarter_integers():
    """The tcgen05.mma page's example draws integers in [-4, 4] / 4 with
    default_rng(0) for A (128,64) and B (64,64) stored (N,K) in fp16 and
    compares with fp32 a @ b.T; with these values every product and partial
    sum is exact, so the oracle equals that fp32 result exactly."""
    rng = np.random.default_rng(0)
    a = (rng.integers(-4, 5, (128, 64)) / 4).astype("float16")
    b = (rng.integers(-4, 5, (64, 64)) / 4).astype("float16")
    ref32 = a.astype("float32") @ b.astype("float32").T
    got = oracle.gemm(128, 64, 64, "f16", "k", a.view(np.uint16), "f16", "k", b.view(np.uint16))
    assert np.array_equal(got, ref32.astype(np.float64))
    # and the same at the single-tile config's shape (128x256x64)
    b2 = (rng.integers(-4, 5, (256, 64)) / 4).astype("float16")
    got2 = oracle.gemm(128, 256, 64, "f16", "k", a.view(np.uint16), "f16", "k", b2.view(np.uint16))
    assert np.array_equal(got2, (a.astype("float32") @ b2.astype("float32").T).astype(np.float64))


@pytest.mark.parametrize("kind,amaj", [("f16", "k"), ("bf16", "mn"), ("e4m3", "k")])
def test_medium_against_numpy_float64_matmul(kind, amaj):
    M, N, K = 96, 80, 320
    rng = np.random.default_rng(9)
    a = _stored(kind, rng.normal(0, 1, (M, K)))
    b = _stored(kind, rng.normal(0, 1, (N, K)))
    D0 = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    got = oracle.gemm(M, N, K, kind, amaj, _store_major(a, amaj), kind, "k", b, beta=1, D0=D0)
    ref = oracle.decode(kind, a).reshape(M, K) @ oracle.decode(kind, b).reshape(N, K).T + D0
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_row_col_selection_matches_full():
    w = wl.custom(64, 96, 128, "bf16", a_major="mn", beta=1)
    x = wl.generate(w, seed=2)
    full = oracle.gemm(w.M, w.N, w.K, "bf16", "mn", x["A"], "bf16", "k", x["B"], beta=1, D0=x["D0"])
    rows = np.array([0, 5, 63])
    cols = np.array([1, 95, 40, 2])
    sub = oracle.gemm(w.M, w.N, w.K, "bf16", "mn", x["A"], "bf16", "k", x["B"], beta=1, D0=x["D0"],
                      rows=rows, cols=cols)
    assert np.array_equal(sub, full[np.ix_(rows, cols)])


# ---- block-scaled -----------------------------------------------------------

def _mx_inputs(M, N, K, seed, V=32):
    rng = np.random.default_rng(seed)
    a = _stored("e4m3", rng.normal(0, 1, (M, K)))
    b = _stored("e4m3", rng.normal(0, 1, (N, K)))
    sfa = (127 + rng.integers(-4, 5, (M, K // V))).astype(np.uint8)
    sfb = (127 + rng.integers(-4, 5, (N, K // V))).astype(np.uint8)
    return a, b, sfa, sfb


def test_unit_scales_equal_dense():
    M, N, K = 12, 9, 128
    a, b, _, _ = _mx_inputs(M, N, K, 1)
    ones_a = np.full((M, K // 32), 127, dtype=np.uint8)
    ones_b = np.full((N, K // 32), 127, dtype=np.uint8)
    scaled = oracle.gemm(M, N, K, "e4m3", "k", a, "e4m3", "k", b, V=32, SFA=ones_a, SFB=ones_b)
    dense = oracle.gemm(M, N, K, "e4m3", "k", a, "e4m3", "k", b)
    assert np.array_equal(scaled, dense)


def test_all_ones_values_closed_form_with_scales():
    """a = b = 1 everywhere: D[m,n] = 32 * sum_j 2^(uA[m,j] + uB[n,j])."""
    M, N, K = 6, 5, 256
    _, _, sfa, sfb = _mx_inputs(M, N, K, 2)
    a = np.full(M * K, ONE["e4m3"], dtype=np.uint8)
    b = np.full(N * K, ONE["e4m3"], dtype=np.uint8)
    D = oracle.gemm(M, N, K, "e4m3", "k", a, "e4m3", "k", b, V=32, SFA=sfa, SFB=sfb)
    ua = sfa.astype(np.int64) - 127
    ub = sfb.astype(np.int64) - 127
    for m in range(M):
        for n in range(N):
            assert D[m, n] == sum(32 * 2.0 ** (ua[m, j] + ub[n, j]) for j in range(K // 32))


def test_scale_row_increment_doubles_that_row_only():
    M, N, K = 8, 7, 96
    a, b, sfa, sfb = _mx_inputs(M, N, K, 3)
    base = oracle.gemm(M, N, K, "e4m3", "k", a, "e4m3", "k", b, V=32, SFA=sfa, SFB=sfb)
    sfa2 = sfa.copy()
    sfa2[3, :] += 1
    twice = oracle.gemm(M, N, K, "e4m3", "k", a, "e4m3", "k", b, V=32, SFA=sfa2, SFB=sfb)
    assert np.array_equal(twice[3], 2 * base[3])
    keep = [i for i in range(M) if i != 3]
    assert np.array_equal(twice[keep], base[keep])
    # one block of one column's scale: only that column changes, by the block's share
    sfb2 = sfb.copy()
    sfb2[4, 1] += 1
    col = oracle.gemm(M, N, K, "e4m3", "k", a, "e4m3", "k", b, V=32, SFA=sfa, SFB=sfb2)
    other = [j for j in range(N) if j != 4]
    assert np.array_equal(col[:, other], base[:, other])
    assert not np.array_equal(col[:, 4], base[:, 4])


def test_blockscaled_exact_against_rationals():
    M, N, K = 3, 4, 64
    a, b, sfa, sfb = _mx_inputs(M, N, K, 4)
    got = oracle.gemm(M, N, K, "e4m3", "k", a, "e4m3", "k", b, V=32, SFA=sfa, SFB=sfb)
    ex = _exact("e4m3", a, b, M, N, K, sfa=sfa, sfb=sfb, V=32)
    for m in range(M):
        for n in range(N):
            assert Fraction(got[m, n]) == ex[m][n]


def test_rejections():
    A = np.zeros(16, dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm(4, 4, 4, "f16", "k", A, "f16", "k", A, beta=2, D0=np.zeros((4, 4), np.float32))
    with pytest.raises(ValueError):
        oracle.gemm(4, 4, 4, "f16", "k", A, "f16", "k", A, rows=[9])
    with pytest.raises(ValueError):
        oracle.gemm(4, 4, 3, "f16", "k", A[:12], "f16", "k", A[:12], V=2,
                    SFA=np.zeros(8, np.uint8), SFB=np.zeros(8, np.uint8))


def _e2m1_to_e4m3(packed: np.ndarray) -> np.ndarray:
    """The same values as E4M3 bytes (every E2M1 value is an E4M3 value)."""
    vals = oracle.decode("e2m1", packed)
    t = torch.from_numpy(vals.astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("M,N,K", [(3, 5, 64), (16, 9, 256)])
def test_e2m1_gemm_equals_e4m3_gemm_of_the_same_values(M, N, K):
    """Packed-nibble access and the E2M1 decoder against the torch-pinned E4M3
    path: both operands re-encoded as E4M3 give the identical result, with
    random block scales and beta = 1."""
    rng = np.random.default_rng(41)
    A = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    B = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    SFA = (127 + rng.integers(-3, 4, (M, K // 32))).astype(np.uint8)
    SFB = (127 + rng.integers(-3, 4, (N, K // 32))).astype(np.uint8)
    D0 = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    got = oracle.gemm(M, N, K, "e2m1", "k", A, "e2m1", "k", B, V=32, SFA=SFA, SFB=SFB, beta=1, D0=D0)
    ref = oracle.gemm(M, N, K, "e4m3", "k", _e2m1_to_e4m3(A), "e4m3", "k", _e2m1_to_e4m3(B),
                      V=32, SFA=SFA, SFB=SFB, beta=1, D0=D0)
    assert np.array_equal(got, ref)


def test_e2m1_all_ones_closed_form():
    """Every element 1.0 (code 0x2, byte 0x22) with unit scales: every entry is K."""
    M, N, K = 4, 6, 128
    A = np.full((M, K // 2), 0x22, np.uint8)
    B = np.full((N, K // 2), 0x22, np.uint8)
    one = np.full((M, K // 32), 127, np.uint8)
    got = oracle.gemm(M, N, K, "e2m1", "k", A, "e2m1", "k", B, V=32, SFA=one,
                      SFB=np.full((N, K // 32), 127, np.uint8))
    assert np.array_equal(got, np.full((M, N), float(K)))


# ---- 16-element scale blocks (the pages' scale_vec::4X for 4-bit operands) ---

@pytest.mark.parametrize("kind", ["e2m1", "e2m1p", "e2m3"])
def test_sixteen_element_blocks(kind):
    """V = 16: every pair of 16-blocks sharing a scale equals V = 32 with that
    scale; all-ones values give D[m,n] = 16 * sum_q 2^(uA[m,q] + uB[n,q]); and
    the exact rational sum on a tiny shape."""
    import workloads as wl
    M, N, K = 5, 6, 256
    rng = np.random.default_rng(21)
    A = wl.to_stored(rng.normal(0, 2, (M, K)), kind)
    B = wl.to_stored(rng.normal(0, 2, (N, K)), kind)
    s32a = (127 + rng.integers(-4, 5, (M, K // 32))).astype(np.uint8)
    s32b = (127 + rng.integers(-4, 5, (N, K // 32))).astype(np.uint8)
    d32 = oracle.gemm(M, N, K, kind, "k", A, kind, "k", B, V=32, SFA=s32a, SFB=s32b)
    d16 = oracle.gemm(M, N, K, kind, "k", A, kind, "k", B, V=16, SFA=np.repeat(s32a, 2, axis=1),
                      SFB=np.repeat(s32b, 2, axis=1))
    assert np.array_equal(d16, d32)
    ones_a = wl.to_stored(np.ones((M, K)), kind)
    ones_b = wl.to_stored(np.ones((N, K)), kind)
    sa = (127 + rng.integers(-4, 5, (M, K // 16))).astype(np.uint8)
    sb = (127 + rng.integers(-4, 5, (N, K // 16))).astype(np.uint8)
    D = oracle.gemm(M, N, K, kind, "k", ones_a, kind, "k", ones_b, V=16, SFA=sa, SFB=sb)
    ua, ub = sa.astype(np.int64) - 127, sb.astype(np.int64) - 127
    want = 16.0 * np.exp2(ua[:, None, :] + ub[None, :, :]).sum(-1)
    assert np.array_equal(D, want)
    # exact rationals: every product and scale is a dyadic rational
    vals_a, vals_b = oracle.decode(kind, A), oracle.decode(kind, B)
    got = oracle.gemm(M, N, K, kind, "k", A, kind, "k", B, V=16, SFA=sa, SFB=sb)
    for m in range(M):
        for n in range(N):
            ex = sum(Fraction(vals_a[m, k]) * Fraction(vals_b[n, k]) * Fraction(2) ** int(ua[m, k // 16] + ub[n, k // 16])
                     for k in range(K))
            assert Fraction(got[m, n]) == ex


@pytest.mark.parametrize("kind,kind_b,V,beta", [("e4m3", "", 32, 0), ("e2m1", "", 16, 1), ("e2m3", "", 32, 0),
                                                 ("e3m2", "e4m3", 32, 1), ("e2m1p", "", 16, 0)])
def test_quarter_scaled_inputs_give_fp32_exact_products(kind, kind_b, V, beta):
    """The exactness argument behind the GPU's bit-exact random-scale tests:
    with quarter-integer (E2M1: half-integer) values and scales 2^u, u in
    [-2, 2], at K = 4096 the exact product A.B^T is a multiple of 2^-8 of
    magnitude at most 2^16, so it is representable in fp32; checked here on
    the oracle's fp64 result."""
    w = wl.custom(32, 48, 4096, kind, V=V, b_kind=kind_b, beta=beta)
    x = wl.generate(w, seed=5, values="quarter_scaled")
    assert set(np.unique(x["SFA"])) == set(range(125, 130))
    P = oracle.gemm(w.M, w.N, w.K, w.kind, "k", x["A"], w.kind_b, "k", x["B"], V=w.V, SFA=x["SFA"], SFB=x["SFB"])
    assert np.all(np.abs(P) <= 2.0 ** 16)
    assert np.array_equal(np.round(P * 256), P * 256)
    assert np.array_equal(P.astype(np.float32).astype(np.float64), P)
