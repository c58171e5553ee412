"""gemm_run_opts (negated operands, saturated D, row mask, zero-column mask,
predicate) against the oracle's apply_opts, through the C ABI.

The options are named on the tcgen05.mma page ("Weight-stationary and block
scaling") without a definition; the readings (oracle.apply_opts) are: the
product's sign is (-1)^(neg_a + neg_b); a zero-column bit makes that column's
product zero; a row-mask bit leaves the row of D untouched; sat_d clamps each
stored value to D's largest finite magnitude (NaN kept); pred = 0 enqueues
nothing.

Tolerances are those of the plain parity tests (tests/gpu_util.py): every
output within 2 (K+1) 2^-24 (S + |beta D0|) of the exact value (plus one
unit in the last place of a bf16 / fp16 D), S the sum of the scaled
products' magnitudes, and for block-scaled operands also a relative
Frobenius error <= 2e-2; quarter-integer
operands make the fp32 result exact, so there the output must equal the
oracle bit for bit.  Masked rows and, with beta = 0, zero columns are exact
in every case.
"""
import numpy as np
import pytest
import torch

import mma_swizzled_operand_amd as mswz
import oracle
import workloads as wl
from gpu_util import reference, say, to_device

pytestmark = pytest.mark.gpu

TORCH_D = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
FRAC_BITS = {"f32": 23, "bf16": 7, "f16": 10}


def bit_words(flags: np.ndarray) -> np.ndarray:
    words = np.zeros((flags.size + 31) // 32, dtype=np.uint32)
    for x in np.flatnonzero(flags):
        words[x // 32] |= np.uint32(1) << np.uint32(x % 32)
    return words


def masks(w, seed, rows=True, cols=True):
    rng = np.random.default_rng(seed)
    rm = bit_words(rng.random(w.M) < 0.2) if rows else None
    cz = bit_words(rng.random(w.N) < 0.25) if cols else None
    return rm, cz


def run_opts(w, x, d_kind="f32", D_before=None, row_mask=None, col_zero=None, **kw):
    """One gemm_run_opts call on device copies; returns D (fp64 numpy)."""
    plan = mswz.gemm_plan_create(w.M, w.N, w.K, w.kind, w.kind_b, d_kind, w.a_major, w.b_major, w.V)
    A, B = to_device(x["A"]), to_device(x["B"])
    D = torch.from_numpy(np.ascontiguousarray(D_before)).to(TORCH_D[d_kind]).cuda()
    sf = {}
    if w.V:
        sf = {"SFA": to_device(x["SFA"]), "SFB": to_device(x["SFB"])}
    rm = to_device(row_mask.view(np.int32)) if row_mask is not None else None
    cz = to_device(col_zero.view(np.int32)) if col_zero is not None else None
    mswz.gemm_run_opts(plan, A, B, D, beta=w.beta, row_mask=rm, col_zero=cz, **sf, **kw)
    torch.cuda.synchronize()
    return D.float().cpu().numpy().astype(np.float64)


def d_before(w, x, d_kind, seed):
    """D's content before the call: D0 with beta = 1, else a sentinel pattern
    (NaN and large values, which beta = 0 must never read), in D's format."""
    if w.beta:
        d = x["D0"]
    else:
        rng = np.random.default_rng(seed)
        d = rng.uniform(-1e4, 1e4, (w.M, w.N)).astype(np.float32)
        d[::7, ::5] = np.nan
    return torch.from_numpy(d).to(TORCH_D[d_kind]).float().numpy()


def check(w, got, want, ref, d0, d_kind, rm, cz):
    """Masked rows and (beta = 0) zero columns exact, the rest within the
    parity tolerance."""
    rows = oracle.mask_bits(rm, w.M) if rm is not None else np.zeros(w.M, bool)
    assert np.array_equal(got[rows], want[rows], equal_nan=True), "masked rows changed"
    if cz is not None and not w.beta:
        cols = oracle.mask_bits(cz, w.N)
        assert np.array_equal(got[~rows][:, cols], want[~rows][:, cols]), "zero columns not zero"
    g, r = got[~rows], want[~rows]
    nan = np.isnan(r)
    assert np.array_equal(np.isnan(g), nan), "NaN positions differ"
    g, r = g[~nan], r[~nan]
    if w.V:
        rel = np.linalg.norm(g - r) / np.linalg.norm(r)
        assert rel <= 2e-2, rel
    extra = np.abs(d0[~rows][~nan]) if w.beta else 0.0
    # plus the block-scaled MFMA's in-group truncation (tests/gpu_util.py)
    tol = (2.0 ** -FRAC_BITS[d_kind] * np.abs(r) + 2 * (w.K + 1) * 2.0 ** -24 * (ref.mag[~rows][~nan] + extra)
           + ref.wabs[~rows][~nan])
    bad = np.abs(g - r) > tol
    assert not bad.any(), {"violations": int(bad.sum()), "max_err": float(np.abs(g - r).max())}


CASES = {
    # name: (workload, D kind, options)
    "bf16-neg_a-masks": (wl.custom(512, 768, 320, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                   name="bf16-neg_a-masks"), "f32", dict(neg_a=True)),
    "f16-amn-tail-neg_b-beta": (wl.custom(264, 300, 192, "f16", a_major="mn", beta=1,
                                          name="f16-amn-tail-neg_b-beta"), "f32", dict(neg_b=True)),
    "bf16-both-mn-negs": (wl.custom(256, 320, 128, "bf16", a_major="mn", b_major="mn", beta=1,
                                    name="bf16-both-mn-negs"), "f32", dict(neg_a=True, neg_b=True)),
    "bf16-skinny-plan": (wl.custom(64, 1024, 1024, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 0.02),
                                   name="bf16-skinny-plan"), "f32", dict(neg_a=True)),
    "bf16-out-neg-beta": (wl.custom(256, 512, 256, "bf16", beta=1, name="bf16-out-neg-beta"), "bf16",
                          dict(neg_b=True)),
    "e4m3-neg_a-masks": (wl.custom(512, 256, 1024, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                   name="e4m3-neg_a-masks"), "f32", dict(neg_a=True)),
    "e2m1-neg_b-beta": (wl.custom(256, 512, 512, "e2m1", V=32, beta=1, a_dist=("normal", 1.0),
                                  b_dist=("normal", 1.0), name="e2m1-neg_b-beta"), "f32", dict(neg_b=True)),
    "e3m2-neg_a-masks": (wl.custom(256, 256, 1024, "e3m2", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                   name="e3m2-neg_a-masks"), "f32", dict(neg_a=True)),
    # E4M3 with dense E2M1: split-row fragments on one side only, through the
    # staged epilogue (fp32 D) and the direct one (fp16 / bf16 D)
    "e4m3xe2m1-f16out-neg_a": (wl.custom(512, 256, 1024, "e4m3", V=32, a_dist=("normal", 1.0),
                                         b_dist=("normal", 1.0), name="e4m3xe2m1-f16out-neg_a", b_kind="e2m1"),
                               "f16", dict(neg_a=True)),
    "e2m1xe4m3-bf16out-beta-neg_b": (wl.custom(300, 264, 512, "e2m1", V=32, beta=1, a_dist=("normal", 1.0),
                                               b_dist=("normal", 1.0), name="e2m1xe4m3-bf16out-beta-neg_b",
                                               b_kind="e4m3"), "bf16", dict(neg_b=True)),
    "e2m1xe4m3-masks": (wl.custom(256, 512, 1024, "e2m1", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                  name="e2m1xe4m3-masks", b_kind="e4m3"), "f32", dict()),
}


@pytest.mark.parametrize("case", list(CASES))
def test_opts_against_oracle(case):
    w, d_kind, kw = CASES[case]
    say(f"[opts] {case} {w.M}x{w.N}x{w.K} {w.kind} {w.a_major}/{w.b_major} beta={w.beta} -> {d_kind} {kw}")
    x = wl.generate(w, seed=61)
    Db = d_before(w, x, d_kind, seed=62)
    if w.beta:
        x["D0"] = Db.astype(np.float32)
    rm, cz = masks(w, seed=63)
    got = run_opts(w, x, d_kind, Db, row_mask=rm, col_zero=cz, **kw)
    ref = reference(replace_beta(w), x)
    want = oracle.apply_opts(ref.value, Db, beta=w.beta, D0=Db, row_mask=rm, col_zero=cz, d_kind=d_kind, **kw)
    check(w, got, want, ref, Db, d_kind, rm, cz)


def replace_beta(w):
    """The same workload with beta = 0 (the oracle's product P)."""
    from dataclasses import replace
    return replace(w, beta=0)


@pytest.mark.parametrize("case", ["bf16-neg_a-masks", "f16-amn-tail-neg_b-beta", "bf16-both-mn-negs",
                                  "e4m3-neg_a-masks", "e2m1-neg_b-beta"])
def test_opts_quarter_integers_bit_exact(case):
    w, _, kw = CASES[case]
    say(f"[opts exact] {case}")
    x = wl.generate(w, seed=64, values="quarter")
    Db = d_before(w, x, "f32", seed=65)
    if w.beta:
        x["D0"] = Db.astype(np.float32)
    rm, cz = masks(w, seed=66)
    got = run_opts(w, x, "f32", Db, row_mask=rm, col_zero=cz, **kw)
    P = reference(replace_beta(w), x, with_mag=False)
    want = oracle.apply_opts(P, Db, beta=w.beta, D0=Db, row_mask=rm, col_zero=cz, **kw)
    want32 = want.astype(np.float32).astype(np.float64)   # exact sum plus D0, rounded once to fp32
    assert np.array_equal(got, want32, equal_nan=True)


@pytest.mark.parametrize("d_kind", ["f32", "f16"])
def test_saturation(d_kind):
    """beta = 1 onto a D holding its format's largest values, infinities and
    NaNs: sums beyond the largest finite value are stored as it, NaN stays."""
    w = wl.custom(256, 256, 256, "f16", beta=1, name=f"sat-{d_kind}")
    say(f"[opts sat] {d_kind}")
    x = wl.generate(w, seed=67)
    big = oracle.D_MAX[d_kind]
    d = x["D0"].astype(np.float64)
    d[0::4, :] = big
    d[1::4, 0::2] = -big
    d[2::8, :] = np.inf
    d[3::8, 1::2] = -np.inf
    d[6::16, 3::4] = np.nan
    Db = torch.from_numpy(d.astype(np.float32)).to(TORCH_D[d_kind]).float().numpy().astype(np.float64)
    x["D0"] = Db.astype(np.float32)
    got = run_opts(w, x, d_kind, Db, sat_d=True, neg_a=True)
    P, mag = reference(replace_beta(w), x)
    want = oracle.apply_opts(P, Db, beta=1, D0=Db, sat_d=True, neg_a=True, d_kind=d_kind)
    fin = np.isfinite(want)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.isfinite(got[fin]).all() and np.abs(got[fin]).max() <= big
    clamped = np.abs(want) == big
    assert clamped.sum() > w.N, "the case must reach the clamp"
    assert np.array_equal(got[clamped], want[clamped])
    rest = fin & ~clamped
    tol = 2.0 ** -FRAC_BITS[d_kind] * np.abs(want[rest]) + 2 * (w.K + 1) * 2.0 ** -24 * (mag[rest] + np.abs(Db[rest]))
    assert (np.abs(got[rest] - want[rest]) <= tol).all()


def test_pred_false_and_no_op_options():
    w = wl.custom(256, 256, 128, "bf16", name="pred")
    say("[opts pred]")
    x = wl.generate(w, seed=68)
    Db = d_before(w, x, "f32", seed=69)
    rm, cz = masks(w, seed=70)
    got = run_opts(w, x, "f32", Db, row_mask=rm, col_zero=cz, neg_a=True, sat_d=True, pred=False)
    assert np.array_equal(got, Db, equal_nan=True)
    # neg_a and neg_b together, no masks: exactly gemm_run
    both = run_opts(w, x, "f32", Db, neg_a=True, neg_b=True)
    plan = mswz.gemm_plan_create(w.M, w.N, w.K, "bf16", "bf16")
    D = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    mswz.gemm_run(plan, to_device(x["A"]), to_device(x["B"]), D, 0)
    torch.cuda.synchronize()
    assert np.array_equal(both, D.cpu().numpy().astype(np.float64))


def test_opts_full_size_sampled():
    """The 4096^3 bf16 workload with both masks and neg_a, on sampled rows and
    columns (masked rows exact, the rest within tolerance)."""
    w = wl.WORKLOADS["c2"]
    say("[opts full] c2 4096^3 with masks and neg_a")
    x = wl.generate(w, seed=0)
    Db = np.full((w.M, w.N), 0.5, dtype=np.float32)
    rm, cz = masks(w, seed=71)
    got = run_opts(w, x, "f32", Db, row_mask=rm, col_zero=cz, neg_a=True)
    rows, cols = wl.sample_points(w, 12, 12, seed=72)
    rows = np.unique(np.concatenate([rows, np.flatnonzero(oracle.mask_bits(rm, w.M))[:4]]))
    P, mag = reference(w, x, rows=rows, cols=cols)
    masked_r = oracle.mask_bits(rm, w.M)[rows]
    zero_c = oracle.mask_bits(cz, w.N)[cols]
    want = oracle.apply_opts(P, Db[np.ix_(rows, cols)], row_mask=bit_words(masked_r),
                             col_zero=bit_words(zero_c), neg_a=True)
    sub = got[np.ix_(rows, cols)]
    assert masked_r.any() and zero_c.any()
    assert np.array_equal(sub[masked_r], want[masked_r])
    assert np.array_equal(sub[~masked_r][:, zero_c], want[~masked_r][:, zero_c])
    tol = 2 * (w.K + 1) * 2.0 ** -24 * mag[~masked_r]
    assert (np.abs(sub[~masked_r] - want[~masked_r]) <= tol).all()
