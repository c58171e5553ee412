"""GPU parity on seeded random shapes: every operand kind and combination the
plan accepts, both majors where they exist, beta 0 and 1, with M, N and K
drawn at random inside the shape rules of include/mswz_gemm.h (tails in M, N
and K, single rows and columns, K below one step), each compared element by
element with the fp64 oracle under the bounds of tests/gpu_util.py.

The cases are drawn once, at import, from a fixed seed, so a failing case
keeps its name and shape from run to run.
"""
import numpy as np
import pytest

import workloads as wl
from gpu_util import compare, plan_for, reference, run_gpu, say

pytestmark = pytest.mark.gpu

DENSE = ["bf16", "f16"]
MX = ["e4m3", "e2m1", "e2m3", "e3m2", "e2m1p"]
MIXABLE = ["e4m3", "e2m3", "e3m2", "e2m1p"]
V16_KINDS = ["e2m1", "e2m1p", "e2m3", "e3m2"]
MAX_WORK = 2.0e8          # M * N * K per case: the oracle finishes each in well under a second


def _draw(rng, i):
    r = rng.random()
    a_major = b_major = "k"
    V, kb = 0, ""
    if r < 0.35:
        ka = DENSE[rng.integers(2)]
        a_major = "mn" if rng.random() < 0.4 else "k"
        b_major = "mn" if rng.random() < 0.4 else "k"
        kstep = 8
    elif r < 0.65:
        ka = MX[rng.integers(len(MX))]
        V = 16 if ka in V16_KINDS and rng.random() < 0.3 else 32
        kstep = 32 if ka == "e2m1" else V
    elif r < 0.9:
        ka, kb = rng.choice(MIXABLE, 2, replace=False)
        V, kstep = 32, 32
    else:
        ka, kb = ("e4m3", "e2m1") if rng.random() < 0.5 else ("e2m1", "e4m3")
        V, kstep = 32, 256
    M = int(rng.integers(1, 641))
    N = 4 * int(rng.integers(1, 161))
    if a_major == "mn":
        M = max(8, M - M % 8)
    if b_major == "mn":
        N = max(8, N - N % 8)
    K = kstep * int(rng.integers(1, 1536 // kstep + 1))
    while M * N * K > MAX_WORK and K > kstep:
        K = max(kstep, (K // 2) // kstep * kstep)
    beta = int(rng.random() < 0.3)
    dist = ("normal", 1.0) if rng.random() < 0.5 else ("uniform", 1.0)
    majors = ("" if a_major == "k" else "-amn") + ("" if b_major == "k" else "-bmn")
    kinds = ka if not kb else f"{ka}x{kb}"
    name = f"r{i:03d}-{kinds}{majors}-v{V}-{M}x{N}x{K}" + ("-beta" if beta else "")
    return wl.custom(M, N, K, str(ka), a_major=a_major, b_major=b_major, beta=beta, V=V,
                     a_dist=dist, b_dist=dist, name=name, b_kind=str(kb))


_rng = np.random.default_rng(20261202)
CASES = {w.name: w for w in (_draw(_rng, i) for i in range(192))}


@pytest.mark.parametrize("name", list(CASES))
def test_random_shape_full_compare(name):
    w = CASES[name]
    plan = plan_for(w)
    say(f"[random] {name} plan {plan.describe()}")
    x = wl.generate(w, seed=int(name[1:4]) + 100)
    got = run_gpu(w, x, plan)
    ref = reference(w, x)
    print(name, compare(w, got, ref, x.get("D0")))


# every fourth case again with bf16 or fp16 D (the fp32 result rounded once;
# with beta = 1 the old D read in D's format), under the bound of
# tests/test_gpu_narrow_d.py
NARROW = {name + ("-bf16d" if i % 8 == 0 else "-f16d"): (w, "bf16" if i % 8 == 0 else "f16")
          for i, (name, w) in enumerate(CASES.items()) if i % 4 == 0}


@pytest.mark.parametrize("case", list(NARROW))
def test_random_shape_narrow_d(case):
    from test_gpu_narrow_d import FRAC_BITS, inputs, run_narrow
    w, d_kind = NARROW[case]
    say(f"[random] {case}")
    x = inputs(w, d_kind, seed=int(case[1:4]) + 300)
    got = run_narrow(w, x, d_kind)
    r = reference(w, x)
    ref, mag = r
    extra = np.abs(x["D0"].astype(np.float64)) if w.beta else 0.0
    tol = 2.0 ** -FRAC_BITS[d_kind] * np.abs(ref) + 1.01 * 2 * (w.K + 1) * 2.0 ** -24 * (mag + extra) + r.wabs
    bad = np.abs(got - ref) > tol
    assert not bad.any(), {"violations": int(bad.sum()), "max_err": float(np.abs(got - ref).max())}
