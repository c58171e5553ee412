"""bf16 / fp16 output D (the fp32 result rounded to nearest even into D's
format; with beta = 1 the old D, read in that format, is added in fp32 first)
against the oracle, through the C ABI.

Tolerance: one unit in the last place of D's format relative to the exact
value (rounding) plus the fp32 accumulation bound of the dense cases
(tests/gpu_util.py), scaled by 1.01.  Quarter-integer operands make the fp32
result exact, so there the output must equal the exact value rounded to
nearest even by torch, bit for bit.
"""
import numpy as np
import pytest
import torch

import mma_swizzled_operand_amd as mswz
import workloads as wl
from gpu_util import reference, say, to_device

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "f16": torch.float16}
FRAC_BITS = {"bf16": 7, "f16": 10}

CASES = {
    "bf16-out": (wl.custom(512, 768, 320, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                           name="bf16-out"), "bf16"),
    "f16-out-beta": (wl.custom(256, 512, 256, "f16", beta=1, name="f16-out-beta"), "f16"),
    "bf16-out-amn-tail": (wl.custom(264, 300, 192, "bf16", a_major="mn", name="bf16-out-amn-tail"), "bf16"),
    "e4m3-bf16-out": (wl.custom(512, 256, 1024, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                name="e4m3-bf16-out"), "bf16"),
    "e2m1-f16-out-beta": (wl.custom(256, 256, 512, "e2m1", V=32, beta=1, a_dist=("normal", 1.0),
                                    b_dist=("normal", 1.0), name="e2m1-f16-out-beta"), "f16"),
    "e2m3-bf16-out": (wl.custom(256, 512, 1024, "e2m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                name="e2m3-bf16-out"), "bf16"),
}


def run_narrow(w, x, d_kind):
    plan = mswz.gemm_plan_create(w.M, w.N, w.K, w.kind, w.kind_b, d_kind, w.a_major, w.b_major, w.V)
    assert plan.describe()["tile_m"] == 256
    A, B = to_device(x["A"]), to_device(x["B"])
    if w.beta:
        D = x["D0n"].clone().cuda()
    else:
        D = torch.zeros((w.M, w.N), dtype=TORCH[d_kind], device="cuda")
    if w.V:
        mswz.gemm_run_blockscaled(plan, A, B, to_device(x["SFA"]), to_device(x["SFB"]), D, w.beta)
    else:
        mswz.gemm_run(plan, A, B, D, w.beta)
    torch.cuda.synchronize()
    return D.float().cpu().numpy().astype(np.float64)


def inputs(w, d_kind, seed, values="config"):
    x = wl.generate(w, seed=seed, values=values)
    if w.beta:
        # D0 in D's format; the oracle reads the same values as fp32
        d0n = torch.from_numpy(x["D0"]).to(TORCH[d_kind])
        x["D0n"] = d0n
        x["D0"] = d0n.float().numpy()
    return x


@pytest.mark.parametrize("case", list(CASES))
def test_narrow_d_against_oracle(case):
    w, d_kind = CASES[case]
    say(f"[narrow-d] {case} {w.M}x{w.N}x{w.K} {w.kind} -> {d_kind} beta={w.beta}")
    x = inputs(w, d_kind, seed=51)
    got = run_narrow(w, x, d_kind)
    r = reference(w, x)
    ref, mag = r
    extra = np.abs(x["D0"].astype(np.float64)) if w.beta else 0.0
    # plus the block-scaled MFMA's in-group truncation (tests/gpu_util.py)
    tol = 2.0 ** -FRAC_BITS[d_kind] * np.abs(ref) + 1.01 * 2 * (w.K + 1) * 2.0 ** -24 * (mag + extra) + r.wabs
    if w.V:   # block-scaled: the global norm gate of the block-scaled cases as well
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel <= 2e-2, rel
    bad = np.abs(got - ref) > tol
    assert not bad.any(), {"violations": int(bad.sum()), "max_err": float(np.abs(got - ref).max())}


@pytest.mark.parametrize("case", ["bf16-out", "f16-out-beta", "e2m1-f16-out-beta"])
def test_narrow_d_quarter_integers_round_like_torch(case):
    """Exact fp32 result: the output is that value rounded to nearest even."""
    w, d_kind = CASES[case]
    say(f"[narrow-d exact] {case}")
    x = inputs(w, d_kind, seed=52, values="quarter")
    got = run_narrow(w, x, d_kind)
    ref = reference(w, x, with_mag=False)
    want = torch.from_numpy(ref.astype(np.float32)).to(TORCH[d_kind]).float().numpy().astype(np.float64)
    assert np.array_equal(got, want)
