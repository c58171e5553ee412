"""GPU parity of block-scaled plans with MN-major scales (gemm_plan_set_scale_major):
SFA stored [K/V][M] and SFB [K/V][N], the tcgen05.mma page's "Operands and
repeat axes" order (the K-repeat axis outside the rows).  The scale values are
the oracle's own ([M][K/V] and [N][K/V]); only their storage is transposed
before the call.  Every case is compared element by element with the fp64
oracle under the bounds of tests/gpu_util.py, and bit for bit with the same
plan run on row-major scales (the same kernel arithmetic, other addresses).
"""
import os

import numpy as np
import pytest
import torch

import mma_swizzled_operand_amd as mswz
import workloads as wl
from gpu_util import compare, reference, run_gpu, say, to_device

pytestmark = pytest.mark.gpu

N01 = ("normal", 1.0)


def _w(name, M, N, K, ka, kb="", beta=0):
    return wl.custom(M, N, K, ka, V=32, beta=beta, a_dist=N01, b_dist=N01, name=name, b_kind=kb)


# every kind combination that takes MN-major scales; M and N multiples of 16
# with tail tiles of 16 .. 240 rows; K one, two and three 32-block groups
# (the wide loop) and other multiples of the K step (the per-step loop)
CASES = {w.name: w for w in [
    _w("e4m3-1040x528-k2048", 1040, 528, 2048, "e4m3"),
    _w("e4m3-256x512-k4096-beta", 256, 512, 4096, "e4m3", beta=1),
    _w("e4m3-304x272-k6144", 304, 272, 6144, "e4m3"),
    _w("e4m3-16x16-k2048", 16, 16, 2048, "e4m3"),
    _w("e4m3xe2m3-528x1040-k2048-beta", 528, 1040, 2048, "e4m3", "e2m3", beta=1),
    _w("e4m3xe3m2-256x256-k4096", 256, 256, 4096, "e4m3", "e3m2"),
    _w("e4m3xe2m1p-400x304-k2048", 400, 304, 2048, "e4m3", "e2m1p"),
    _w("e2m3-1040x272-k2048", 1040, 272, 2048, "e2m3"),
    _w("e3m2-256x512-k4096-beta", 256, 512, 4096, "e3m2", beta=1),
    _w("e2m1p-304x528-k2048", 304, 528, 2048, "e2m1p"),
    _w("e2m1-1040x272-k2048", 1040, 272, 2048, "e2m1"),
    _w("e2m1-304x528-k4096-beta", 304, 528, 4096, "e2m1", beta=1),
    _w("e2m1-256x256-k6144", 256, 256, 6144, "e2m1"),
    # K not a multiple of 2048: the per-step loop (one K step's scales per
    # copy), single-step K included
    _w("e4m3-528x272-k640", 528, 272, 640, "e4m3"),
    _w("e4m3-272x528-k3072-beta", 272, 528, 3072, "e4m3", beta=1),
    _w("e4m3xe2m1p-304x400-k1152", 304, 400, 1152, "e4m3", "e2m1p"),
    _w("e4m3xe3m2-256x256-k1024", 256, 256, 1024, "e4m3", "e3m2"),
    _w("e2m3-272x304-k1408-beta", 272, 304, 1408, "e2m3", beta=1),
    _w("e3m2-400x272-k128", 400, 272, 128, "e3m2"),
    _w("e2m1p-256x528-k384", 256, 528, 384, "e2m1p"),
    _w("e2m1-528x272-k768", 528, 272, 768, "e2m1"),
    _w("e2m1-304x304-k1280-beta", 304, 304, 1280, "e2m1", beta=1),
    _w("e2m1-256x256-k256", 256, 256, 256, "e2m1"),
    # a 6-bit or padded 4-bit A with another kind of B (the per-step loop
    # for every K)
    _w("e2m3xe4m3-528x272-k2048", 528, 272, 2048, "e2m3", "e4m3"),
    _w("e3m2xe2m1p-304x400-k1152-beta", 304, 400, 1152, "e3m2", "e2m1p", beta=1),
    _w("e2m1pxe2m3-272x272-k4096", 272, 272, 4096, "e2m1p", "e2m3"),
    _w("e2m3xe3m2-256x528-k640", 256, 528, 640, "e2m3", "e3m2"),
    # E4M3 A with dense E2M1 B (K a multiple of 256; the per-step loop)
    _w("e4m3xe2m1-528x272-k2048", 528, 272, 2048, "e4m3", "e2m1"),
    _w("e4m3xe2m1-304x400-k1280-beta", 304, 400, 1280, "e4m3", "e2m1", beta=1),
    _w("e4m3xe2m1-256x256-k256", 256, 256, 256, "e4m3", "e2m1"),
]}


def mn_plan(w, d_dt="f32"):
    plan = mswz.gemm_plan_create(w.M, w.N, w.K, w.kind, w.kind_b, d_dt, "k", "k", w.V)
    mswz.gemm_plan_set_scale_major(plan, "mn")
    return plan


def mn_scales(x):
    """The same scale values stored [K/V][rows]."""
    y = dict(x)
    y["SFA"] = np.ascontiguousarray(x["SFA"].T)
    y["SFB"] = np.ascontiguousarray(x["SFB"].T)
    return y


def row_major_plan(w, d_dt="f32"):
    """The same kernel with row-major scales: the 256x256 tile, which MN-major
    scales always take (MSWZ_TILE, read when a plan is created, overrides the
    smaller tiles chosen for small grids)."""
    old = os.environ.get("MSWZ_TILE")
    os.environ["MSWZ_TILE"] = "256"
    try:
        plan = mswz.gemm_plan_create(w.M, w.N, w.K, w.kind, w.kind_b, d_dt, "k", "k", w.V)
    finally:
        if old is None:
            os.environ.pop("MSWZ_TILE", None)
        else:
            os.environ["MSWZ_TILE"] = old
    assert plan.describe()["tile_m"] == 256
    return plan


@pytest.mark.parametrize("name", list(CASES))
def test_mn_scales_full_compare(name):
    w = CASES[name]
    plan = mn_plan(w)
    say(f"[sf-mn] {name} plan {plan.describe()}")
    x = wl.generate(w, seed=41)
    got = run_gpu(w, mn_scales(x), plan)
    print(name, compare(w, got, reference(w, x), x.get("D0")))
    assert np.array_equal(got, run_gpu(w, x, row_major_plan(w)))


@pytest.mark.parametrize("name", [n for n in CASES if CASES[n].K <= 4096])
def test_mn_scales_random_scales_bit_exact(name):
    """Quarter-integer values (half-integers for E2M1) with random scales
    2^u, u in [-2, 2]: every product and partial sum is exact in fp32."""
    w = CASES[name]
    say(f"[sf-mn-exact] {name}")
    x = wl.generate(w, seed=42, values="quarter_scaled")
    got = run_gpu(w, mn_scales(x), mn_plan(w))
    ref = reference(w, x, with_mag=False)
    assert np.array_equal(got, ref.astype(np.float32))


@pytest.mark.parametrize("ka,kb,K", [("e4m3", "e4m3", 2048), ("e4m3", "e4m3", 6144), ("e4m3", "e2m3", 4096),
                                     ("e3m2", "e3m2", 2048), ("e2m1p", "e2m1p", 4096), ("e2m1", "e2m1", 2048),
                                     ("e2m1", "e2m1", 6144), ("e4m3", "e4m3", 1152), ("e4m3", "e2m1p", 640),
                                     ("e3m2", "e3m2", 384), ("e2m1", "e2m1", 1280), ("e2m3", "e4m3", 2048),
                                     ("e3m2", "e2m1p", 1152), ("e4m3", "e2m1", 1024)])
def test_mn_scale_bytes_select_the_right_block(ka, kb, K):
    """Scales only: every element 1.0, so D[m,n] = 32 sum_j 2^(uA[m,j]+uB[n,j])
    exactly; a wrong row, K block or group of the MN-major stage changes it."""
    M, N = 272, 528
    w = wl.custom(M, N, K, ka, V=32, b_kind="" if kb == ka else kb, name="sf-mn-scale-only")
    rng = np.random.default_rng(43)
    x = {"A": wl.to_stored(np.ones((M, K)), ka), "B": wl.to_stored(np.ones((N, K)), kb),
         "SFA": (127 + rng.integers(-4, 5, (M, K // 32))).astype(np.uint8),
         "SFB": (127 + rng.integers(-4, 5, (N, K // 32))).astype(np.uint8)}
    ua = x["SFA"].astype(np.int64) - 127
    ub = x["SFB"].astype(np.int64) - 127
    expect = 32.0 * (np.exp2(ua[:, None, :] + ub[None, :, :])).sum(-1)
    say(f"[sf-mn] scale closed form {ka} x {kb} K={K}")
    ref = reference(w, x, with_mag=False)
    assert np.array_equal(ref, expect)          # the operands are the ones the closed form assumes
    got = run_gpu(w, mn_scales(x), mn_plan(w))
    assert np.array_equal(got.astype(np.float64), expect)


@pytest.mark.parametrize("name,d_dt", [("e2m3-1040x272-k2048", "bf16"), ("e3m2-256x512-k4096-beta", "f16"),
                                       ("e2m1-304x528-k4096-beta", "bf16"), ("e2m1p-304x528-k2048", "f16"),
                                       ("e4m3-1040x528-k2048", "bf16"), ("e4m3-256x512-k4096-beta", "f16"),
                                       ("e4m3-272x528-k3072-beta", "bf16"), ("e4m3-528x272-k640", "f16"),
                                       ("e4m3xe2m3-528x1040-k2048-beta", "bf16"), ("e4m3xe2m1p-304x400-k1152", "f16"),
                                       ("e2m3xe4m3-528x272-k2048", "bf16"), ("e3m2xe2m1p-304x400-k1152-beta", "f16"),
                                       ("e4m3xe2m1-304x400-k1280-beta", "bf16")])
def test_mn_scales_narrow_d_match_row_major_scales(name, d_dt):
    """bf16 / fp16 D (the fp32 result rounded once; beta reads the old D in
    D's format): the MN-major plan stores the same bits as the row-major one,
    whose parity tests/test_gpu_narrow_d.py covers."""
    w = CASES[name]
    say(f"[sf-mn-narrow] {name} {d_dt}")
    x = wl.generate(w, seed=44)
    tdt = torch.bfloat16 if d_dt == "bf16" else torch.float16
    d0 = torch.from_numpy(x["D0"]).to(tdt) if w.beta else torch.zeros((w.M, w.N), dtype=tdt)
    outs = []
    for plan, xs in ((row_major_plan(w, d_dt), x), (mn_plan(w, d_dt), mn_scales(x))):
        D = d0.clone().cuda()
        mswz.gemm_run_blockscaled(plan, to_device(xs["A"]), to_device(xs["B"]), to_device(xs["SFA"]),
                                  to_device(xs["SFB"]), D, w.beta)
        torch.cuda.synchronize()
        outs.append(D.cpu())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_mn_scales_full_size_mx_fp8():
    """MX-fp8 8192^3 with MN-major scales (the benchmark's c14, in its launch
    configuration): sampled whole rows and columns against the oracle, and
    every output bit for bit against the same inputs with row-major scales."""
    w = wl.WORKLOADS["c14"]
    assert w.sf_major == "mn"
    x = wl.generate(w, seed=0)
    plan = mn_plan(w)
    say(f"[sf-mn-full] c14 plan {plan.describe()}")
    got = run_gpu(w, mn_scales(x), plan)
    rows, cols = wl.sample_points(w, 8, 8)
    print(compare(w, got[rows], reference(w, x, rows=rows)), compare(w, got[:, cols], reference(w, x, cols=cols)))
    assert np.array_equal(got, run_gpu(w, x, row_major_plan(w)))


@pytest.mark.parametrize("name", ["e4m3-1040x528-k2048", "e4m3xe2m3-528x1040-k2048-beta", "e2m1-304x528-k4096-beta"])
def test_mn_scales_with_call_options_match_row_major_scales(name):
    """gemm_run_opts (negated A, saturated D, a row mask and a zero-column
    mask) on an MN-major-scale plan stores the same bits as on the row-major
    plan, whose options tests/test_gpu_opts.py checks against the oracle."""
    w = CASES[name]
    say(f"[sf-mn-opts] {name}")
    x = wl.generate(w, seed=45)
    rng = np.random.default_rng(46)
    row_mask = to_device(rng.integers(0, 2**31, (w.M + 31) // 32, dtype=np.int64).astype(np.int32))
    col_zero = to_device(rng.integers(0, 2**31, (w.N + 31) // 32, dtype=np.int64).astype(np.int32))
    outs = []
    for plan, xs in ((row_major_plan(w), x), (mn_plan(w), mn_scales(x))):
        D = to_device(x["D0"]) if w.beta else torch.full((w.M, w.N), 7.0, dtype=torch.float32, device="cuda")
        mswz.gemm_run_opts(plan, to_device(xs["A"]), to_device(xs["B"]), D, w.beta, SFA=to_device(xs["SFA"]),
                           SFB=to_device(xs["SFB"]), neg_a=True, sat_d=True, row_mask=row_mask, col_zero=col_zero)
        torch.cuda.synchronize()
        outs.append(D.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
