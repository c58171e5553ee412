"""GPU parity: libmswz.so (called through the C ABI) against the fp64 oracle on
the same seeded inputs.  Tolerances are documented in tests/gpu_util.py.

Small cases compare every output and span several tiles with each tile
variant, odd K-step counts and grids whose size is and is not a multiple of
eight (the XCD re-ordering path); the full-size workloads compare whole
sampled rows and columns, in the launch configuration the benchmark times.
"""
import os

import numpy as np
import pytest

import mma_swizzled_operand_amd as mswz
import workloads as wl
from gpu_util import compare, plan_for, reference, run_gpu, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture
def tile_env():
    old = os.environ.get("MSWZ_TILE")
    yield
    if old is None:
        os.environ.pop("MSWZ_TILE", None)
    else:
        os.environ["MSWZ_TILE"] = old


SMALL = {
    "c1": wl.WORKLOADS["c1"],
    "bf16-k": wl.custom(512, 768, 320, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0), name="bf16-k"),
    "f16-k": wl.custom(768, 512, 192, "f16", name="f16-k"),
    "f16-mn-beta": wl.custom(512, 512, 256, "f16", a_major="mn", beta=1, name="f16-mn-beta"),
    "bf16-mn": wl.custom(256, 768, 128, "bf16", a_major="mn", name="bf16-mn"),
    "e4m3-mx": wl.custom(512, 768, 384, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                         name="e4m3-mx"),
    "e4m3-mx-beta": wl.custom(256, 512, 256, "e4m3", V=32, beta=1, a_dist=("normal", 1.0),
                              b_dist=("normal", 1.0), name="e4m3-mx-beta"),
    "e4m3-mx-k2048": wl.custom(512, 512, 2048, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                               name="e4m3-mx-k2048"),
    "f16-bmn": wl.custom(512, 256, 192, "f16", b_major="mn", name="f16-bmn"),
    "bf16-both-mn-beta": wl.custom(256, 512, 320, "bf16", a_major="mn", b_major="mn", beta=1,
                                   a_dist=("normal", 1.0), b_dist=("normal", 1.0), name="bf16-both-mn-beta"),
    "skinny": wl.custom(64, 2048, 1024, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 0.02), name="skinny"),
    "skinny-k4096": wl.custom(64, 1024, 4096, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 0.02),
                              name="skinny-k4096"),
    "skinny-m32-beta": wl.custom(32, 1024, 2048, "f16", beta=1, name="skinny-m32-beta"),
}

# "plan": the library's own choice (no MSWZ_TILE override)
TILES = ["plan", "256", "128", "64"]


def _set_tile(w, tile):
    if tile == "plan":
        os.environ.pop("MSWZ_TILE", None)
        return
    if w.M % int(tile) or w.N % int(tile):
        pytest.skip("tile does not divide the shape")
    os.environ["MSWZ_TILE"] = tile


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("case", sorted(SMALL))
def test_small_full_compare(case, tile, tile_env):
    w = SMALL[case]
    _set_tile(w, tile)
    plan = plan_for(w)
    if tile != "plan":
        assert plan.describe()["tile_m"] == int(tile)
    say(f"[parity] {case} tile={tile} {w.M}x{w.N}x{w.K} {w.kind} A:{w.a_major} beta={w.beta}")
    x = wl.generate(w, seed=0)
    got = run_gpu(w, x, plan)
    ref = reference(w, x)
    print(case, tile, compare(w, got, ref, x.get("D0")))


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("case", sorted(SMALL))
def test_quarter_integers_bit_exact(case, tile, tile_env):
    """Quarter-integer operands (the tcgen05.mma page's example distribution)
    with unit scales: every partial sum of products is exact in fp32, so the
    GPU result must equal the oracle exactly, whatever the summation order.
    With beta = 1 the fp32 D0 is added last, so the result is the exact sum
    plus D0 rounded once to fp32."""
    w = SMALL[case]
    _set_tile(w, tile)
    say(f"[exact] {case} tile={tile}")
    x = wl.generate(w, seed=0, values="quarter")
    got = run_gpu(w, x, plan_for(w))
    ref = reference(w, x, with_mag=False)
    if not w.beta:
        assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    assert np.array_equal(got, ref.astype(np.float32))


def test_page_example_128x64x64():
    """The tcgen05.mma page's 128x64x64 fp16 example, padded to the library's
    64-column tile: B (64,64) stored (N,K), quarter-integer values from
    default_rng(0); result compared with fp32 a @ b.T (exact)."""
    rng = np.random.default_rng(0)
    a = (rng.integers(-4, 5, (128, 64)) / 4).astype("float16")
    b = (rng.integers(-4, 5, (64, 64)) / 4).astype("float16")
    w = wl.custom(128, 64, 64, "f16", name="page-example")
    say("[exact] page example 128x64x64")
    got = run_gpu(w, {"A": a.view(np.uint16), "B": b.view(np.uint16)})
    assert np.array_equal(got, a.astype("float32") @ b.astype("float32").T)


def test_beta_zero_ignores_nan_in_D():
    w = wl.custom(128, 128, 64, "bf16", name="nan-d")
    x = wl.generate(w, seed=3)
    say("[edge] beta=0 over NaN-filled D")
    got = run_gpu(w, x, D_init=np.full((w.M, w.N), np.nan, dtype=np.float32))
    ref = reference(w, x)
    compare(w, got, ref)


def test_single_k_step_single_tile():
    w = wl.custom(64, 64, 64, "f16", name="one-tile")
    x = wl.generate(w, seed=4)
    say("[edge] 64x64x64")
    got = run_gpu(w, x)
    ref = reference(w, x)
    compare(w, got, ref)


def test_deterministic_bits():
    w = wl.custom(1024, 1024, 512, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0), name="det")
    x = wl.generate(w, seed=5)
    say("[det] two runs")
    assert np.array_equal(run_gpu(w, x), run_gpu(w, x))


# M and N that are not multiples of the tile (the 256 tile with masked
# stores): both ragged, each major combination, MX, degenerate outputs
TAILS = {
    "tail-bf16-k": wl.custom(1000, 520, 128, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                             name="tail-bf16-k"),
    "tail-f16-amn-beta": wl.custom(200, 264, 192, "f16", a_major="mn", beta=1, name="tail-f16-amn-beta"),
    "tail-bf16-bmn": wl.custom(136, 776, 64, "bf16", b_major="mn", name="tail-bf16-bmn"),
    "tail-f16-both-mn": wl.custom(264, 520, 128, "f16", a_major="mn", b_major="mn", name="tail-f16-both-mn"),
    "tail-e4m3-mx": wl.custom(300, 292, 256, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                              name="tail-e4m3-mx"),
    "tail-e4m3-mx-k1024-beta": wl.custom(264, 520, 1024, "e4m3", V=32, beta=1, a_dist=("normal", 1.0),
                                         b_dist=("normal", 1.0), name="tail-e4m3-mx-k1024-beta"),
    # K a multiple of 2048: E4M3 with 32-byte scale groups of eight steps
    # (two and three sixteen-step iterations), and K = 3072 (16-byte groups)
    "tail-e4m3-mx-k4096-beta": wl.custom(300, 292, 4096, "e4m3", V=32, beta=1, a_dist=("normal", 1.0),
                                         b_dist=("normal", 1.0), name="tail-e4m3-mx-k4096-beta"),
    "tail-e4m3-mx-k6144": wl.custom(264, 256, 6144, "e4m3", V=32, a_dist=("normal", 1.0),
                                    b_dist=("normal", 1.0), name="tail-e4m3-mx-k6144"),
    "tail-e4m3-mx-k3072": wl.custom(256, 264, 3072, "e4m3", V=32, a_dist=("normal", 1.0),
                                    b_dist=("normal", 1.0), name="tail-e4m3-mx-k3072"),
    "tail-one-row": wl.custom(1, 4, 64, "bf16", name="tail-one-row"),
    "tail-257": wl.custom(257, 256, 64, "f16", beta=1, name="tail-257"),
}


@pytest.mark.parametrize("name", list(TAILS))
def test_tail_shapes_full_compare(name):
    w = TAILS[name]
    plan = plan_for(w)
    say(f"[tail] {name} {w.M}x{w.N}x{w.K} {w.kind} A:{w.a_major} B:{w.b_major} beta={w.beta} {plan.describe()}")
    x = wl.generate(w, seed=21)
    got = run_gpu(w, x, plan)
    ref = reference(w, x)
    print(name, compare(w, got, ref, x.get("D0")))


def test_tail_output_untouched_outside_d():
    """Stores stay inside D: a canary buffer around D is unchanged."""
    w = TAILS["tail-bf16-k"]
    plan = plan_for(w)
    x = wl.generate(w, seed=22)
    import torch
    A, B = (torch.from_numpy(np.ascontiguousarray(x[k]).view(np.int16)).cuda() for k in ("A", "B"))
    n = w.M * w.N
    buf = torch.full((n + 2 * 4096,), 7.0, dtype=torch.float32, device="cuda")
    D = buf[4096:4096 + n]
    say("[tail] canary")
    mswz.gemm_run(plan, A, B, D, 0)
    torch.cuda.synchronize()
    assert torch.all(buf[:4096] == 7.0) and torch.all(buf[4096 + n:] == 7.0)


# K not a multiple of the 64-element step (16-bit; the 256 tile, whose last
# step reads the values beyond K as zeros): each major combination, K below
# one step, K % 8 != 0 with both operands MN-major, ragged M and N, beta = 1,
# narrow D, and shapes that would otherwise take another kernel
KTAILS = {
    "ktail-bf16-k": wl.custom(512, 256, 72, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                              name="ktail-bf16-k"),
    "ktail-f16-amn-beta": wl.custom(264, 300, 200, "f16", a_major="mn", beta=1, name="ktail-f16-amn-beta"),
    "ktail-bf16-bmn": wl.custom(256, 512, 40, "bf16", b_major="mn", name="ktail-bf16-bmn"),
    "ktail-f16-both-mn-k100": wl.custom(256, 320, 100, "f16", a_major="mn", b_major="mn", beta=1,
                                        name="ktail-f16-both-mn-k100"),
    "ktail-bf16-both-mn-k1": wl.custom(256, 256, 1, "bf16", a_major="mn", b_major="mn",
                                       name="ktail-bf16-both-mn-k1"),
    "ktail-f16-k8": wl.custom(128, 256, 8, "f16", name="ktail-f16-k8"),
    "ktail-skinny-shape": wl.custom(64, 1024, 1032, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 0.02),
                                    name="ktail-skinny-shape"),
    "ktail-bf16-k-odd-steps": wl.custom(512, 512, 3 * 64 + 24, "bf16", beta=1, name="ktail-bf16-k-odd-steps"),
}


@pytest.mark.parametrize("name", list(KTAILS))
def test_k_tail_full_compare(name):
    w = KTAILS[name]
    plan = plan_for(w)
    assert plan.describe()["tile_m"] == 256
    say(f"[k-tail] {name} {w.M}x{w.N}x{w.K} {w.kind} A:{w.a_major} B:{w.b_major} beta={w.beta}")
    x = wl.generate(w, seed=31)
    got = run_gpu(w, x, plan)
    ref = reference(w, x)
    print(name, compare(w, got, ref, x.get("D0")))


@pytest.mark.parametrize("name", list(KTAILS))
def test_k_tail_quarter_integers_bit_exact(name):
    w = KTAILS[name]
    say(f"[k-tail exact] {name}")
    x = wl.generate(w, seed=32, values="quarter")
    got = run_gpu(w, x, plan_for(w))
    ref = reference(w, x, with_mag=False)
    assert np.array_equal(got, ref.astype(np.float32))


def test_k_tail_full_size_sampled():
    """4096 x 4096 x 4040 bf16 (63 full steps and a 8-element tail), both
    K-major, on sampled rows and columns."""
    w = wl.custom(4096, 4096, 4040, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0), name="ktail-4096")
    say("[k-tail full] 4096x4096x4040 bf16")
    x = wl.generate(w, seed=33)
    got = run_gpu(w, x)
    rows, cols = wl.sample_points(w, 12, 12, seed=34)
    ref = reference(w, x, rows=rows, cols=cols)
    print(compare(w, got[np.ix_(rows, cols)], ref))


# MX-fp4 (OCP E2M1, two per byte; the 256 tile only): several tiles and K
# steps, ragged M and N, beta = 1
FP4 = {
    "e2m1-mx": wl.custom(512, 768, 512, "e2m1", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                         name="e2m1-mx"),
    "e2m1-mx-beta-k1280": wl.custom(256, 512, 1280, "e2m1", V=32, beta=1, a_dist=("normal", 1.0),
                                    b_dist=("normal", 1.0), name="e2m1-mx-beta-k1280"),
    "e2m1-mx-tail": wl.custom(300, 292, 768, "e2m1", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                              name="e2m1-mx-tail"),
    # K a multiple of 1024: scale bytes copied per group of two steps
    "e2m1-mx-k2048": wl.custom(512, 512, 2048, "e2m1", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                               name="e2m1-mx-k2048"),
    "e2m1-mx-tail-k1024-beta": wl.custom(300, 292, 1024, "e2m1", V=32, beta=1, a_dist=("normal", 1.0),
                                         b_dist=("normal", 1.0), name="e2m1-mx-tail-k1024-beta"),
    # K a multiple of 2048: 32-byte scale groups of four steps (one and three
    # loop iterations)
    "e2m1-mx-tail-k4096-beta": wl.custom(300, 292, 4096, "e2m1", V=32, beta=1, a_dist=("normal", 1.0),
                                         b_dist=("normal", 1.0), name="e2m1-mx-tail-k4096-beta"),
    "e2m1-mx-k6144": wl.custom(256, 512, 6144, "e2m1", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                               name="e2m1-mx-k6144"),
}


@pytest.mark.parametrize("name", list(FP4))
def test_fp4_full_compare(name):
    w = FP4[name]
    plan = plan_for(w)
    say(f"[fp4] {name} {w.M}x{w.N}x{w.K} beta={w.beta} {plan.describe()}")
    x = wl.generate(w, seed=31)
    got = run_gpu(w, x, plan)
    ref = reference(w, x)
    print(name, compare(w, got, ref, x.get("D0")))


@pytest.mark.parametrize("name", list(FP4))
def test_fp4_half_integers_bit_exact(name):
    """E2M1 half-integer operands in [-1, 1] with unit scales: every product
    and partial sum is exact in fp32, so the result equals the oracle exactly."""
    w = FP4[name]
    say(f"[fp4-exact] {name}")
    x = wl.generate(w, seed=32, values="quarter")
    got = run_gpu(w, x, plan_for(w))
    ref = reference(w, x, with_mag=False)
    assert np.array_equal(got, ref.astype(np.float32))


@pytest.mark.parametrize("K", [1024, 4096])
def test_fp4_scale_bytes_select_the_right_block(K):
    """Scales only: every E2M1 element 1.0 (byte 0x22), so D[m,n] =
    32 sum_j 2^(uA[m,j]+uB[n,j]) exactly; a wrong scale byte, lane or word
    for any of the eight blocks of a K step changes the value (K = 4096: the
    32-byte scale groups)."""
    M, N = 256, 512
    w = wl.custom(M, N, K, "e2m1", V=32, name="fp4-scale-only")
    rng = np.random.default_rng(7)
    x = {"A": np.full((M, K // 2), 0x22, np.uint8), "B": np.full((N, K // 2), 0x22, np.uint8),
         "SFA": (127 + rng.integers(-4, 5, (M, K // 32))).astype(np.uint8),
         "SFB": (127 + rng.integers(-4, 5, (N, K // 32))).astype(np.uint8)}
    say(f"[fp4] scale closed form K={K}")
    got = run_gpu(w, x)
    ua = x["SFA"].astype(np.int64) - 127
    ub = x["SFB"].astype(np.int64) - 127
    expect = 32.0 * (np.exp2(ua[:, None, :] + ub[None, :, :])).sum(-1)
    assert np.array_equal(got.astype(np.float64), expect)


# MX-fp6 (OCP E2M3 / E3M2, sixteen per 16-byte block with four bytes of
# padding; the 256 tile only): per-step and grouped scale copies (K a multiple
# of 1024), ragged M and N, beta = 1
FP6 = {
    "e2m3-mx": wl.custom(512, 768, 512, "e2m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                         name="e2m3-mx"),
    "e3m2-mx-k1024-beta": wl.custom(256, 512, 1024, "e3m2", V=32, beta=1, a_dist=("normal", 1.0),
                                    b_dist=("normal", 1.0), name="e3m2-mx-k1024-beta"),
    "e2m3-mx-tail": wl.custom(300, 292, 384, "e2m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                              name="e2m3-mx-tail"),
    "e3m2-mx-k2048": wl.custom(512, 512, 2048, "e3m2", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                               name="e3m2-mx-k2048"),
    # 32-byte scale groups of eight steps (K a multiple of 2048), padded E2M1
    # alone as well
    "e2m3-mx-tail-k4096-beta": wl.custom(300, 292, 4096, "e2m3", V=32, beta=1, a_dist=("normal", 1.0),
                                         b_dist=("normal", 1.0), name="e2m3-mx-tail-k4096-beta"),
    "e3m2-mx-k6144": wl.custom(256, 256, 6144, "e3m2", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                               name="e3m2-mx-k6144"),
    "e2m1p-k4096-tail-beta": wl.custom(300, 292, 4096, "e2m1p", V=32, beta=1, a_dist=("normal", 1.0),
                                       b_dist=("normal", 1.0), name="e2m1p-k4096-tail-beta"),
}


@pytest.mark.parametrize("name", list(FP6))
def test_fp6_full_compare(name):
    w = FP6[name]
    plan = plan_for(w)
    say(f"[fp6] {name} {w.M}x{w.N}x{w.K} beta={w.beta} {plan.describe()}")
    x = wl.generate(w, seed=41)
    got = run_gpu(w, x, plan)
    ref = reference(w, x)
    print(name, compare(w, got, ref, x.get("D0")))


@pytest.mark.parametrize("name", list(FP6))
def test_fp6_quarter_integers_bit_exact(name):
    w = FP6[name]
    say(f"[fp6-exact] {name}")
    x = wl.generate(w, seed=42, values="quarter")
    got = run_gpu(w, x, plan_for(w))
    ref = reference(w, x, with_mag=False)
    assert np.array_equal(got, ref.astype(np.float32))


@pytest.mark.parametrize("name", ["e2m3-mx", "e3m2-mx-k1024-beta", "e2m1p", "e4m3xe2m1p"])
def test_padding_bytes_are_never_read(name):
    """Random bytes in every block's padding (the last four bytes of a 6-bit
    block, the last eight of a padded 4-bit one) give the same bits."""
    w = FP6[name] if name in FP6 else MIXED[name]
    say(f"[pad] {name}")
    x = wl.generate(w, seed=43)
    base = run_gpu(w, x)
    rng = np.random.default_rng(44)
    y = dict(x)
    for k, kind in (("A", w.kind), ("B", w.kind_b)):
        first = {"e2m3": 12, "e3m2": 12, "e2m1p": 8}.get(kind)
        if first is None:
            continue
        a = x[k].copy().reshape(-1, 16)
        a[:, first:] = rng.integers(0, 256, (a.shape[0], 16 - first), dtype=np.uint8)
        y[k] = a.reshape(x[k].shape)
    assert np.array_equal(run_gpu(w, y), base)


@pytest.mark.parametrize("K", [1024, 4096])
@pytest.mark.parametrize("kind,one", [("e2m3", 8), ("e3m2", 12)])
def test_fp6_scale_bytes_select_the_right_block(kind, one, K):
    """Scales only: every element 1.0, so D[m,n] = 32 sum_j 2^(uA[m,j]+uB[n,j])
    exactly; a wrong scale byte or lane for any block changes the value (K =
    4096: the 32-byte scale groups)."""
    M, N = 256, 512
    w = wl.custom(M, N, K, kind, V=32, name=f"{kind}-scale-only")
    rng = np.random.default_rng(9)
    ones = wl.to_stored(np.ones((1, 16)), kind)[0]
    assert ones[0] == one
    x = {"A": np.tile(ones, (M, K // 16)), "B": np.tile(ones, (N, K // 16)),
         "SFA": (127 + rng.integers(-4, 5, (M, K // 32))).astype(np.uint8),
         "SFB": (127 + rng.integers(-4, 5, (N, K // 32))).astype(np.uint8)}
    say(f"[fp6] scale closed form {kind} K={K}")
    got = run_gpu(w, x)
    ua = x["SFA"].astype(np.int64) - 127
    ub = x["SFB"].astype(np.int64) - 127
    expect = 32.0 * (np.exp2(ua[:, None, :] + ub[None, :, :])).sum(-1)
    assert np.array_equal(got.astype(np.float64), expect)


# mixed block-scaled kinds (E4M3, E2M3, E3M2 for A and B independently): each
# E4M3 / 6-bit pairing in both orders and the two 6-bit formats together,
# grouped and per-step scale copies, ragged M and N, beta = 1
MIXED = {
    "e4m3xe2m3": wl.custom(512, 768, 1024, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                           name="e4m3xe2m3", b_kind="e2m3"),
    "e2m3xe4m3-beta": wl.custom(256, 512, 512, "e2m3", V=32, beta=1, a_dist=("normal", 1.0),
                                b_dist=("normal", 1.0), name="e2m3xe4m3-beta", b_kind="e4m3"),
    "e4m3xe3m2-tail": wl.custom(300, 292, 384, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                name="e4m3xe3m2-tail", b_kind="e3m2"),
    "e3m2xe4m3-k2048": wl.custom(512, 256, 2048, "e3m2", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                 name="e3m2xe4m3-k2048", b_kind="e4m3"),
    "e2m3xe3m2": wl.custom(256, 256, 1024, "e2m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                           name="e2m3xe3m2", b_kind="e3m2"),
    "e3m2xe2m3-beta": wl.custom(264, 256, 640, "e3m2", V=32, beta=1, a_dist=("normal", 1.0),
                                b_dist=("normal", 1.0), name="e3m2xe2m3-beta", b_kind="e2m3"),
    # E2M1 in the pages' padded form, alone and mixed
    "e2m1p": wl.custom(512, 512, 1024, "e2m1p", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                       name="e2m1p"),
    "e2m1p-tail-beta": wl.custom(300, 292, 384, "e2m1p", V=32, beta=1, a_dist=("normal", 1.0),
                                 b_dist=("normal", 1.0), name="e2m1p-tail-beta"),
    "e4m3xe2m1p": wl.custom(512, 768, 1024, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                            name="e4m3xe2m1p", b_kind="e2m1p"),
    "e2m1pxe4m3-beta": wl.custom(256, 512, 512, "e2m1p", V=32, beta=1, a_dist=("normal", 1.0),
                                 b_dist=("normal", 1.0), name="e2m1pxe4m3-beta", b_kind="e4m3"),
    "e2m1pxe2m3": wl.custom(256, 256, 640, "e2m1p", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                            name="e2m1pxe2m3", b_kind="e2m3"),
    # E4M3 with dense E2M1 (K a multiple of 256), either side
    "e4m3xe2m1": wl.custom(512, 768, 1024, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                           name="e4m3xe2m1", b_kind="e2m1"),
    "e4m3xe2m1-k2560-tail": wl.custom(264, 300, 2560, "e4m3", V=32, a_dist=("normal", 1.0),
                                      b_dist=("normal", 1.0), name="e4m3xe2m1-k2560-tail", b_kind="e2m1"),
    "e2m1xe4m3-beta": wl.custom(512, 256, 512, "e2m1", V=32, beta=1, a_dist=("normal", 1.0),
                                b_dist=("normal", 1.0), name="e2m1xe4m3-beta", b_kind="e4m3"),
    "e2m1xe4m3-tail": wl.custom(300, 292, 1536, "e2m1", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                name="e2m1xe4m3-tail", b_kind="e4m3"),
    # K a multiple of 1024 with E2M1 as A: scale words copied per group of four steps
    "e2m1xe4m3-k2048-tail-beta": wl.custom(300, 292, 2048, "e2m1", V=32, beta=1, a_dist=("normal", 1.0),
                                           b_dist=("normal", 1.0), name="e2m1xe4m3-k2048-tail-beta", b_kind="e4m3"),
    # step counts 2 and 6: the pair of steps after the four-step loop
    "e4m3xe2m1-k256-beta": wl.custom(256, 512, 256, "e4m3", V=32, beta=1, a_dist=("normal", 1.0),
                                     b_dist=("normal", 1.0), name="e4m3xe2m1-k256-beta", b_kind="e2m1"),
    "e2m1xe4m3-k768": wl.custom(512, 264, 768, "e2m1", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                name="e2m1xe4m3-k768", b_kind="e4m3"),
    # E4M3 A with K a multiple of 2048: 32-byte scale groups of eight steps
    "e4m3xe2m3-k4096-tail-beta": wl.custom(300, 292, 4096, "e4m3", V=32, beta=1, a_dist=("normal", 1.0),
                                           b_dist=("normal", 1.0), name="e4m3xe2m3-k4096-tail-beta",
                                           b_kind="e2m3"),
    "e4m3xe2m1p-k2048": wl.custom(512, 256, 2048, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                  name="e4m3xe2m1p-k2048", b_kind="e2m1p"),
    "e4m3xe3m2-k6144": wl.custom(256, 264, 6144, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                 name="e4m3xe3m2-k6144", b_kind="e3m2"),
}


@pytest.mark.parametrize("name", list(MIXED))
def test_mixed_full_compare(name):
    w = MIXED[name]
    plan = plan_for(w)
    assert plan.describe()["tile_m"] == 256
    say(f"[mixed] {name} {w.M}x{w.N}x{w.K} {w.kind} x {w.kind_b} beta={w.beta}")
    x = wl.generate(w, seed=51)
    got = run_gpu(w, x, plan)
    ref = reference(w, x)
    print(name, compare(w, got, ref, x.get("D0")))


@pytest.mark.parametrize("name", list(MIXED))
def test_mixed_quarter_integers_bit_exact(name):
    w = MIXED[name]
    say(f"[mixed-exact] {name}")
    x = wl.generate(w, seed=52, values="quarter")
    got = run_gpu(w, x, plan_for(w))
    assert np.array_equal(got, reference(w, x, with_mag=False).astype(np.float32))


@pytest.mark.parametrize("ka,kb,K", [("e4m3", "e2m3", 1024), ("e3m2", "e4m3", 1024), ("e2m1p", "e2m1p", 1024),
                                     ("e2m1p", "e4m3", 1024), ("e4m3", "e2m1", 1024), ("e2m1", "e4m3", 1024),
                                     ("e4m3", "e2m3", 4096), ("e4m3", "e2m1p", 4096), ("e4m3", "e4m3", 4096)])
def test_mixed_scale_bytes_select_the_right_block(ka, kb, K):
    """Scales only, every element 1.0 in its own format: D[m,n] =
    32 sum_j 2^(uA[m,j]+uB[n,j]) exactly; a value meeting a partner from
    another K block, or a wrong scale byte, changes the value (K = 4096: the
    32-byte scale groups of an E4M3 A)."""
    M, N = 256, 512
    w = wl.custom(M, N, K, ka, V=32, name=f"{ka}x{kb}-scale-only", b_kind=kb)
    rng = np.random.default_rng(10)
    x = {"A": wl.to_stored(np.ones((M, K)), ka), "B": wl.to_stored(np.ones((N, K)), kb),
         "SFA": (127 + rng.integers(-4, 5, (M, K // 32))).astype(np.uint8),
         "SFB": (127 + rng.integers(-4, 5, (N, K // 32))).astype(np.uint8)}
    say(f"[mixed] scale closed form {ka} x {kb} K={K}")
    got = run_gpu(w, x)
    ua = x["SFA"].astype(np.int64) - 127
    ub = x["SFB"].astype(np.int64) - 127
    expect = 32.0 * (np.exp2(ua[:, None, :] + ub[None, :, :])).sum(-1)
    assert np.array_equal(got.astype(np.float64), expect)


@pytest.mark.parametrize("ka,kb", [("e4m3", "e2m3"), ("e4m3", "e2m1p"), ("e4m3", "e2m1"), ("e2m1", "e4m3")])
def test_mixed_k_positions_meet(ka, kb):
    """A one-hot in K per row of A against random B rows: D[m,n] = B[n] at
    A's hot position, so any K-order mismatch between the E4M3 fragments and
    the 6- or 4-bit ones shows (hot positions cover every k of a 256-element
    span, in random spans)."""
    M, N, K = 512, 256, 1024
    w = wl.custom(M, N, K, ka, V=32, name="mixed-one-hot", b_kind=kb)
    rng = np.random.default_rng(11)
    hot = np.arange(M) % 256 + 256 * rng.integers(0, K // 256, M)
    a = np.zeros((M, K))
    a[np.arange(M), hot] = 1.0
    b = rng.integers(-3, 4, (N, K)) / 2.0          # half-integers in [-1.5, 1.5]: exact in every kind here
    x = {"A": wl.to_stored(a, ka), "B": wl.to_stored(b, kb),
         "SFA": np.full((M, K // 32), 127, np.uint8), "SFB": np.full((N, K // 32), 127, np.uint8)}
    assert len(set(hot % 256)) == 256
    say(f"[mixed] one-hot K positions {ka} x {kb}")
    got = run_gpu(w, x)
    assert np.array_equal(got.astype(np.float64), b[:, hot].T)


# 16-element scale blocks (scale_vec_len 16: the pages' scale_vec::4X) for
# E2M1 (dense and padded) and the 6-bit kinds
V16 = {
    "e2m1-v16": wl.custom(512, 512, 1024, "e2m1", V=16, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                          name="e2m1-v16"),
    "e2m1-v16-tail-beta": wl.custom(300, 292, 768, "e2m1", V=16, beta=1, a_dist=("normal", 1.0),
                                    b_dist=("normal", 1.0), name="e2m1-v16-tail-beta"),
    "e2m1p-v16": wl.custom(512, 256, 1024, "e2m1p", V=16, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                           name="e2m1p-v16"),
    "e2m3-v16-beta": wl.custom(256, 512, 512, "e2m3", V=16, beta=1, a_dist=("normal", 1.0),
                               b_dist=("normal", 1.0), name="e2m3-v16-beta"),
    "e3m2-v16-tail": wl.custom(264, 300, 384, "e3m2", V=16, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                               name="e3m2-v16-tail"),
}


@pytest.mark.parametrize("name", list(V16))
def test_v16_full_compare(name):
    w = V16[name]
    plan = plan_for(w)
    say(f"[v16] {name} {w.M}x{w.N}x{w.K} {w.kind} beta={w.beta}")
    x = wl.generate(w, seed=61)
    got = run_gpu(w, x, plan)
    ref = reference(w, x)
    print(name, compare(w, got, ref, x.get("D0")))


@pytest.mark.parametrize("name", list(V16))
def test_v16_quarter_integers_bit_exact(name):
    w = V16[name]
    say(f"[v16-exact] {name}")
    x = wl.generate(w, seed=62, values="quarter")
    got = run_gpu(w, x, plan_for(w))
    assert np.array_equal(got, reference(w, x, with_mag=False).astype(np.float32))


@pytest.mark.parametrize("kind", ["e2m1", "e2m1p", "e3m2"])
def test_v16_scale_bytes_select_the_right_block(kind):
    """Scales only: every element 1.0, D[m,n] = 16 sum_q 2^(uA[m,q]+uB[n,q])
    exactly; a wrong scale byte, word or half for any 16-block changes it."""
    M, N, K = 256, 512, 1024
    w = wl.custom(M, N, K, kind, V=16, name=f"{kind}-v16-scale-only")
    rng = np.random.default_rng(12)
    x = {"A": wl.to_stored(np.ones((M, K)), kind), "B": wl.to_stored(np.ones((N, K)), kind),
         "SFA": (127 + rng.integers(-4, 5, (M, K // 16))).astype(np.uint8),
         "SFB": (127 + rng.integers(-4, 5, (N, K // 16))).astype(np.uint8)}
    say(f"[v16] scale closed form {kind}")
    got = run_gpu(w, x)
    ua = x["SFA"].astype(np.int64) - 127
    ub = x["SFB"].astype(np.int64) - 127
    expect = 16.0 * (np.exp2(ua[:, None, :] + ub[None, :, :])).sum(-1)
    assert np.array_equal(got.astype(np.float64), expect)


def test_v16_full_size_sampled():
    """4096^3 E2M1 with 16-element blocks, sampled rows and columns."""
    w = wl.custom(4096, 4096, 4096, "e2m1", V=16, a_dist=("normal", 1.0), b_dist=("normal", 1.0), name="e2m1-v16-4096")
    say("[v16 full] 4096^3 e2m1")
    x = wl.generate(w, seed=63)
    got = run_gpu(w, x)
    rows, cols = wl.sample_points(w, 8, 8, seed=64)
    ref_r = reference(w, x, rows=rows)
    print(compare(w, got[rows], ref_r))


# long K: large per-step offsets, long fp32 accumulation chains
LONGK = {
    "bf16-k65536": wl.custom(256, 512, 65536, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                             name="bf16-k65536"),
    "f16-amn-k16384-beta": wl.custom(256, 256, 16384, "f16", a_major="mn", beta=1, name="f16-amn-k16384-beta"),
    "e4m3-k32768": wl.custom(256, 256, 32768, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                             name="e4m3-k32768"),
}


@pytest.mark.parametrize("name", list(LONGK))
def test_long_k(name):
    w = LONGK[name]
    say(f"[long-k] {name} {w.M}x{w.N}x{w.K}")
    x = wl.generate(w, seed=71)
    got = run_gpu(w, x)
    ref = reference(w, x)
    print(name, compare(w, got, ref, x.get("D0")))
    xq = wl.generate(w, seed=72, values="quarter")
    assert np.array_equal(run_gpu(w, xq), reference(w, xq, with_mag=False).astype(np.float32))


# the remaining dense operand layouts at full size (fp16 K-major, bf16 with
# MN-major A, MN-major B alone, both MN-major with beta)
EXTRA_FULL = {
    "bmn-4096": wl.custom(4096, 4096, 4096, "bf16", a_major="mn", b_major="mn",
                          a_dist=("normal", 1.0), b_dist=("normal", 1.0), name="bmn-4096"),
    "f16-k-8192": wl.custom(8192, 8192, 8192, "f16", name="f16-k-8192"),
    "bf16-amn-8192": wl.custom(8192, 8192, 8192, "bf16", a_major="mn",
                               a_dist=("normal", 1.0), b_dist=("normal", 1.0), name="bf16-amn-8192"),
    "f16-bmn-4096": wl.custom(4096, 4096, 4096, "f16", b_major="mn", name="f16-bmn-4096"),
    "bf16-both-mn-beta-4096": wl.custom(4096, 4096, 4096, "bf16", a_major="mn", b_major="mn", beta=1,
                                        name="bf16-both-mn-beta-4096"),
    "tail-4000x4004": wl.custom(4000, 4004, 512, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                name="tail-4000x4004"),
}


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "c6", "c7", "c8", "c9", "c10", "c3b", "c11", "c12", "c13",
                                  *EXTRA_FULL])
def test_full_size_sampled(name):
    """Full-size workloads in the benchmark's launch configuration; whole
    sampled rows and columns are compared with the oracle."""
    w = wl.WORKLOADS[name] if name in wl.WORKLOADS else EXTRA_FULL[name]
    say(f"[full] {name}: {w.title}")
    x = wl.generate(w, seed=0)
    plan = plan_for(w)
    say(f"[full] {name} plan {plan.describe()}")
    got = run_gpu(w, x, plan)
    rows, cols = wl.sample_points(w, 8, 8)
    ref_r = reference(w, x, rows=rows)
    ref_c = reference(w, x, cols=cols)
    d0 = x.get("D0")
    r1 = compare(w, got[rows], ref_r, None if d0 is None else d0[rows])
    r2 = compare(w, got[:, cols], ref_c, None if d0 is None else d0[:, cols])
    print(name, r1, r2)


def test_full_size_c5_quarter_exact():
    """MX-fp8 8192^3 with quarter-integer operands and unit scales: exact."""
    w = wl.WORKLOADS["c5"]
    x = wl.generate(w, seed=0, values="quarter")
    say("[full-exact] c5 quarter")
    got = run_gpu(w, x)
    rows, cols = wl.sample_points(w, 4, 4)
    assert np.array_equal(got[rows].astype(np.float64), reference(w, x, rows=rows, with_mag=False))
    assert np.array_equal(got[:, cols].astype(np.float64), reference(w, x, cols=cols, with_mag=False))


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (512, 256, 2048), (300, 260, 1024), (264, 300, 4096)])
def test_scale_bytes_select_the_right_block(M, N, K):
    """Scales only: a = b = 1 everywhere, so D[m,n] = 32 sum_j 2^(uA[m,j]+uB[n,j])
    exactly (block-scale closed form); a wrong byte or lane for any scale
    block changes the value.  K = 512 copies scales per K step; K a multiple
    of 1024 copies them per group of four steps (ragged M, N too), a multiple
    of 2048 per group of eight (32 bytes per row)."""
    w = wl.custom(M, N, K, "e4m3", V=32, name="scale-only")
    rng = np.random.default_rng(6)
    x = {"A": np.full((M, K), 0x38, np.uint8), "B": np.full((N, K), 0x38, np.uint8),
         "SFA": (127 + rng.integers(-4, 5, (M, K // 32))).astype(np.uint8),
         "SFB": (127 + rng.integers(-4, 5, (N, K // 32))).astype(np.uint8)}
    say("[scale] closed form")
    got = run_gpu(w, x)
    ua = x["SFA"].astype(np.int64) - 127
    ub = x["SFB"].astype(np.int64) - 127
    expect = 32.0 * (np.exp2(ua[:, None, :] + ub[None, :, :])).sum(-1)
    assert np.array_equal(got.astype(np.float64), expect)


def _block_scaled_cases():
    out = {}
    for group in (SMALL, TAILS, FP4, FP6, MIXED, V16):
        for name, w in group.items():
            if w.V and w.K <= 4096:
                out[name] = w
    return out


MX_RANDOM_SCALES = _block_scaled_cases()


@pytest.mark.parametrize("name", sorted(MX_RANDOM_SCALES))
def test_mx_random_scales_bit_exact(name):
    """Quarter-integer values (half-integers for E2M1) with random scale bytes
    127 + u, u in [-2, 2], for both operands: every scaled product and partial
    sum is exact in fp32 (K <= 4096), so the result must equal the oracle bit
    for bit, element by element.  A value meeting the wrong scale byte, or a
    scale byte applied to the wrong block or row, changes the output."""
    w = MX_RANDOM_SCALES[name]
    say(f"[mx-exact-scaled] {name} {w.M}x{w.N}x{w.K} {w.kind} x {w.kind_b} V={w.V} beta={w.beta}")
    x = wl.generate(w, seed=81, values="quarter_scaled")
    assert len(np.unique(x["SFA"])) == 5 and len(np.unique(x["SFB"])) == 5
    got = run_gpu(w, x, plan_for(w))
    ref = reference(w, x, with_mag=False)
    assert np.array_equal(got, ref.astype(np.float32))


# Block-scaled K that is not a multiple of the kernel's K step (128 elements,
# E2M1 256): the last step is zero-padded and the scale words are assembled
# in registers (a row's K/V scale bytes are not whole 4-byte words)
MXKTAILS = {
    "e4m3-k160": wl.custom(512, 256, 160, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                           name="e4m3-k160"),
    "e4m3-k96-tail-beta": wl.custom(300, 292, 96, "e4m3", V=32, beta=1, a_dist=("normal", 1.0),
                                    b_dist=("normal", 1.0), name="e4m3-k96-tail-beta"),
    "e4m3-k4000": wl.custom(256, 256, 4000, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                            name="e4m3-k4000"),
    "e2m1-k288": wl.custom(256, 512, 288, "e2m1", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                           name="e2m1-k288"),
    "e2m1-v16-k96-beta": wl.custom(264, 256, 96, "e2m1", V=16, beta=1, a_dist=("normal", 1.0),
                                   b_dist=("normal", 1.0), name="e2m1-v16-k96-beta"),
    "e2m3-v16-k176": wl.custom(256, 256, 176, "e2m3", V=16, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                               name="e2m3-v16-k176"),
    "e3m2-k224-beta": wl.custom(256, 264, 224, "e3m2", V=32, beta=1, a_dist=("normal", 1.0),
                                b_dist=("normal", 1.0), name="e3m2-k224-beta"),
    "e2m1p-v16-k80": wl.custom(256, 256, 80, "e2m1p", V=16, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                               name="e2m1p-v16-k80"),
    "e4m3xe2m3-k160": wl.custom(512, 256, 160, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                name="e4m3xe2m3-k160", b_kind="e2m3"),
    "e4m3xe2m1p-k352-beta": wl.custom(256, 512, 352, "e4m3", V=32, beta=1, a_dist=("normal", 1.0),
                                      b_dist=("normal", 1.0), name="e4m3xe2m1p-k352-beta", b_kind="e2m1p"),
}


@pytest.mark.parametrize("name", list(MXKTAILS))
def test_mx_k_tail_full_compare(name):
    w = MXKTAILS[name]
    plan = plan_for(w)
    assert plan.describe()["tile_m"] == 256
    say(f"[mx-k-tail] {name} {w.M}x{w.N}x{w.K} {w.kind} x {w.kind_b} V={w.V} beta={w.beta}")
    x = wl.generate(w, seed=91)
    got = run_gpu(w, x, plan)
    ref = reference(w, x)
    print(name, compare(w, got, ref, x.get("D0")))


@pytest.mark.parametrize("name", list(MXKTAILS))
def test_mx_k_tail_random_scales_bit_exact(name):
    w = MXKTAILS[name]
    say(f"[mx-k-tail exact] {name}")
    x = wl.generate(w, seed=92, values="quarter_scaled")
    got = run_gpu(w, x, plan_for(w))
    assert np.array_equal(got, reference(w, x, with_mag=False).astype(np.float32))


@pytest.mark.parametrize("name", ["e4m3-k160", "e2m1-v16-k96-beta", "e3m2-k224-beta"])
def test_mx_k_tail_reads_no_scale_byte_beyond_the_array(name):
    """SFA and SFB are views at the very end of larger buffers whose following
    bytes are 255 (the NaN code): the result is still finite and exact for
    quarter-integer values, so no scale byte past the last row's K/V was
    used (blocks beyond K take 2^0 without a read)."""
    import torch
    w = MXKTAILS[name]
    x = wl.generate(w, seed=93, values="quarter_scaled")
    plan = plan_for(w)
    A, B = to_device(x["A"]), to_device(x["B"])

    def at_end(sf):
        """The scale bytes followed by 256 bytes of 255 in one allocation."""
        n = sf.size
        buf = torch.full((n + 256,), 255, dtype=torch.uint8, device="cuda")
        view = buf[:n]
        view.copy_(torch.from_numpy(np.ascontiguousarray(sf).reshape(-1)).cuda())
        return view

    SFA, SFB = at_end(x["SFA"]), at_end(x["SFB"])
    D = to_device(x["D0"]) if w.beta else torch.zeros((w.M, w.N), dtype=torch.float32, device="cuda")
    say(f"[mx-k-tail nan-guard] {name}")
    mswz.gemm_run_blockscaled(plan, A, B, SFA, SFB, D, w.beta)
    torch.cuda.synchronize()
    got = D.cpu().numpy()
    assert np.isfinite(got).all()
    assert np.array_equal(got, reference(w, x, with_mag=False).astype(np.float32))
