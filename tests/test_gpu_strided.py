"""Row pitches (gemm_plan_create_ld): A, B and D as views into wider row-major
storage, through the C ABI, against the oracle.

The storage around each view is filled with values that would poison any
result they entered (infinities for 16-bit operands, NaN for E4M3, the
largest E2M1 magnitude) and, for D, with a sentinel whose bits must survive
the call.  Tolerances are those of tests/gpu_util.py; quarter-integer cases
are exact.  Where the packed plan also takes the 256 tile, the strided
result must also equal the packed one bit for bit (same kernel, same
summation order).
"""
import numpy as np
import pytest
import torch

import mma_swizzled_operand_amd as mswz
import workloads as wl
from gpu_util import compare, plan_for, reference, run_gpu, say

pytestmark = pytest.mark.gpu

# stored element -> (torch storage dtype, elements per storage element)
STORE = {"f16": (torch.int16, 1), "bf16": (torch.int16, 1), "e4m3": (torch.uint8, 1), "e2m1": (torch.uint8, 2),
         "e2m3": (torch.uint8, 1), "e3m2": (torch.uint8, 1)}
# padding that would poison any output it entered
POISON = {"f16": 0x7C00, "bf16": 0x7F80, "e4m3": 0x7F, "e2m1": 0x77, "e2m3": 0xFF, "e3m2": 0xFF}
D_SENTINEL = {"f32": -12345.5, "bf16": -123.5, "f16": -123.5}
D_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

# (workload, lda, ldb, ldd, D format)
CASES = {
    "bf16-k": (wl.custom(512, 768, 320, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                         name="bf16-k"), 384, 328, 772, "f32"),
    "f16-amn-tail-beta": (wl.custom(296, 260, 192, "f16", a_major="mn", beta=1, name="f16-amn-tail-beta"),
                          304, 208, 264, "f32"),
    "bf16-both-mn": (wl.custom(256, 512, 128, "bf16", a_major="mn", b_major="mn", name="bf16-both-mn"),
                     264, 520, 0, "f32"),
    "f16-bmn-beta": (wl.custom(512, 256, 192, "f16", b_major="mn", beta=1, name="f16-bmn-beta"),
                     0, 264, 260, "f32"),
    "e4m3-mx": (wl.custom(512, 256, 1024, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                          name="e4m3-mx"), 1040, 1072, 268, "f32"),
    "e4m3-mx-tail-beta": (wl.custom(300, 260, 384, "e4m3", V=32, beta=1, a_dist=("normal", 1.0),
                                    b_dist=("normal", 1.0), name="e4m3-mx-tail-beta"), 400, 0, 264, "f32"),
    "e2m1-beta": (wl.custom(256, 384, 512, "e2m1", V=32, beta=1, a_dist=("normal", 1.0),
                            b_dist=("normal", 1.0), name="e2m1-beta"), 544, 576, 388, "f32"),
    "bf16-out-tail": (wl.custom(264, 300, 192, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                                name="bf16-out-tail"), 256, 200, 304, "bf16"),
    "e3m2-beta": (wl.custom(256, 264, 512, "e3m2", V=32, beta=1, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                            name="e3m2-beta"), 544, 528, 268, "f32"),
    # K tails: the poisoned storage between K and the pitch must never reach the sums
    "bf16-ktail": (wl.custom(256, 256, 72, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                             name="bf16-ktail"), 136, 80, 0, "f32"),
    "f16-amn-ktail-beta": (wl.custom(264, 260, 200, "f16", a_major="mn", beta=1, name="f16-amn-ktail-beta"),
                           272, 264, 268, "f32"),
    "bf16-bmn-ktail-out": (wl.custom(256, 264, 24, "bf16", b_major="mn", name="bf16-bmn-ktail-out"),
                           32, 272, 0, "bf16"),
    # block-scaled K tails: the poisoned storage (NaN codes) between K and the
    # pitch must never reach the sums
    "e4m3-ktail-beta": (wl.custom(264, 256, 160, "e4m3", V=32, beta=1, a_dist=("normal", 1.0),
                                  b_dist=("normal", 1.0), name="e4m3-ktail-beta"), 192, 176, 260, "f32"),
    "e3m2-ktail": (wl.custom(256, 256, 96, "e3m2", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                             name="e3m2-ktail"), 128, 112, 0, "f32"),
}


def embed(arr: np.ndarray, kind: str, ld: int):
    """(storage, view): ``arr`` (stored rows) copied into the left of a
    device buffer whose rows are ``ld`` elements apart, the rest poisoned."""
    tdt, per = STORE[kind]
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a)
    rows, cols = t.shape
    width = ld // per if ld else cols
    poison = POISON[kind]
    if tdt == torch.int16 and poison >= 0x8000:
        poison -= 0x10000
    big = torch.full((rows, width), poison, dtype=tdt)
    big[:, :cols] = t
    big = big.cuda()
    return big, big[:, :cols]


def d_storage(w, d_fmt, ldd, d0=None):
    width = ldd or w.N
    big = torch.full((w.M, width), D_SENTINEL[d_fmt], dtype=D_TORCH[d_fmt])
    if d0 is not None:
        big[:, :w.N] = torch.from_numpy(np.ascontiguousarray(d0)).to(D_TORCH[d_fmt])
    big = big.cuda()
    return big, big[:, :w.N]


def run_strided(w, x, lda, ldb, ldd, d_fmt):
    plan = mswz.gemm_plan_create_ld(w.M, w.N, w.K, w.kind, w.kind_b, d_fmt, w.a_major, w.b_major, w.V,
                                    lda=lda, ldb=ldb, ldd=ldd)
    assert plan.describe()["tile_m"] == 256
    _, A = embed(x["A"], w.kind, lda)
    _, B = embed(x["B"], w.kind_b, ldb)
    Dbig, D = d_storage(w, d_fmt, ldd, x.get("D0") if w.beta else None)
    if w.V:
        sfa = torch.from_numpy(np.ascontiguousarray(x["SFA"])).cuda()
        sfb = torch.from_numpy(np.ascontiguousarray(x["SFB"])).cuda()
        mswz.gemm_run_blockscaled(plan, A, B, sfa, sfb, D, w.beta)
    else:
        mswz.gemm_run(plan, A, B, D, w.beta)
    torch.cuda.synchronize()
    big = Dbig.cpu()
    if ldd and ldd > w.N:
        bits = torch.int32 if d_fmt == "f32" else torch.int16
        pad = big[:, w.N:].contiguous()
        want = torch.full_like(pad, D_SENTINEL[d_fmt])
        assert torch.equal(pad.view(bits), want.view(bits)), "D padding written"
    return big[:, :w.N].float().numpy()


def packed_run(w, x, d_fmt):
    """The same problem with packed storage; None unless it also takes the 256 tile."""
    plan = mswz.gemm_plan_create(w.M, w.N, w.K, w.kind, w.kind_b, d_fmt, w.a_major, w.b_major, w.V)
    if plan.describe()["tile_m"] != 256:
        return None
    _, A = embed(x["A"], w.kind, 0)
    _, B = embed(x["B"], w.kind_b, 0)
    _, D = d_storage(w, d_fmt, 0, x.get("D0") if w.beta else None)
    if w.V:
        sfa = torch.from_numpy(np.ascontiguousarray(x["SFA"])).cuda()
        sfb = torch.from_numpy(np.ascontiguousarray(x["SFB"])).cuda()
        mswz.gemm_run_blockscaled(plan, A, B, sfa, sfb, D, w.beta)
    else:
        mswz.gemm_run(plan, A, B, D, w.beta)
    torch.cuda.synchronize()
    return D.cpu().float().numpy()


def d0_in_format(x, d_fmt):
    """Round D0 into D's format first, so that the oracle reads what D holds."""
    if "D0" in x and d_fmt != "f32":
        x["D0"] = torch.from_numpy(x["D0"]).to(D_TORCH[d_fmt]).float().numpy()
    return x


@pytest.mark.parametrize("case", sorted(CASES))
def test_strided_against_oracle(case):
    w, lda, ldb, ldd, d_fmt = CASES[case]
    say(f"[strided] {case} {w.M}x{w.N}x{w.K} {w.kind} lda={lda} ldb={ldb} ldd={ldd} D={d_fmt}")
    x = d0_in_format(wl.generate(w, seed=61), d_fmt)
    got = run_strided(w, x, lda, ldb, ldd, d_fmt)
    ref = reference(w, x)
    if d_fmt == "f32":
        compare(w, got, ref, x.get("D0"))
    else:   # rounding to D's format (7 fraction bits for bf16) on top of the fp32 bound
        tol = 2.0 ** -7 * np.abs(ref.value) + 1.01 * 2 * (w.K + 1) * 2.0 ** -24 * ref.mag + ref.wabs
        assert not (np.abs(got - ref.value) > tol).any()
    pk = packed_run(w, x, d_fmt)
    if pk is not None:
        assert np.array_equal(got, pk), "strided and packed results differ"


@pytest.mark.parametrize("case", ["bf16-k", "f16-amn-tail-beta", "bf16-both-mn", "e4m3-mx", "e2m1-beta", "e3m2-beta",
                                  "e4m3-ktail-beta"])
def test_strided_quarter_integers_exact(case):
    w, lda, ldb, ldd, d_fmt = CASES[case]
    say(f"[strided-exact] {case}")
    x = wl.generate(w, seed=62, values="quarter")
    got = run_strided(w, x, lda, ldb, ldd, d_fmt)
    ref = reference(w, x, with_mag=False)
    assert np.array_equal(got, ref.astype(np.float32))


def test_strided_full_size_column_block_of_a_wider_matrix():
    """bf16 4096^3 with A the left half of a [4096][8192] matrix, B the right
    half of a [4096][8192] matrix (the pitch alone differs), and D a block of
    a [4096][4352] output: equal to the packed plan bit for bit, and to the
    oracle on sampled rows and columns."""
    w = wl.custom(4096, 4096, 4096, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0),
                  name="bf16-4096-views")
    say("[strided-full] bf16 4096^3 lda=ldb=8192 ldd=4352")
    x = wl.generate(w, seed=63)
    _, A = embed(x["A"], "bf16", 8192)
    Bbig = torch.full((4096, 8192), POISON["bf16"], dtype=torch.int16)
    Bbig[:, 4096:] = torch.from_numpy(x["B"].view(np.int16))
    Bbig = Bbig.cuda()
    B = Bbig[:, 4096:]
    Dbig, D = d_storage(w, "f32", 4352)
    plan = mswz.gemm_plan_create_ld(4096, 4096, 4096, "bf16", "bf16", lda=8192, ldb=8192, ldd=4352)
    mswz.gemm_run(plan, A, B, D)
    torch.cuda.synchronize()
    big = Dbig.cpu()
    assert torch.equal(big[:, 4096:], torch.full_like(big[:, 4096:], D_SENTINEL["f32"]))
    got = big[:, :4096].numpy()
    packed = run_gpu(w, x, plan_for(w))
    assert np.array_equal(got, packed)
    rows, cols = wl.sample_points(w, 8, 8)
    ref_r = reference(w, x, rows=rows)
    ref_c = reference(w, x, cols=cols)
    compare(w, got[rows], ref_r)
    compare(w, got[:, cols], ref_c)


def test_binding_rejects_mismatched_views():
    plan = mswz.gemm_plan_create_ld(256, 256, 64, "bf16", "bf16", lda=128)
    big = torch.zeros((256, 128), dtype=torch.int16, device="cuda")
    B = torch.zeros((256, 64), dtype=torch.int16, device="cuda")
    D = torch.zeros((256, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        mswz.gemm_run(plan, big, B, D)              # whole storage instead of the view
    with pytest.raises(ValueError):
        mswz.gemm_run(plan, big[:, :60], B, D)      # rows shorter than K
    wide = torch.zeros((256, 192), dtype=torch.int16, device="cuda")
    with pytest.raises(ValueError):
        mswz.gemm_run(plan, wide[:, :64], B, D)     # rows 192 elements apart, plan says 128
    mswz.gemm_run(plan, big[:, :64], B, D)          # the matching view runs
    torch.cuda.synchronize()
