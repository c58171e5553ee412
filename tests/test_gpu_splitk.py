"""Weight streaming with K split over workgroups (gemm_run_ws) against the
oracle, through the C ABI.

The streaming kernel stores S fp32 partials per output in the workspace and a
second kernel sums them in a fixed part order and applies beta, so besides
parity with the oracle these tests check that results are bit-identical run to
run on one workspace (also when a captured graph replays the call), that the
workspace's prior contents (filled with NaNs here) do not matter, and beta =
1.  Tolerances are those of the dense cases (tests/gpu_util.py): any fp32
summation order of the exact 16-bit products stays within the componentwise
bound.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import compare, plan_for, reference, run_gpu, say, poisoned_workspace

pytestmark = pytest.mark.gpu

SMALL = {
    # (M, N, K): K parts chosen by the plan (16, 8, 4 and 4)
    "ws-bf16-2048x4096": wl.custom(64, 2048, 4096, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 0.02),
                                   name="ws-bf16-2048x4096"),
    "ws-f16-1024x2048-beta": wl.custom(64, 1024, 2048, "f16", beta=1, name="ws-f16-1024x2048-beta"),
    "ws-bf16-256x1024": wl.custom(64, 256, 1024, "bf16", name="ws-bf16-256x1024"),
    "ws-f16-4096x1024": wl.custom(64, 4096, 1024, "f16", name="ws-f16-4096x1024"),
    # M below 64 (decode-style batches): padded rows are never read nor stored
    "ws-bf16-m1": wl.custom(1, 2048, 4096, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 0.02),
                            name="ws-bf16-m1"),
    "ws-f16-m17-beta": wl.custom(17, 1024, 2048, "f16", beta=1, name="ws-f16-m17-beta"),
    "ws-bf16-m32": wl.custom(32, 4096, 2048, "bf16", name="ws-bf16-m32"),
    "ws-bf16-m48-beta": wl.custom(48, 2048, 1024, "bf16", beta=1, a_dist=("normal", 1.0),
                                  b_dist=("normal", 0.02), name="ws-bf16-m48-beta"),
}

# parts of 2048 or 1024 K elements: the K-sliced streaming kernel (each wave
# keeps a 256- or 128-element slice of A in registers), M padded to 16, 32 or 64
KSLICE = {
    "ks-bf16-m64-k32768": wl.custom(64, 256, 32768, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 0.02),
                                    name="ks-bf16-m64-k32768"),      # S = 16, slices of 256
    "ks-f16-m20-k16384-beta": wl.custom(20, 512, 16384, "f16", beta=1, name="ks-f16-m20-k16384-beta"),  # S = 16, 128
    "ks-bf16-m1-k32768": wl.custom(1, 1024, 32768, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 0.02),
                                   name="ks-bf16-m1-k32768"),        # S = 16, 256
    "ks-bf16-m48-k16384-beta": wl.custom(48, 4096, 16384, "bf16", beta=1, name="ks-bf16-m48-k16384-beta"),  # 128
    "ks-f16-m64-n16384-k4096": wl.custom(64, 16384, 4096, "f16", name="ks-f16-m64-n16384-k4096"),  # S = 4, 128
    "ks-bf16-m32-n8192-k16384": wl.custom(32, 8192, 16384, "bf16", a_dist=("normal", 1.0),
                                          b_dist=("normal", 0.02), name="ks-bf16-m32-n8192-k16384"),  # S = 8, 256
    "ks-f16-m16-n32768-k2048-beta": wl.custom(16, 32768, 2048, "f16", beta=1,
                                              name="ks-f16-m16-n32768-k2048-beta"),  # S = 2, 128
}

# the same kernels without a workspace (K not split), ragged M
UNSPLIT = {
    "skinny-f16-m1": wl.custom(1, 1024, 1024, "f16", name="skinny-f16-m1"),
    "skinny-bf16-m20-beta": wl.custom(20, 2048, 2048, "bf16", beta=1, name="skinny-bf16-m20-beta"),
    "skinny-bf16-m33": wl.custom(33, 1024, 3072, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 0.02),
                                 name="skinny-bf16-m33"),
    "skinny-f16-m63-n1088": wl.custom(63, 1088, 1024, "f16", name="skinny-f16-m63-n1088"),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_split_small_full_compare(name):
    w = SMALL[name]
    plan = plan_for(w)
    ws = poisoned_workspace(plan)
    say(f"[splitk] {name} {w.M}x{w.N}x{w.K} {w.kind} beta={w.beta} ws={ws.numel()} B")
    x = wl.generate(w, seed=11)
    got = run_gpu(w, x, plan, workspace=ws)
    ref = reference(w, x)
    print(name, compare(w, got, ref, x.get("D0")))


def ks_parts(w):
    """K parts the plan picks (the smallest power of two up to 16 giving at
    least 256 workgroups of 256 columns, else the largest that fits K)."""
    best = 0
    for s in (2, 4, 8, 16):
        if w.K % (256 * s):
            continue
        best = s
        if w.N // 256 * s >= 256:
            break
    return best


@pytest.mark.parametrize("name", list(KSLICE))
def test_kslice_full_compare(name):
    w = KSLICE[name]
    assert w.K // ks_parts(w) in (1024, 2048), "case must reach the K-sliced kernel"
    plan = plan_for(w)
    ws = poisoned_workspace(plan)
    say(f"[splitk-ks] {name} {w.M}x{w.N}x{w.K} {w.kind} beta={w.beta} parts={ks_parts(w)}")
    x = wl.generate(w, seed=21)
    got = run_gpu(w, x, plan, workspace=ws)
    if w.M * w.N * w.K <= (1 << 30):
        ref = reference(w, x)
        print(name, compare(w, got, ref, x.get("D0")))
    else:
        cols = wl.sample_points(w, 8, 64)[1]
        ref = reference(w, x, cols=cols)
        print(name, compare(w, got[:, cols], ref, None if x.get("D0") is None else x["D0"][:, cols]))
    again = run_gpu(w, x, plan, workspace=ws)
    assert np.array_equal(got, again), "not bit-identical run to run"


def test_kslice_graph_replays():
    """One K-sliced call (S = 4, beta = 1) captured in a graph and replayed
    three times with other work, workspace fills and synchronisations between
    the replays; each replay restores D0 first (inside the graph) and must
    give the eager call's bits."""
    import mma_swizzled_operand_amd as mswz
    w = wl.custom(64, 16384, 4096, "bf16", beta=1, a_dist=("normal", 1.0), b_dist=("normal", 0.02),
                  name="ks-graph")
    plan = plan_for(w)
    x = wl.generate(w, seed=24)
    A, B = (torch.from_numpy(np.ascontiguousarray(x[k]).view(np.int16)).cuda() for k in ("A", "B"))
    D0 = torch.from_numpy(x["D0"]).cuda()
    ws = poisoned_workspace(plan)
    say("[splitk-ks] graph replays")
    D = D0.clone()
    mswz.gemm_run_ws(plan, A, B, D, ws, 1)
    torch.cuda.synchronize()
    eager = D.cpu()
    ref = reference(w, x, cols=wl.sample_points(w, 8, 16)[1])
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            D.copy_(D0)
            mswz.gemm_run_ws(plan, A, B, D, ws, 1)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(3):
        junk = torch.randn(1 << 20, device="cuda") * 3.0
        ws.fill_(0xFF if r == 1 else 0)   # the partials' old contents do not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(D.cpu().view(torch.int32), eager.view(torch.int32)), f"replay {r} differs"
        del junk
    cols = wl.sample_points(w, 8, 16)[1]
    compare(w, eager.numpy()[:, cols], ref, x["D0"][:, cols])


@pytest.mark.parametrize("name", ["ks-bf16-m64-k32768", "ks-bf16-m1-k32768"])
def test_kslice_quarter_exact(name):
    """Quarter-integer operands: every product, per-wave partial and sum is
    exact in fp32, so the result equals the exact product bit for bit."""
    w = KSLICE[name]
    plan = plan_for(w)
    x = wl.generate(w, seed=22, values="quarter")
    say(f"[splitk-ks] quarter exact {name}")
    got = run_gpu(w, x, plan, workspace=poisoned_workspace(plan))
    assert np.array_equal(got.astype(np.float64), reference(w, x, with_mag=False))


def test_kslice_stores_stay_inside_d_and_workspace():
    """M = 20 (padded to 32): canaries after D and after the workspace."""
    import mma_swizzled_operand_amd as mswz
    w = KSLICE["ks-f16-m20-k16384-beta"]
    plan = plan_for(w)
    x = wl.generate(w, seed=23)
    A, B = (torch.from_numpy(np.ascontiguousarray(x[k]).view(np.int16)).cuda() for k in ("A", "B"))
    n = w.M * w.N
    dbuf = torch.full((n + 4096,), 7.0, dtype=torch.float32, device="cuda")
    dbuf[:n] = torch.from_numpy(x["D0"].reshape(-1)).cuda()
    need = plan.workspace_bytes()
    wbuf = torch.full((need + 4096,), 0xFF, dtype=torch.uint8, device="cuda")
    wbuf[need:] = 0xA5
    say("[splitk-ks] canaries")
    mswz.gemm_run_ws(plan, A, B, dbuf[:n], wbuf[:need], 1)
    torch.cuda.synchronize()
    assert torch.all(dbuf[n:] == 7.0)
    assert torch.all(wbuf[need:] == 0xA5)
    ref = reference(w, x)
    compare(w, dbuf[:n].cpu().numpy().reshape(w.M, w.N), ref, x.get("D0"))


def test_split_repeatable():
    """Three calls on one workspace: identical bits."""
    w = SMALL["ws-bf16-2048x4096"]
    plan = plan_for(w)
    ws = poisoned_workspace(plan)
    x = wl.generate(w, seed=12)
    say("[splitk] repeat x3")
    outs = [run_gpu(w, x, plan, workspace=ws) for _ in range(3)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


def test_split_quarter_exact():
    """Quarter-integer operands: every partial and sum is exact, so the split
    result equals the exact product bit for bit."""
    w = SMALL["ws-bf16-2048x4096"]
    plan = plan_for(w)
    x = wl.generate(w, seed=13, values="quarter")
    say("[splitk] quarter exact")
    got = run_gpu(w, x, plan, workspace=poisoned_workspace(plan))
    assert np.array_equal(got.astype(np.float64), reference(w, x, with_mag=False))


def test_split_full_size_c4_sampled():
    """The weight-streaming workload at full size through the workspace path."""
    w = wl.WORKLOADS["c4"]
    plan = plan_for(w)
    ws = poisoned_workspace(plan)
    say(f"[splitk] c4 full size, workspace {ws.numel()} B")
    x = wl.generate(w, seed=0)
    got = run_gpu(w, x, plan, workspace=ws)
    rows, cols = wl.sample_points(w, 8, 8)
    ref_r = reference(w, x, rows=rows)
    ref_c = reference(w, x, cols=cols)
    print("c4 ws", compare(w, got[rows], ref_r), compare(w, got[:, cols], ref_c))


@pytest.mark.parametrize("name", list(UNSPLIT))
def test_unsplit_ragged_m(name):
    w = UNSPLIT[name]
    plan = plan_for(w)
    assert plan.describe()["variant"] == 21
    say(f"[skinny] {name} {w.M}x{w.N}x{w.K} {w.kind} beta={w.beta}")
    x = wl.generate(w, seed=14)
    got = run_gpu(w, x, plan)
    ref = reference(w, x)
    print(name, compare(w, got, ref, x.get("D0")))
    xq = wl.generate(w, seed=15, values="quarter")
    assert np.array_equal(run_gpu(w, xq, plan), reference(w, xq, with_mag=False).astype(np.float32))


@pytest.mark.parametrize("split", [True, False])
def test_ragged_m_stores_stay_inside_d_and_workspace(split):
    """M = 17: canaries after D (and after the workspace) are unchanged."""
    import mma_swizzled_operand_amd as mswz
    w = SMALL["ws-f16-m17-beta"]
    plan = plan_for(w)
    x = wl.generate(w, seed=16)
    A, B = (torch.from_numpy(np.ascontiguousarray(x[k]).view(np.int16)).cuda() for k in ("A", "B"))
    n = w.M * w.N
    dbuf = torch.full((n + 4096,), 7.0, dtype=torch.float32, device="cuda")
    dbuf[:n] = torch.from_numpy(x["D0"].reshape(-1)).cuda()
    need = plan.workspace_bytes()
    wbuf = torch.full((need + 4096,), 0xFF, dtype=torch.uint8, device="cuda")
    wbuf[need:] = 0xA5
    say(f"[skinny] canaries split={split}")
    if split:
        mswz.gemm_run_ws(plan, A, B, dbuf[:n], wbuf[:need], 1)
    else:
        mswz.gemm_run(plan, A, B, dbuf[:n], 1)
    torch.cuda.synchronize()
    assert torch.all(dbuf[n:] == 7.0)
    assert torch.all(wbuf[need:] == 0xA5)
    ref = reference(w, x)
    compare(w, dbuf[:n].cpu().numpy().reshape(w.M, w.N), ref, x.get("D0"))


def test_decode_m16_full_size_sampled():
    """16 x 16384 x 8192 bf16 (the weight-streaming workload with a 16-row
    batch) through the workspace path, on sampled rows and columns."""
    w = wl.custom(16, 16384, 8192, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 0.02), name="decode-m16")
    plan = plan_for(w)
    ws = poisoned_workspace(plan)
    say("[splitk] 16x16384x8192")
    x = wl.generate(w, seed=17)
    got = run_gpu(w, x, plan, workspace=ws)
    cols = wl.sample_points(w, 8, 16)[1]
    ref = reference(w, x, cols=cols)
    print("decode-m16", compare(w, got[:, cols], ref))
