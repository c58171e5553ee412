"""gemm_run_ws_noalloc (the split weight-streaming path with the library's own
static scratch instead of a caller workspace) against gemm_run_ws, through
the C ABI: the same kernels, so the outputs must agree bit for bit; both are
also checked against the oracle with the parity tolerances
(tests/gpu_util.py).  Two calls in a row share the scratch, the second with
a smaller problem, so a stale partial left by the first would show."""
import numpy as np
import pytest
import torch

import mma_swizzled_operand_amd as mswz
import workloads as wl
from gpu_util import compare, plan_for, poisoned_workspace, reference, say, to_device

pytestmark = pytest.mark.gpu


def _run(w, x, noalloc):
    plan = plan_for(w)
    A, B = to_device(x["A"]), to_device(x["B"])
    if w.beta:
        D = to_device(x["D0"])
    else:
        D = torch.full((w.M, w.N), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        mswz.gemm_run_ws_noalloc(plan, A, B, D, w.beta)
    else:
        mswz.gemm_run_ws(plan, A, B, D, poisoned_workspace(plan), w.beta)
    torch.cuda.synchronize()
    return D.cpu().numpy()


def test_noalloc_matches_workspace_path_on_two_calls_the_second_smaller():
    big = wl.WORKLOADS["c4"]                      # 64 x 16384 x 8192: 16 MiB of partials, the whole scratch
    small = wl.custom(17, 4096, 4096, "f16", beta=1, name="noalloc-small")   # 16 parts x 17 x 4096
    assert plan_for(big).workspace_bytes() == mswz.gemm_noalloc_scratch_bytes()
    assert 0 < plan_for(small).workspace_bytes() < plan_for(big).workspace_bytes()
    for w, seed in ((big, 91), (small, 92)):
        say(f"[noalloc] {w.name} {w.M}x{w.N}x{w.K} {w.kind} beta={w.beta}")
        x = wl.generate(w, seed=seed)
        got = _run(w, x, noalloc=True)
        want = _run(w, x, noalloc=False)
        assert np.array_equal(got, want), "noalloc and workspace paths differ"
        cols = wl.sample_points(w, 8, 32)[1]
        ref = reference(w, x, cols=cols)
        print(w.name, compare(w, got[:, cols], ref, x["D0"][:, cols] if w.beta else None))


def test_noalloc_without_split_path_runs_as_gemm_run():
    w = wl.custom(256, 512, 128, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0), name="noalloc-dense")
    assert plan_for(w).workspace_bytes() == 0
    x = wl.generate(w, seed=93)
    say("[noalloc] dense plan")
    got = _run(w, x, noalloc=True)
    plan = plan_for(w)
    A, B = to_device(x["A"]), to_device(x["B"])
    D = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    mswz.gemm_run(plan, A, B, D, 0)
    torch.cuda.synchronize()
    assert np.array_equal(got, D.cpu().numpy())
