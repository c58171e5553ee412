"""Weight streaming with K split over workgroups (gemm_run_ws) against the
oracle, through the C ABI.

The split kernel sums S fp32 partials per output in a fixed part order inside
the kernel (the last workgroup of a column block does it), so besides parity
with the oracle these tests check that results are bit-identical run to run
on one workspace, that every call leaves the workspace's counters at zero,
and beta = 1.  Tolerances are those of the dense cases (tests/gpu_util.py):
any fp32 summation order of the exact 16-bit products stays within the
componentwise bound.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import compare, plan_for, reference, run_gpu, say, zero_workspace

pytestmark = pytest.mark.gpu

SMALL = {
    # (M, N, K): K parts chosen by the plan (16, 8, 4 and 4)
    "ws-bf16-2048x4096": wl.custom(64, 2048, 4096, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 0.02),
                                   name="ws-bf16-2048x4096"),
    "ws-f16-1024x2048-beta": wl.custom(64, 1024, 2048, "f16", beta=1, name="ws-f16-1024x2048-beta"),
    "ws-bf16-256x1024": wl.custom(64, 256, 1024, "bf16", name="ws-bf16-256x1024"),
    "ws-f16-4096x1024": wl.custom(64, 4096, 1024, "f16", name="ws-f16-4096x1024"),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_split_small_full_compare(name):
    w = SMALL[name]
    plan = plan_for(w)
    ws = zero_workspace(plan)
    say(f"[splitk] {name} {w.M}x{w.N}x{w.K} {w.kind} beta={w.beta} ws={ws.numel()} B")
    x = wl.generate(w, seed=11)
    got = run_gpu(w, x, plan, workspace=ws)
    ref, mag = reference(w, x)
    print(name, compare(w, got, ref, mag, x.get("D0")))
    counters = ws[:256].cpu().numpy()
    assert not counters.any(), "counters not reset"


def test_split_repeatable_and_counters_reset():
    """Three calls on one workspace: identical bits, counters zero after each."""
    w = SMALL["ws-bf16-2048x4096"]
    plan = plan_for(w)
    ws = zero_workspace(plan)
    x = wl.generate(w, seed=12)
    say("[splitk] repeat x3")
    outs = []
    for _ in range(3):
        outs.append(run_gpu(w, x, plan, workspace=ws))
        assert not ws[:256].cpu().numpy().any()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


def test_split_quarter_exact():
    """Quarter-integer operands: every partial and sum is exact, so the split
    result equals the exact product bit for bit."""
    w = SMALL["ws-bf16-2048x4096"]
    plan = plan_for(w)
    x = wl.generate(w, seed=13, values="quarter")
    say("[splitk] quarter exact")
    got = run_gpu(w, x, plan, workspace=zero_workspace(plan))
    assert np.array_equal(got.astype(np.float64), reference(w, x, with_mag=False))


def test_split_full_size_c4_sampled():
    """The weight-streaming workload at full size through the workspace path."""
    w = wl.WORKLOADS["c4"]
    plan = plan_for(w)
    ws = zero_workspace(plan)
    say(f"[splitk] c4 full size, workspace {ws.numel()} B")
    x = wl.generate(w, seed=0)
    got = run_gpu(w, x, plan, workspace=ws)
    rows, cols = wl.sample_points(w, 8, 8)
    ref_r, mag_r = reference(w, x, rows=rows)
    ref_c, mag_c = reference(w, x, cols=cols)
    print("c4 ws", compare(w, got[rows], ref_r, mag_r), compare(w, got[:, cols], ref_c, mag_c))
    assert not ws[:256].cpu().numpy().any()
