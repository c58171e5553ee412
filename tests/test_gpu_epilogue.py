"""The 256x256 epilogue on ragged tiles, in each of its forms: staged through
LDS with non-temporal stores (16-bit, E2M1, 6-bit, E4M3 kinds with fp32 D)
or stored directly from the accumulators (E4M3 A with 6-bit B).  D sits
inside a larger buffer whose margins must keep their canary value, and the
result is compared with the oracle (tolerances of tests/gpu_util.py).
"""
import numpy as np
import pytest
import torch

import mma_swizzled_operand_amd as mswz
import workloads as wl
from gpu_util import compare, plan_for, reference, say, to_device

pytestmark = pytest.mark.gpu

N01 = dict(a_dist=("normal", 1.0), b_dist=("normal", 1.0))

# M and N not multiples of 256 (nor of 32): partial tiles in both directions
CASES = {
    "e4m3-ragged": wl.custom(300, 292, 256, "e4m3", V=32, name="e4m3-ragged", **N01),
    "e2m3-ragged-beta": wl.custom(264, 300, 384, "e2m3", V=32, beta=1, name="e2m3-ragged-beta", **N01),
    "e2m1-ragged": wl.custom(296, 264, 512, "e2m1", V=32, name="e2m1-ragged", **N01),
    "e2m1p-ragged": wl.custom(260, 296, 256, "e2m1p", V=32, name="e2m1p-ragged", **N01),
    "e4m3xe2m3-ragged": wl.custom(300, 292, 384, "e4m3", V=32, name="e4m3xe2m3-ragged", b_kind="e2m3", **N01),
    "bf16-ragged-beta": wl.custom(300, 292, 192, "bf16", beta=1, name="bf16-ragged-beta"),
    "f16-amn-ragged": wl.custom(264, 300, 128, "f16", a_major="mn", name="f16-amn-ragged"),
}

PAD = 4096   # canary floats before and after D


@pytest.mark.parametrize("name", list(CASES))
def test_epilogue_stays_inside_d(name):
    w = CASES[name]
    plan = plan_for(w)
    assert plan.describe()["tile_m"] == 256
    say(f"[epilogue] {name} {w.M}x{w.N}x{w.K} {w.kind}/{w.kind_b} beta={w.beta}")
    x = wl.generate(w, seed=31)
    n = w.M * w.N
    buf = torch.full((n + 2 * PAD,), 7.0, dtype=torch.float32, device="cuda")
    D = buf[PAD:PAD + n]
    if w.beta:
        D.copy_(torch.from_numpy(np.ascontiguousarray(x["D0"]).reshape(-1)))
    A, B = to_device(x["A"]), to_device(x["B"])
    if w.V:
        mswz.gemm_run_blockscaled(plan, A, B, to_device(x["SFA"]), to_device(x["SFB"]), D, w.beta)
    else:
        mswz.gemm_run(plan, A, B, D, w.beta)
    torch.cuda.synchronize()
    assert torch.all(buf[:PAD] == 7.0) and torch.all(buf[PAD + n:] == 7.0), "store outside D"
    got = D.cpu().numpy().reshape(w.M, w.N)
    ref = reference(w, x)
    print(name, compare(w, got, ref, x.get("D0")))
