"""Helpers for the GPU parity tests: device upload of the stored inputs,
one library call, and the comparison against the oracle.

Tolerances (fixed before any GPU result was seen):
* dense (fp16 / bf16): relative Frobenius error <= 1e-3 and max abs error
  <= 1e-2 * sqrt(K / 64), over the compared outputs;
* block-scaled E4M3: relative Frobenius error <= 2e-2;
* additionally, for 16-bit operands (whose products are exact in fp32), every
  output obeys |gpu - ref| <= 2 (K+1) 2^-24 (S + |beta D0|) with S = sum |a b|:
  a rigorous bound for any fp32 summation order of exact products, with a
  factor 2 for adders that truncate;
* quarter-integer inputs: every product and partial sum is exact in fp32, so
  the result must equal the oracle bit for bit.
"""
import sys

import numpy as np
import torch

import mma_swizzled_operand_amd as mswz
import oracle
import workloads as wl

TORCH_STORE = {"f16": torch.int16, "bf16": torch.int16, "e4m3": torch.uint8}


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def to_device(arr: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def plan_for(w: wl.Workload) -> mswz.Plan:
    return mswz.gemm_plan_create(w.M, w.N, w.K, w.kind, w.kind_b, "f32", w.a_major, w.b_major, w.V)


def run_gpu(w: wl.Workload, x: dict, plan=None, D_init=None, workspace=None) -> np.ndarray:
    """One library call on fresh device copies; returns D as fp32 numpy.  With
    a workspace tensor the call goes through gemm_run_ws."""
    plan = plan or plan_for(w)
    A, B = to_device(x["A"]), to_device(x["B"])
    if w.beta:
        D = to_device(x["D0"])
    elif D_init is not None:
        D = to_device(D_init)
    else:
        D = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    if w.V:
        mswz.gemm_run_blockscaled(plan, A, B, to_device(x["SFA"]), to_device(x["SFB"]), D, w.beta)
    elif workspace is not None:
        mswz.gemm_run_ws(plan, A, B, D, workspace, w.beta)
    else:
        mswz.gemm_run(plan, A, B, D, w.beta)
    torch.cuda.synchronize()
    return D.cpu().numpy()


def zero_workspace(plan):
    """A zero-filled device workspace of the size the plan asks for."""
    n = plan.workspace_bytes()
    assert n > 0, "plan has no workspace path"
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def reference(w: wl.Workload, x: dict, rows=None, cols=None, with_mag=True):
    return oracle.gemm(w.M, w.N, w.K, w.kind, w.a_major, x["A"], w.kind_b, w.b_major, x["B"],
                       V=w.V, SFA=x.get("SFA"), SFB=x.get("SFB"), beta=w.beta, D0=x.get("D0"),
                       rows=rows, cols=cols, with_mag=with_mag)


def compare(w: wl.Workload, got: np.ndarray, ref: np.ndarray, mag: np.ndarray, d0=None) -> dict:
    got = got.astype(np.float64)
    diff = got - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    out = {"rel_fro": rel, "max_abs": mx, "n": int(diff.size)}
    assert np.isfinite(got).all(), "non-finite output"
    if w.V:
        assert rel <= 2e-2, out
    else:
        assert rel <= 1e-3, out
        assert mx <= 1e-2 * np.sqrt(w.K / 64), out
        extra = np.abs(d0.astype(np.float64)) if (w.beta and d0 is not None) else 0.0
        bound = 2 * (w.K + 1) * 2.0 ** -24 * (mag + extra)
        bad = np.abs(diff) > bound
        assert not bad.any(), {"violations": int(bad.sum()), **out}
    return out
