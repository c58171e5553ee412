"""Build libmswz.so in-tree from csrc/*.hip for gfx950 with hipcc.

Every HIP source is compiled with packed-fp32 instructions disabled (the
compiler's own float code is used instead) and linked into one shared library
next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmswz.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


# Per-source additions: an LLVM scheduling strategy where it measured faster
# (8192^3, same-box A/B).  The kernels with an E4M3 A, fp32 D and 32-byte
# scale groups fit their registers only under the iterative ILP strategy
# (E4M3 alone: 20 registers spilled and reloaded every K step under the
# default); under it the 16-bit kernels with a K-major A run 1.5 % faster
# (0.6 % with B MN-major) and the padded 6-bit ones 2.3 %, the MN-major-A
# ones 0.5-4.5 % slower.  Both operands MN-major (32x32x16 MFMAs) run 4 %
# faster under the max-ILP strategy, which slows the others by 2-5 %; so
# do the weight-streaming kernels for a few rows of A (64 x 16384 x 8192,
# K-sliced: 3 %, the same registers in another order).  The remaining units
# keep the default, under which they spill least.
_ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
_MAX_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
EXTRA_FLAGS = {
    "gemm256_e4m3_f32.hip": _ILP,
    "gemm256_mixed_e4m3_f32.hip": _ILP,
    "gemm256_bf16_ak.hip": _ILP,
    "gemm256_f16_ak.hip": _ILP,
    "gemm256_fp6.hip": _ILP,
    "gemm256_bf16_amn_bmn.hip": _MAX_ILP,
    "gemm256_f16_amn_bmn.hip": _MAX_ILP,
    "gemm_skinny_sk.hip": _MAX_ILP,
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmswz.so")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _stale(src: str) -> bool:
    """True if src's object is missing or older than src or any csrc header."""
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [src] + glob.glob(os.path.join(CSRC, "*.hpp"))
    return any(os.path.getmtime(d) > t for d in deps)


def build(jobs: int | None = None, only_changed: bool = False) -> str:
    """Compile every csrc/*.hip and link libmswz.so (always rebuilds, unless
    only_changed: then sources whose objects are current are not recompiled)."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    if only_changed:
        fresh = [s for s in srcs if not _stale(s)]
        srcs = [s for s in srcs if _stale(s)]
    else:
        fresh = []
    jobs = jobs or max(1, min(len(srcs), 8))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    objs = sorted(objs + [os.path.join(OBJ, os.path.basename(f) + ".o") for f in fresh])
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    import sys
    print(build(only_changed="--changed" in sys.argv[1:]))
