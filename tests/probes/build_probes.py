"""Build tests/probes/libprobes.so (the one-wave instruction probes the GPU
tests use) with hipcc for gfx950, with the library's compile flags."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libprobes.so")


def build() -> str:
    import sys
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from mma_swizzled_operand_amd import _build as B
    src = os.path.join(HERE, "probes.hip")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, "-shared", "-I", B.CSRC, src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
