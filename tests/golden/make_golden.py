"""Writes tests/golden/tensor_mma_example.json from the fp64 oracle only.

Inputs follow the tcgen05.mma page's example test ("Example: four K16 issues
for a 128x64x64 product"): default_rng(0), A = integers(-4, 5, (128, 64)) / 4
and B = integers(-4, 5, (64, 64)) / 4 as fp16, B held (N, K); the same draw
continued for a (256, 64) B gives the single-tile (128x256x64) shape.
Run from the repository root: python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def main():
    rng = np.random.default_rng(0)
    a = (rng.integers(-4, 5, (128, 64)) / 4).astype("float16")
    b = (rng.integers(-4, 5, (64, 64)) / 4).astype("float16")
    b2 = (rng.integers(-4, 5, (256, 64)) / 4).astype("float16")
    out = {"source": "tcgen05.mma page, 'Example: four K16 issues for a 128x64x64 product' (test block)",
           "recipe": "default_rng(0); a=(integers(-4,5,(128,64))/4).astype(f16); "
                     "b=(integers(-4,5,(64,64))/4).astype(f16); b2=(integers(-4,5,(256,64))/4).astype(f16)",
           "cases": {}}
    for name, bb in (("128x64x64", b), ("128x256x64", b2)):
        d = oracle.gemm(128, bb.shape[0], 64, "f16", "k", a.view(np.uint16), "f16", "k", bb.view(np.uint16))
        d32 = d.astype(np.float32)
        assert np.array_equal(d32.astype(np.float64), d)   # exact in fp32
        out["cases"][name] = {
            "M": 128, "N": int(bb.shape[0]), "K": 64,
            "sha256_f32_le": hashlib.sha256(d32.astype("<f4").tobytes()).hexdigest(),
            "row0_first8": [float(v) for v in d[0, :8]],
            "diag_first8": [float(d[i, i]) for i in range(8)],
            "sum": float(d.sum()),
            "abs_max": float(np.abs(d).max()),
        }
    path = os.path.join(ROOT, "tests", "golden", "tensor_mma_example.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path)


if __name__ == "__main__":
    main()
