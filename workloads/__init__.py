"""Seeded synthetic inputs for the swizzled-operand GEMM.

This module is shared by the tests, the benchmark and the oracle side.  It
holds no GEMM arithmetic: it only draws random numbers and rounds them into
the stored element formats with numpy / torch conversions.

Every config is described by its stored layouts (row-major, contiguous):
    A: K-major [M,K] or MN-major [K,M];  B: K-major [N,K] or MN-major [K,N];
    D0: fp32 [M,N] (beta = 1 only);  SFA [M,K/32], SFB [N,K/32] e8m0 bytes.

Recipe (identical for every config): ``numpy.random.default_rng(seed)``,
draws in the order A, B, D0, SFA, SFB, each in the C order of its stored
layout; fp64 samples are rounded to nearest-even into the storage type
(fp16 by numpy; bf16 and e4m3 through an fp32 intermediate by torch; e2m1 to
the nearest of its 16 values, ties to the even code, magnitudes above 6
saturating to 6, then packed two per byte, element 2j in the low nibble;
e2m3 and e3m2 to the nearest of their 64 values, ties to the even code,
saturating at 7.5 and 28, then packed sixteen per 16-byte block in bits
6j .. 6j+5 of the block's first twelve bytes, little-endian, the last four
bytes zero; "e2m1p" rounds like e2m1 and stores sixteen per 16-byte block,
eight bytes of nibbles then eight zero bytes);
e8m0 scale bytes are 127 + u with u a uniform integer in [-4, 4].
SFA and SFB are generated [M,K/32] and [N,K/32] for every config; a config
with sf_major "mn" hands the library their transposes, [K/32,M] and
[K/32,N] (the same values).
The quarter-integer variant (the tcgen05.mma page's example test draws
integers in [-4, 4] divided by 4) replaces every operand value, keeps D0's
recipe and sets every scale byte to 127, so every product and partial sum is
exact in fp32; for e2m1, which has no 0.25 or 0.75, it draws integers in
[-2, 2] divided by 2 instead.  The "quarter_scaled" variant draws the same
values but keeps random scale bytes, 127 + u with u uniform in [-2, 2]: each
scaled product is then a multiple of 2^-8 of magnitude at most 16, so for
K <= 4096 every partial sum is a multiple of 2^-8 of magnitude at most 2^16,
i.e. an integer multiple of 2^-8 below 2^24 units, and still exact in fp32.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field, replace

import numpy as np
import torch

#: Stored element kinds, named as in the oracle and the binding.
KINDS = ("f16", "bf16", "e4m3", "e2m1", "e2m3", "e3m2", "e2m1p")


@dataclass(frozen=True)
class Workload:
    name: str
    title: str
    M: int
    N: int
    K: int
    kind: str                 # operand element kind for A (and B unless b_kind is set)
    a_major: str = "k"        # "k" or "mn"
    b_major: str = "k"
    beta: int = 0
    V: int = 0                # 0 dense, 32 MX block-scaled
    a_dist: tuple = ("uniform", 1.0)   # ("uniform", half-width) or ("normal", sigma)
    b_dist: tuple = ("uniform", 1.0)
    tags: tuple = field(default=())
    b_kind: str = ""          # B's element kind when it differs from A's
    sf_major: str = "k"       # scales handed to the library [M,K/32] ("k") or [K/32,M] ("mn")

    @property
    def kind_b(self) -> str:
        return self.b_kind or self.kind

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def algorithmic_bytes(self) -> int:
        """Minimal HBM traffic of one call: A + B (+ scales) + D write
        (+ D read when beta = 1)."""
        def per(kind):   # stored bytes per element (6-bit kinds: sixteen per 16 bytes)
            return {"e4m3": (1, 1), "e2m1": (1, 2), "e2m3": (1, 1), "e3m2": (1, 1), "e2m1p": (1, 1)}.get(kind, (2, 1))
        (na, da), (nb, db) = per(self.kind), per(self.kind_b)
        b = self.M * self.K * na // da + self.N * self.K * nb // db + self.M * self.N * 4
        if self.V:
            b += (self.M + self.N) * (self.K // self.V)
        if self.beta:
            b += self.M * self.N * 4
        return b


WORKLOADS = {
    "c1": Workload("c1", "single tile: D[128,256] fp32 = A[128,64] fp16 . B[256,64]^T, K-major, U[-1,1)",
                   128, 256, 64, "f16", tags=("oracle-full",)),
    "c2": Workload("c2", "square dense 4096^3 bf16, A and B K-major, N(0,1)",
                   4096, 4096, 4096, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0)),
    "c3": Workload("c3", "8192^3 fp16, A MN-major [K,M], B K-major [N,K], U[-1,1), beta=1 onto seeded D0",
                   8192, 8192, 8192, "f16", a_major="mn", beta=1),
    "c4": Workload("c4", "skinny weight-streaming M=64 N=16384 K=8192 bf16, A N(0,1), B N(0,0.02)",
                   64, 16384, 8192, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 0.02)),
    "c5": Workload("c5", "MX-fp8 8192^3 e4m3 K-major, one e8m0 scale 2^u (u in [-4,4]) per 32 K per row",
                   8192, 8192, 8192, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0)),
    "c6": Workload("c6", "MX-fp4 8192^3 e2m1 K-major, N(0,1) rounded to e2m1, one e8m0 scale 2^u (u in [-4,4]) per 32 K per row",
                   8192, 8192, 8192, "e2m1", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0)),
    "c7": Workload("c7", "MX-fp6 8192^3 e2m3 K-major (padded, sixteen per 16 bytes), N(0,1) rounded to e2m3, one e8m0 scale 2^u (u in [-4,4]) per 32 K per row",
                   8192, 8192, 8192, "e2m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0)),
    "c8": Workload("c8", "MX-fp6 8192^3 e3m2 K-major (padded, sixteen per 16 bytes), N(0,1) rounded to e3m2, one e8m0 scale 2^u (u in [-4,4]) per 32 K per row",
                   8192, 8192, 8192, "e3m2", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0)),
    "c9": Workload("c9", "MX mixed 8192^3: A e4m3, B e2m3 (padded), K-major, N(0,1) rounded to each format, one e8m0 scale 2^u (u in [-4,4]) per 32 K per row",
                   8192, 8192, 8192, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0), b_kind="e2m3"),
    "c10": Workload("c10", "MX mixed 8192^3: A e4m3, B e2m1 padded (sixteen per 16 bytes), K-major, N(0,1) rounded to each format, one e8m0 scale 2^u (u in [-4,4]) per 32 K per row",
                    8192, 8192, 8192, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0), b_kind="e2m1p"),
    "c3b": Workload("c3b", "square dense 8192^3 bf16, A and B K-major, N(0,1)",
                    8192, 8192, 8192, "bf16", a_dist=("normal", 1.0), b_dist=("normal", 1.0)),
    # the remaining operand layouts at the square size
    "c11": Workload("c11", "8192^3 bf16, A K-major [M,K], B MN-major [K,N], N(0,1)",
                    8192, 8192, 8192, "bf16", b_major="mn", a_dist=("normal", 1.0), b_dist=("normal", 1.0)),
    "c12": Workload("c12", "8192^3 bf16, A MN-major [K,M], B MN-major [K,N], N(0,1)",
                    8192, 8192, 8192, "bf16", a_major="mn", b_major="mn", a_dist=("normal", 1.0),
                    b_dist=("normal", 1.0)),
    "c13": Workload("c13", "MX mixed 8192^3: A e4m3, B e2m1 dense (two per byte), K-major, N(0,1) rounded to each format, one e8m0 scale 2^u (u in [-4,4]) per 32 K per row",
                    8192, 8192, 8192, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0), b_kind="e2m1"),
    "c14": Workload("c14", "MX-fp8 8192^3 e4m3 K-major as c5, scales stored MN-major ([K/32,M] and [K/32,N])",
                    8192, 8192, 8192, "e4m3", V=32, a_dist=("normal", 1.0), b_dist=("normal", 1.0), sf_major="mn"),
}


def custom(M, N, K, kind, a_major="k", b_major="k", beta=0, V=0,
           a_dist=("uniform", 1.0), b_dist=("uniform", 1.0), name="custom", b_kind="") -> Workload:
    kinds = kind if not b_kind or b_kind == kind else f"{kind}x{b_kind}"
    return Workload(name, f"{name} {M}x{N}x{K} {kinds} A:{a_major} B:{b_major} beta={beta} V={V}",
                    M, N, K, kind, a_major, b_major, beta, V, a_dist, b_dist, b_kind=b_kind if b_kind != kind else "")


def scaled(w: Workload, M=None, N=None, K=None, name=None) -> Workload:
    """Same recipe at another size (for parity cases the oracle finishes fast)."""
    return replace(w, M=M or w.M, N=N or w.N, K=K or w.K, name=name or (w.name + "-small"))


# ---- rounding of fp64 samples into stored formats (library conversions) -------

def to_stored(x: np.ndarray, kind: str) -> np.ndarray:
    """Round fp64 values into the stored bit patterns of ``kind``."""
    if kind == "e2m1":
        return _to_e2m1_packed(x)
    if kind in _FP6_MAG:
        return _to_fp6_padded(x, kind)
    if kind == "e2m1p":
        return _to_e2m1_padded(x)
    if kind == "f16":
        return np.ascontiguousarray(x.astype(np.float16)).view(np.uint16)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if kind == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if kind == "e4m3":
        if np.abs(x).max(initial=0.0) > 448.0:
            raise ValueError("value outside the e4m3 range")
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(kind)


# E2M1 magnitudes by code 0..7, and the midpoints between neighbours
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MID = (_E2M1_MAG[1:] + _E2M1_MAG[:-1]) / 2


def _to_e2m1_packed(x: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code (ties to the even code, saturating at 6), packed two
    per byte along the last axis, element 2j in the low nibble."""
    if x.shape[-1] % 2:
        raise ValueError("e2m1 rows need an even number of elements")
    a = np.abs(x)
    lo = np.searchsorted(_E2M1_MID, a, side="left")
    hi = np.searchsorted(_E2M1_MID, a, side="right")
    code = np.where((lo != hi) & (lo % 2 == 1), hi, lo).astype(np.uint8)   # exact tie: even code
    code |= (np.signbit(x).astype(np.uint8) << 3)
    return np.ascontiguousarray(code[..., 0::2] | (code[..., 1::2] << 4))


# E2M3 / E3M2 magnitudes by code 0..31 (the OCP MX formats' value lists:
# E2M3 subnormals 0.125 apart up to 0.875, then 1 .. 1.875, 2 .. 3.75,
# 4 .. 7.5; E3M2 subnormals 0.0625 apart up to 0.1875, then four values per
# binade from 0.25 up to 28)
_FP6_MAG = {
    "e2m3": np.array([i / 8 for i in range(8)] + [1 + i / 8 for i in range(8)] +
                     [2 + i / 4 for i in range(8)] + [4 + i / 2 for i in range(8)]),
    "e3m2": np.array([i / 16 for i in range(4)] +
                     [2.0 ** (e - 3) * (1 + i / 4) for e in range(1, 8) for i in range(4)]),
}


def _to_fp6_padded(x: np.ndarray, kind: str) -> np.ndarray:
    """Nearest code (ties to the even code, saturating at the largest value),
    packed sixteen per 16-byte block along the last axis: value j of a block
    in bits 6j .. 6j+5 of its first twelve bytes (little-endian), the last
    four bytes zero."""
    if x.shape[-1] % 16:
        raise ValueError("6-bit rows need a multiple of 16 elements")
    mag = _FP6_MAG[kind]
    mid = torch.from_numpy((mag[1:] + mag[:-1]) / 2)
    flat = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64).reshape(-1, 16))
    out = torch.zeros((flat.shape[0], 16), dtype=torch.uint8)
    step = 1 << 20   # blocks per chunk (bounded temporaries)
    for b0 in range(0, flat.shape[0], step):
        xb = flat[b0:b0 + step]
        a = xb.abs()
        lo = torch.bucketize(a, mid)                                   # first midpoint >= a
        tie = (lo < mid.numel()) & (mid[lo.clamp(max=mid.numel() - 1)] == a)
        code = (lo + (tie & (lo % 2 == 1))).to(torch.int32)           # exact tie: even code
        code |= torch.signbit(xb).to(torch.int32) << 5
        # four values = 24 bits = three bytes; value 4q + t at bits 6t of group q
        g = code.reshape(-1, 4, 4)
        v = g[..., 0] | (g[..., 1] << 6) | (g[..., 2] << 12) | (g[..., 3] << 18)
        out[b0:b0 + step, :12] = torch.stack([v & 0xFF, (v >> 8) & 0xFF, (v >> 16) & 0xFF], dim=-1).reshape(-1, 12).to(torch.uint8)
    return np.ascontiguousarray(out.numpy().reshape(x.shape))


def _to_e2m1_padded(x: np.ndarray) -> np.ndarray:
    """E2M1 codes (as for the packed form) stored sixteen per 16-byte block:
    eight bytes of nibbles (value 2i in the low nibble of byte i), then eight
    zero bytes of padding."""
    if x.shape[-1] % 16:
        raise ValueError("padded e2m1 rows need a multiple of 16 elements")
    packed = _to_e2m1_packed(x).reshape(x.shape[:-1] + (x.shape[-1] // 16, 8))
    out = np.zeros(x.shape[:-1] + (x.shape[-1] // 16, 16), dtype=np.uint8)
    out[..., :8] = packed
    return np.ascontiguousarray(out.reshape(x.shape))


def _draw(rng, dist, size):
    kind, p = dist
    if kind == "uniform":
        return rng.uniform(-p, p, size)
    if kind == "normal":
        return rng.normal(0.0, p, size)
    raise ValueError(kind)


def _quarter(rng, size, kind="f16"):
    if kind in ("e2m1", "e2m1p"):
        return rng.integers(-2, 3, size) / 2.0
    return rng.integers(-4, 5, size) / 4.0


def value_shapes(w: Workload) -> dict:
    """Shapes of the drawn values (one per element, before packing)."""
    s = {
        "A": (w.M, w.K) if w.a_major == "k" else (w.K, w.M),
        "B": (w.N, w.K) if w.b_major == "k" else (w.K, w.N),
    }
    if w.beta:
        s["D0"] = (w.M, w.N)
    if w.V:
        s["SFA"] = (w.M, w.K // w.V)
        s["SFB"] = (w.N, w.K // w.V)
    return s


def stored_shapes(w: Workload) -> dict:
    """Shapes of the stored arrays (e2m1 rows hold two elements per byte)."""
    s = value_shapes(w)
    for name, kind in (("A", w.kind), ("B", w.kind_b)):
        if kind == "e2m1":
            r, c = s[name]
            s[name] = (r, c // 2)
    return s


def generate(w: Workload, seed: int = 0, values: str = "config") -> dict:
    """Stored inputs of workload ``w`` (numpy arrays, raw bit patterns).

    values = "config": the config's distributions; "quarter": quarter-integer
    operands in [-1, 1] with unit scales (exact in fp32 in any summation order);
    "quarter_scaled": the same operands with scale bytes 127 + u, u uniform in
    [-2, 2] (still exact for K <= 4096).
    """
    if values not in ("config", "quarter", "quarter_scaled"):
        raise ValueError(values)
    if values == "quarter_scaled" and w.K > 4096:
        raise ValueError("quarter_scaled inputs are exact in fp32 only for K <= 4096")
    rng = np.random.default_rng(seed)
    shapes = value_shapes(w)
    out = {}
    for name, dist, kind in (("A", w.a_dist, w.kind), ("B", w.b_dist, w.kind_b)):
        x = _quarter(rng, shapes[name], kind) if values != "config" else _draw(rng, dist, shapes[name])
        out[name] = to_stored(x, kind)
    if w.beta:
        out["D0"] = rng.uniform(-1.0, 1.0, shapes["D0"]).astype(np.float32)
    if w.V:
        for name in ("SFA", "SFB"):
            u = rng.integers(-4, 5, shapes[name])
            if values == "quarter":
                u = np.zeros_like(u)
            elif values == "quarter_scaled":
                u = rng.integers(-2, 3, shapes[name])
            out[name] = (127 + u).astype(np.uint8)
    return out


def digest(inputs: dict) -> str:
    """sha256 over the stored bytes, in key order (reproducibility check)."""
    h = hashlib.sha256()
    for k in sorted(inputs):
        h.update(k.encode())
        h.update(np.ascontiguousarray(inputs[k]).tobytes())
    return h.hexdigest()


def sample_points(w: Workload, n_rows: int = 8, n_cols: int = 8, seed: int = 1):
    """Rows and columns whose full cross product is checked at full size.

    Always includes the first and last row/column and rows/columns at every
    position a 32x32 sub-tile and a 256x256 tile can take modulo their size,
    then random others."""
    rng = np.random.default_rng(seed)

    def pick(n, total):
        base = {0, total - 1}
        for off in (31, 32, 127, 128, 255):
            if off < total:
                base.add(off)
        while len(base) < min(n, total):
            base.add(int(rng.integers(0, total)))
        return np.array(sorted(base), dtype=np.int64)

    return pick(n_rows, w.M), pick(n_cols, w.N)
