"""Python binding of libmswz.so — the swizzled-operand GEMM for MI355X (gfx950).

A thin ctypes layer over the C ABI in include/mswz_gemm.h, with the same
names.  It only marshals arguments: every step of the computation runs in the
HIP kernels of libmswz.so.  PyTorch supplies device memory and the stream;
tensors are checked against the plan's sizes so that a kernel never indexes
outside the buffers it is given.  There is no fallback path: if the library
is missing and cannot be built, importing this package fails.

    plan = gemm_plan_create(M, N, K, "bf16", "bf16", "f32", "k", "k", 0)
    gemm_run(plan, A, B, D, beta=0)            # D = beta*D + A.B^T
    gemm_run_blockscaled(plan, A, B, SFA, SFB, D, beta=0)

A plan made with row pitches (``gemm_plan_create_ld``) takes operands and D
as 2-D views whose rows are ``ld`` elements apart, e.g. ``big[:, :K]``.
"""
from __future__ import annotations

import ctypes
import os
import threading

from . import _build

__all__ = [
    "DTYPES", "MAJORS", "MswzError", "Plan", "gemm_plan_create", "gemm_plan_create_ld", "gemm_run",
    "gemm_run_blockscaled", "gemm_run_opts", "gemm_run_ws", "gemm_run_ws_noalloc", "gemm_noalloc_scratch_bytes", "GemmOpts", "gemm_plan_destroy", "gemm_status_str", "gemm_plan_describe",
    "gemm_plan_set_scale_major",
    "desc_address", "desc_check", "tile_offset", "lds_lanes", "library_path", "load",
]

DTYPES = {"f16": 1, "bf16": 2, "e4m3": 3, "f32": 4, "e2m1": 5, "e2m3": 6, "e3m2": 7, "e2m1p": 8}
MAJORS = {"k": 0, "mn": 1}
STATUS = {"ok": 0, "invalid": -1, "unsupported": -2, "align": -3, "hip": -4, "kind": -5, "scratch": -6}
# bytes per element (the padded 6- and 4-bit kinds: sixteen per 16-byte block, padding included)
_ITEMSIZE = {"f16": 2, "bf16": 2, "e4m3": 1, "f32": 4, "e2m1": 0.5, "e2m3": 1, "e3m2": 1, "e2m1p": 1}
_DESCRIBE_KEYS = ("variant", "tile_m", "tile_n", "tile_k", "threads", "blocks", "lds_bytes", "group_m")

_lock = threading.Lock()
_lib = None


class GemmOpts(ctypes.Structure):
    """The C struct gemm_opts (include/mswz_gemm.h)."""
    _fields_ = [("neg_a", ctypes.c_int), ("neg_b", ctypes.c_int), ("sat_d", ctypes.c_int),
                ("row_mask", ctypes.c_void_p), ("col_zero", ctypes.c_void_p), ("pred", ctypes.c_int)]


class MswzError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        msg = gemm_status_str(code)
        super().__init__(f"{what}: {msg} ({code})" if what else f"{msg} ({code})")


def library_path() -> str:
    return _build.LIB


def load():
    """Load libmswz.so, building it first only if it is not there."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_build.LIB):
            _build.build()
        h = ctypes.CDLL(_build.LIB)
        i64, i32, vp, c_int = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int
        h.gemm_plan_create.argtypes = [ctypes.POINTER(vp), i64, i64, i64, c_int, c_int, c_int,
                                       c_int, c_int, i32]
        h.gemm_plan_create.restype = c_int
        h.gemm_plan_create_ld.argtypes = [ctypes.POINTER(vp), i64, i64, i64, c_int, c_int, c_int,
                                          c_int, c_int, i32, i64, i64, i64]
        h.gemm_plan_create_ld.restype = c_int
        h.gemm_run.argtypes = [vp, vp, vp, vp, c_int, vp]
        h.gemm_run.restype = c_int
        h.gemm_plan_set_scale_major.argtypes = [vp, c_int]
        h.gemm_plan_set_scale_major.restype = c_int
        h.gemm_plan_workspace_size.argtypes = [vp]
        h.gemm_plan_workspace_size.restype = i64
        h.gemm_run_ws.argtypes = [vp, vp, vp, vp, c_int, vp, i64, vp]
        h.gemm_run_ws.restype = c_int
        h.gemm_run_ws_noalloc.argtypes = [vp, vp, vp, vp, c_int, vp]
        h.gemm_run_ws_noalloc.restype = c_int
        h.gemm_noalloc_scratch_bytes.argtypes = []
        h.gemm_noalloc_scratch_bytes.restype = i64
        h.gemm_run_blockscaled.argtypes = [vp, vp, vp, vp, vp, vp, c_int, vp]
        h.gemm_run_blockscaled.restype = c_int
        h.gemm_run_opts.argtypes = [vp, vp, vp, vp, vp, vp, c_int, ctypes.POINTER(GemmOpts), vp]
        h.gemm_run_opts.restype = c_int
        h.gemm_plan_destroy.argtypes = [vp]
        h.gemm_plan_destroy.restype = None
        h.gemm_status_str.argtypes = [c_int]
        h.gemm_status_str.restype = ctypes.c_char_p
        h.gemm_plan_describe.argtypes = [vp, ctypes.POINTER(i64), c_int]
        h.gemm_plan_describe.restype = c_int
        h.mswz_desc_address.argtypes = [i64, i64, i64, i64, c_int, c_int, i64]
        h.mswz_desc_address.restype = i64
        h.mswz_desc_check.argtypes = [i64, i64, c_int, i64]
        h.mswz_desc_check.restype = c_int
        h.mswz_tile_offset.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
        h.mswz_tile_offset.restype = ctypes.c_uint32
        h.mswz_lds_lanes.argtypes = [c_int, c_int, c_int, ctypes.POINTER(ctypes.c_uint32), c_int]
        h.mswz_lds_lanes.restype = c_int
        _lib = h
        return _lib


def gemm_status_str(code: int) -> str:
    return load().gemm_status_str(int(code)).decode()


def _code(x, table, what):
    if isinstance(x, str):
        if x not in table:
            raise ValueError(f"unknown {what} {x!r}")
        return table[x]
    return int(x)


class Plan:
    """An immutable problem description; owns the C plan handle."""

    def __init__(self, M, N, K, a_dt, b_dt, d_dt="f32", a_major="k", b_major="k", scale_vec_len=0,
                 lda=0, ldb=0, ldd=0):
        lib = load()
        h = ctypes.c_void_p()
        self.M, self.N, self.K = int(M), int(N), int(K)
        self.a_dt = a_dt if isinstance(a_dt, str) else _name(DTYPES, a_dt)
        self.b_dt = b_dt if isinstance(b_dt, str) else _name(DTYPES, b_dt)
        self.d_dt = d_dt if isinstance(d_dt, str) else _name(DTYPES, d_dt)
        self.a_major = a_major if isinstance(a_major, str) else _name(MAJORS, a_major)
        self.b_major = b_major if isinstance(b_major, str) else _name(MAJORS, b_major)
        self.scale_vec_len = int(scale_vec_len)
        rc = lib.gemm_plan_create_ld(ctypes.byref(h), self.M, self.N, self.K,
                                     _code(a_dt, DTYPES, "dtype"), _code(b_dt, DTYPES, "dtype"),
                                     _code(d_dt, DTYPES, "dtype"), _code(a_major, MAJORS, "major"),
                                     _code(b_major, MAJORS, "major"), self.scale_vec_len,
                                     int(lda), int(ldb), int(ldd))
        if rc != 0:
            self._h = None
            raise MswzError(rc, "gemm_plan_create_ld")
        self._h = h
        # stored rows and row lengths in elements, and pitches (packed when 0)
        self.a_rows, self.a_cols = (self.K, self.M) if self.a_major == "mn" else (self.M, self.K)
        self.b_rows, self.b_cols = (self.K, self.N) if self.b_major == "mn" else (self.N, self.K)
        self.lda = int(lda) or self.a_cols
        self.ldb = int(ldb) or self.b_cols
        self.ldd = int(ldd) or self.N
        self.sf_major = "k"      # SFA [M][K/V], SFB [N][K/V]; "mn": [K/V][M], [K/V][N]

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("plan has been destroyed")
        return self._h

    def describe(self) -> dict:
        buf = (ctypes.c_int64 * len(_DESCRIBE_KEYS))()
        n = load().gemm_plan_describe(self.handle, buf, len(_DESCRIBE_KEYS))
        if n < 0:
            raise MswzError(n, "gemm_plan_describe")
        return {k: int(buf[i]) for i, k in enumerate(_DESCRIBE_KEYS[:n])}

    def destroy(self):
        if getattr(self, "_h", None) is not None:
            load().gemm_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    # expected storage sizes in bytes
    def a_bytes(self):
        return int(self.M * self.K * _ITEMSIZE[self.a_dt])

    def b_bytes(self):
        return int(self.N * self.K * _ITEMSIZE[self.b_dt])

    def d_bytes(self):
        return int(self.M * self.N * _ITEMSIZE[self.d_dt])

    def sf_bytes(self):
        v = self.scale_vec_len
        return (self.M * (self.K // v), self.N * (self.K // v)) if v else (0, 0)

    def workspace_bytes(self) -> int:
        """Device workspace gemm_run_ws can use for this plan (0: none)."""
        n = int(load().gemm_plan_workspace_size(self.handle))
        if n < 0:
            raise MswzError(n, "gemm_plan_workspace_size")
        return n


def _name(table, code):
    for k, v in table.items():
        if v == code:
            return k
    return str(code)


def gemm_plan_create(M, N, K, a_dt, b_dt, d_dt="f32", a_major="k", b_major="k", scale_vec_len=0) -> Plan:
    return Plan(M, N, K, a_dt, b_dt, d_dt, a_major, b_major, scale_vec_len)


def gemm_plan_create_ld(M, N, K, a_dt, b_dt, d_dt="f32", a_major="k", b_major="k", scale_vec_len=0,
                        lda=0, ldb=0, ldd=0) -> Plan:
    """A plan whose A, B and D rows are lda, ldb, ldd elements apart (0: packed)."""
    return Plan(M, N, K, a_dt, b_dt, d_dt, a_major, b_major, scale_vec_len, lda, ldb, ldd)


def gemm_plan_destroy(plan: Plan) -> None:
    plan.destroy()


def gemm_plan_set_scale_major(plan: Plan, sf_major) -> None:
    """Store SFA / SFB MN-major ("mn": [K/V][M] and [K/V][N]) or row-major
    ("k", the default) for this block-scaled plan."""
    rc = load().gemm_plan_set_scale_major(plan.handle, _code(sf_major, MAJORS, "major"))
    if rc != 0:
        raise MswzError(rc, "gemm_plan_set_scale_major")
    plan.sf_major = sf_major if isinstance(sf_major, str) else _name(MAJORS, sf_major)


def gemm_plan_describe(plan: Plan) -> dict:
    return plan.describe()


def _dev_ptr(t, nbytes: int, name: str):
    """Device pointer of a tensor (or an int address) after checking that the
    tensor is a contiguous CUDA/HIP tensor holding exactly ``nbytes``."""
    if isinstance(t, int):
        return t
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor or an int device address")
    if not t.is_cuda:
        raise ValueError(f"{name}: tensor must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    got = t.numel() * t.element_size()
    if got != nbytes:
        raise ValueError(f"{name}: holds {got} bytes, the plan needs {nbytes}")
    return t.data_ptr()


def _view_ptr(t, rows: int, cols: int, ld: int, itemsize, name: str):
    """Device pointer of operand or output storage of ``rows`` rows of
    ``cols`` elements, ``ld`` elements apart.  Packed storage takes any
    contiguous tensor of the right size; otherwise ``t`` must be a 2-D view
    with unit column stride whose rows hold exactly ``cols`` elements and lie
    ``ld`` elements apart (in ``itemsize`` bytes per element)."""
    if ld == cols or isinstance(t, int):
        return _dev_ptr(t, int(rows * cols * itemsize), name)
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor")
    es = t.element_size()
    if (t.dim() != 2 or t.shape[0] != rows or t.shape[1] * es != cols * itemsize or
            (rows > 1 and t.stride(0) * es != ld * itemsize) or (t.shape[1] > 1 and t.stride(1) != 1)):
        raise ValueError(f"{name}: expected a ({rows}, {cols}) view with rows {ld} elements apart, "
                         f"got shape {tuple(t.shape)} strides {t.stride()}")
    return t.data_ptr()


def _operands(plan: Plan, A, B, D):
    return (_view_ptr(A, plan.a_rows, plan.a_cols, plan.lda, _ITEMSIZE[plan.a_dt], "A"),
            _view_ptr(B, plan.b_rows, plan.b_cols, plan.ldb, _ITEMSIZE[plan.b_dt], "B"),
            _view_ptr(D, plan.M, plan.N, plan.ldd, _ITEMSIZE[plan.d_dt], "D"))


def _stream_ptr(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def gemm_run(plan: Plan, A, B, D, beta: int = 0, stream=None) -> None:
    """Enqueue D = beta*D + A.B^T on ``stream`` (default: torch's current stream)."""
    a, b, d = _operands(plan, A, B, D)
    rc = load().gemm_run(plan.handle, a, b, d, int(beta), _stream_ptr(stream))
    if rc != 0:
        raise MswzError(rc, "gemm_run")


def gemm_run_ws(plan: Plan, A, B, D, workspace, beta: int = 0, stream=None) -> None:
    """gemm_run with a device workspace (a contiguous GPU tensor of at least
    ``plan.workspace_bytes()`` bytes; its prior contents do not matter).
    Plans without a workspace path run as gemm_run."""
    a, b, d = _operands(plan, A, B, D)
    need = plan.workspace_bytes()
    if isinstance(workspace, int):
        w, wb = workspace, need
    else:
        import torch
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace: expected a contiguous GPU tensor")
        w, wb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        if wb < need:
            raise ValueError(f"workspace: holds {wb} bytes, the plan needs {need}")
    rc = load().gemm_run_ws(plan.handle, a, b, d, int(beta), w, int(wb), _stream_ptr(stream))
    if rc != 0:
        raise MswzError(rc, "gemm_run_ws")


def gemm_run_ws_noalloc(plan: Plan, A, B, D, beta: int = 0, stream=None) -> None:
    """gemm_run_ws with the library's own static scratch instead of a caller
    workspace (for callers that cannot allocate); calls that overlap on one
    GPU race on that scratch."""
    a, b, d = _operands(plan, A, B, D)
    rc = load().gemm_run_ws_noalloc(plan.handle, a, b, d, int(beta), _stream_ptr(stream))
    if rc != 0:
        raise MswzError(rc, "gemm_run_ws_noalloc")


def gemm_noalloc_scratch_bytes() -> int:
    """Bytes of the per-GPU scratch gemm_run_ws_noalloc uses."""
    return int(load().gemm_noalloc_scratch_bytes())


def gemm_run_blockscaled(plan: Plan, A, B, SFA, SFB, D, beta: int = 0, stream=None) -> None:
    """Enqueue the block-scaled product on ``stream``."""
    sfa_b, sfb_b = plan.sf_bytes()
    a, b, d = _operands(plan, A, B, D)
    sa = _dev_ptr(SFA, sfa_b, "SFA")
    sb = _dev_ptr(SFB, sfb_b, "SFB")
    rc = load().gemm_run_blockscaled(plan.handle, a, b, sa, sb, d, int(beta), _stream_ptr(stream))
    if rc != 0:
        raise MswzError(rc, "gemm_run_blockscaled")


def _mask_ptr(t, nbits: int, name: str):
    """Device pointer of a bit mask of ``nbits`` bits (ceil(nbits/32) 32-bit
    words, bit x of word x // 32), or None."""
    if t is None:
        return None
    return _dev_ptr(t, 4 * ((nbits + 31) // 32), name)


def gemm_run_opts(plan: Plan, A, B, D, beta: int = 0, SFA=None, SFB=None, neg_a=False, neg_b=False,
                  sat_d=False, row_mask=None, col_zero=None, pred=True, stream=None) -> None:
    """gemm_run / gemm_run_blockscaled with the per-call options of gemm_opts:
    negated operands, saturated D, a row mask (rows left untouched), a column
    mask (columns whose product is zero) and a predicate.  Masks are GPU
    tensors of ceil(M/32) / ceil(N/32) 32-bit words (int32 or uint32)."""
    a, b, d = _operands(plan, A, B, D)
    sa = sb = None
    if plan.scale_vec_len:
        sfa_b, sfb_b = plan.sf_bytes()
        sa, sb = _dev_ptr(SFA, sfa_b, "SFA"), _dev_ptr(SFB, sfb_b, "SFB")
    elif SFA is not None or SFB is not None:
        raise ValueError("dense plan: SFA and SFB must be None")
    o = GemmOpts(int(bool(neg_a)), int(bool(neg_b)), int(bool(sat_d)),
                 _mask_ptr(row_mask, plan.M, "row_mask"), _mask_ptr(col_zero, plan.N, "col_zero"),
                 int(bool(pred)))
    rc = load().gemm_run_opts(plan.handle, a, b, sa, sb, d, int(beta), ctypes.byref(o), _stream_ptr(stream))
    if rc != 0:
        raise MswzError(rc, "gemm_run_opts")


def desc_address(r, w, ldo, sdo, mode, major="k", origin=0) -> int:
    """The library's shared-descriptor walk (physical byte address of word w of row r)."""
    return int(load().mswz_desc_address(int(r), int(w), int(ldo), int(sdo), int(mode),
                                        _code(major, MAJORS, "major"), int(origin)))


def desc_check(ldo, sdo, mode, origin=0) -> int:
    return int(load().mswz_desc_check(int(ldo), int(sdo), int(mode), int(origin)))


def tile_offset(row, chunk) -> int:
    """Byte offset of 16-byte chunk ``chunk`` of row ``row`` in the kernels' LDS tile."""
    return int(load().mswz_tile_offset(int(row), int(chunk)))


#: access patterns of lds_lanes (include/mswz_gemm.h, MSWZ_LDS_*)
LDS_PATTERNS = {"dma_k": 1, "dma_mn": 2, "frag_k16": 3, "frag_mn16": 4, "frag_e4m3": 5, "frag_pad": 6,
                "frag_e4m3_mixed": 7, "frag_e2m1": 8, "scale_grp": 9, "scale_dma": 10, "epi_write": 11,
                "epi_read": 12, "frag_e4m3_fp4": 13, "scale_grp_wide": 14, "scale_dma_wide": 15,
                "scale_dma_wide_nat": 16, "scale_fp4_wide": 17, "scale_dma_mn": 18, "scale_grp_mn": 19,
                "scale_fp4_mn": 20}


def lds_lanes(pattern: str, p0: int = 0, p1: int = 0) -> list[int]:
    """The 256x256 kernel's per-lane LDS offsets for one access pattern (see
    mswz_lds_lanes in include/mswz_gemm.h); 64 or 128 values."""
    buf = (ctypes.c_uint32 * 128)()
    n = load().mswz_lds_lanes(LDS_PATTERNS[pattern], int(p0), int(p1), buf, 128)
    if n < 0:
        raise MswzError(n, "mswz_lds_lanes")
    return list(buf[:n])
