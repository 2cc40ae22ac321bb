"""ctypes binding of libgemm_rs.so (include/gemm_rs.h).

Argument marshalling only: every step of the operation runs in the HIP
kernels behind the C ABI.  Tensors are passed as device pointers
(``tensor.data_ptr()``) and the stream as its ``hipStream_t`` handle.  If
the shared library has not been built, loading raises: there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libgemm_rs.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "gemm_rs.h")
HEADERS = [HEADER, os.path.join(os.path.dirname(_PKG), "include", "gemm_ag.h")]

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_HIP = -3
ERR_TIMEOUT = -4
ERR_PROTOCOL = -5
ERR_SCRATCH = -6

BF16, F32 = 0, 1
ORDER_FLAT, ORDER_TWO_LEVEL = 0, 1
SWIZZLE_REMOTE_FIRST, SWIZZLE_SELF_FIRST, SWIZZLE_IDENTITY, SWIZZLE_TILE_INTERLEAVED = 0, 1, 2, 3
STAGING_F32, STAGING_BF16 = 0, 1
RUN_GEMM, RUN_REDUCE, KEEP_FLAGS, TRACE_TILES, OVERLAP_REDUCE = 1, 2, 4, 8, 16
LAST_ARRIVER = 32
RUN_ALL = RUN_GEMM | RUN_REDUCE
AG_RUN_COPY, AG_RUN_GEMM, AG_FUSED, AG_EXPECT_NEXT = 1, 2, 4, 8
AG_RUN_ALL = AG_RUN_COPY | AG_RUN_GEMM


class gemm_rs_desc_t(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("W", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
        ("group_m", ctypes.c_int32), ("order", ctypes.c_int32),
        ("groups", ctypes.c_int32), ("swizzle", ctypes.c_int32),
        ("has_c", ctypes.c_int32), ("materialize_sub", ctypes.c_int32),
        ("ldc", ctypes.c_int64), ("timeout_ms", ctypes.c_uint32),
        ("staging_dtype", ctypes.c_uint32), ("interleave", ctypes.c_int32),
    ]


class gemm_rs_info_t(ctypes.Structure):
    _fields_ = [
        ("Mc", ctypes.c_int64),
        ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
        ("tiles_m", ctypes.c_int32), ("tiles_n", ctypes.c_int32),
        ("T", ctypes.c_int32), ("group_m", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64),
        ("staging", ctypes.c_void_p), ("flags", ctypes.c_void_p),
        ("sub", ctypes.c_void_p), ("sub_flags", ctypes.c_void_p),
        ("trace", ctypes.c_void_p),
        ("staging_bytes", ctypes.c_int64), ("flags_bytes", ctypes.c_int64),
        ("sub_bytes", ctypes.c_int64), ("sub_flags_bytes", ctypes.c_int64),
        ("slot_elems", ctypes.c_int64),
    ]


class gemm_ag_desc_t(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("W", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
        ("group_m", ctypes.c_int32), ("timeout_ms", ctypes.c_uint32), ("pad", ctypes.c_uint32),
    ]


class gemm_ag_info_t(ctypes.Structure):
    _fields_ = [
        ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
        ("tiles_m", ctypes.c_int32), ("tiles_n", ctypes.c_int32),
        ("group_m", ctypes.c_int32), ("epoch", ctypes.c_uint32),
        ("gathered", ctypes.c_void_p), ("signals", ctypes.c_void_p),
        ("gathered_bytes", ctypes.c_int64),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library; raise if it is missing (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            "libgemm_rs.so is not built (%s); run "
            "`python -m tensor_gemm_reduce_lds_amd.build`" % path)
    # One HIP runtime per process: torch ships its own libamdhip64, and the
    # device pointers and streams it hands out are only valid in that
    # instance.  Loading torch first makes this library bind to it instead
    # of pulling a second runtime from /opt/rocm.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32
    lib.gemm_rs_plan.argtypes = [ctypes.POINTER(gemm_rs_desc_t), ctypes.POINTER(vp)]
    lib.gemm_rs_run.argtypes = [vp, vp, vp, vp, ctypes.c_float, ctypes.c_float,
                                vp, vp, u32]
    lib.gemm_rs_run_noalloc.argtypes = [ctypes.POINTER(gemm_rs_desc_t), vp, vp, vp,
                                        ctypes.c_float, ctypes.c_float, vp, vp, u32, vp]
    lib.gemm_rs_destroy.argtypes = [vp]
    lib.gemm_rs_query.argtypes = [vp, ctypes.POINTER(gemm_rs_info_t)]
    lib.gemm_rs_tile_order.argtypes = [vp, vp]
    lib.gemm_rs_status.argtypes = [vp, vp, ctypes.POINTER(i32)]
    lib.gemm_rs_strerror.argtypes = [ctypes.c_int]
    lib.gemm_rs_strerror.restype = ctypes.c_char_p
    lib.gemm_ag_plan.argtypes = [ctypes.POINTER(gemm_ag_desc_t), ctypes.POINTER(vp)]
    lib.gemm_ag_run.argtypes = [vp, vp, vp, vp, vp, u32]
    lib.gemm_ag_query.argtypes = [vp, ctypes.POINTER(gemm_ag_info_t)]
    lib.gemm_ag_status.argtypes = [vp, vp, ctypes.POINTER(i32)]
    lib.gemm_ag_destroy.argtypes = [vp]
    for f in ("gemm_rs_plan", "gemm_rs_run", "gemm_rs_run_noalloc", "gemm_rs_destroy",
              "gemm_rs_query",
              "gemm_rs_tile_order", "gemm_rs_status", "gemm_ag_plan", "gemm_ag_run",
              "gemm_ag_query", "gemm_ag_status", "gemm_ag_destroy"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def header_functions(paths=None):
    """Names of the functions the public headers declare."""
    names = set()
    for path in paths or HEADERS:
        text = open(path).read()
        names.update(re.findall(r"GEMM_RS_API\s+[\w\s\*]+?\b(gemm_(?:rs|ag)_\w+)\s*\(", text))
    return sorted(names)


class GemmRsError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s: %s (%d)" % (where, gemm_rs_strerror(code), code))


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_desc(M, N, K, W, dtype=BF16, tile_m=0, tile_n=0, group_m=0,
              order=ORDER_FLAT, groups=1, swizzle=SWIZZLE_REMOTE_FIRST,
              has_c=0, ldc=0, materialize_sub=0, timeout_ms=0,
              staging_dtype=0, interleave=0) -> gemm_rs_desc_t:
    return gemm_rs_desc_t(M=M, N=N, K=K, W=W, dtype=dtype, tile_m=tile_m,
                          tile_n=tile_n, group_m=group_m, order=order,
                          groups=groups, swizzle=swizzle, has_c=int(has_c),
                          materialize_sub=int(materialize_sub), ldc=ldc,
                          timeout_ms=timeout_ms, staging_dtype=staging_dtype,
                          interleave=interleave)


# ---- the C entry points, same names --------------------------------------
def gemm_rs_plan(desc: Optional[gemm_rs_desc_t]):
    """Returns (status, plan handle or None)."""
    h = ctypes.c_void_p()
    rc = load_library().gemm_rs_plan(
        None if desc is None else ctypes.byref(desc), ctypes.byref(h))
    return rc, h.value


def gemm_rs_run(plan, A, B, C, alpha, beta, out, stream=None, run_flags=RUN_ALL) -> int:
    return load_library().gemm_rs_run(plan, _ptr(A), _ptr(B), _ptr(C), alpha, beta,
                                      _ptr(out), _stream_handle(stream), run_flags)


def gemm_rs_run_noalloc(desc: Optional[gemm_rs_desc_t], A, B, C, alpha, beta, out,
                        stream=None, run_flags=RUN_ALL, status=None) -> int:
    return load_library().gemm_rs_run_noalloc(
        None if desc is None else ctypes.byref(desc), _ptr(A), _ptr(B), _ptr(C), alpha, beta,
        _ptr(out), _stream_handle(stream), run_flags, _ptr(status))


def gemm_rs_destroy(plan) -> int:
    return load_library().gemm_rs_destroy(plan)


def gemm_rs_query(plan):
    """Returns (status, gemm_rs_info_t)."""
    info = gemm_rs_info_t()
    rc = load_library().gemm_rs_query(plan, ctypes.byref(info))
    return rc, info


def gemm_rs_tile_order(plan, host_trace) -> int:
    """host_trace: a writable int32 numpy array of W*T entries."""
    return load_library().gemm_rs_tile_order(plan, host_trace.ctypes.data)


def gemm_rs_status(plan, stream=None):
    """Returns (status, [code, rank, tile, value])."""
    detail = (ctypes.c_int32 * 4)()
    rc = load_library().gemm_rs_status(plan, _stream_handle(stream), detail)
    return rc, list(detail)


def gemm_rs_strerror(code: int) -> str:
    return load_library().gemm_rs_strerror(code).decode()


# ---- small owning wrapper -------------------------------------------------
class Plan:
    """Owns one plan handle; raises GemmRsError on a non-OK status."""

    def __init__(self, **desc_fields):
        self.desc = make_desc(**desc_fields)
        rc, h = gemm_rs_plan(self.desc)
        if rc != OK:
            raise GemmRsError(rc, "gemm_rs_plan")
        self.handle = h
        rc, self.info = gemm_rs_query(h)
        if rc != OK:
            gemm_rs_destroy(h)
            raise GemmRsError(rc, "gemm_rs_query")

    def run(self, A, B, C, alpha, beta, out, stream=None, run_flags=RUN_ALL):
        rc = gemm_rs_run(self.handle, A, B, C, alpha, beta, out, stream, run_flags)
        if rc != OK:
            raise GemmRsError(rc, "gemm_rs_run")

    def status(self, stream=None):
        return gemm_rs_status(self.handle, stream)

    def tile_order(self):
        import numpy as np
        tr = np.empty(self.desc.W * self.info.T, dtype=np.int32)
        rc = gemm_rs_tile_order(self.handle, tr)
        if rc != OK:
            raise GemmRsError(rc, "gemm_rs_tile_order")
        return tr

    def close(self):
        if self.handle is not None:
            gemm_rs_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- all-gather + GEMM (include/gemm_ag.h), same names ------------------------
def make_ag_desc(M, N, K, W, tile_m=0, tile_n=0, group_m=0, timeout_ms=0,
                 pad=0) -> gemm_ag_desc_t:
    return gemm_ag_desc_t(M=M, N=N, K=K, W=W, tile_m=tile_m, tile_n=tile_n,
                          group_m=group_m, timeout_ms=timeout_ms, pad=pad)


def gemm_ag_plan(desc: Optional[gemm_ag_desc_t]):
    """Returns (status, plan handle or None)."""
    h = ctypes.c_void_p()
    rc = load_library().gemm_ag_plan(None if desc is None else ctypes.byref(desc),
                                     ctypes.byref(h))
    return rc, h.value


def gemm_ag_run(plan, X, B, out, stream=None, run_flags=AG_RUN_ALL | AG_FUSED) -> int:
    return load_library().gemm_ag_run(plan, _ptr(X), _ptr(B), _ptr(out),
                                      _stream_handle(stream), run_flags)


def gemm_ag_query(plan):
    """Returns (status, gemm_ag_info_t)."""
    info = gemm_ag_info_t()
    rc = load_library().gemm_ag_query(plan, ctypes.byref(info))
    return rc, info


def gemm_ag_status(plan, stream=None):
    """Returns (status, [code, rank, tile-row, 0])."""
    detail = (ctypes.c_int32 * 4)()
    rc = load_library().gemm_ag_status(plan, _stream_handle(stream), detail)
    return rc, list(detail)


def gemm_ag_destroy(plan) -> int:
    return load_library().gemm_ag_destroy(plan)


class AgPlan:
    """Owns one all-gather + GEMM plan; raises GemmRsError on a non-OK status."""

    def __init__(self, **desc_fields):
        self.desc = make_ag_desc(**desc_fields)
        rc, h = gemm_ag_plan(self.desc)
        if rc != OK:
            raise GemmRsError(rc, "gemm_ag_plan")
        self.handle = h

    @property
    def info(self) -> gemm_ag_info_t:
        rc, info = gemm_ag_query(self.handle)
        if rc != OK:
            raise GemmRsError(rc, "gemm_ag_query")
        return info

    def run(self, X, B, out, stream=None, run_flags=AG_RUN_ALL | AG_FUSED):
        rc = gemm_ag_run(self.handle, X, B, out, stream, run_flags)
        if rc != OK:
            raise GemmRsError(rc, "gemm_ag_run")

    def status(self, stream=None):
        return gemm_ag_status(self.handle, stream)

    def close(self):
        if self.handle is not None:
            gemm_ag_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
