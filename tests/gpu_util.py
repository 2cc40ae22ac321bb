"""Helpers for the GPU tests: upload seeded inputs, run a plan through the
C ABI, read back plan-owned device buffers with plain hipMemcpy."""
from __future__ import annotations

import ctypes
import sys

import numpy as np

import oracle as O
from tensor_gemm_reduce_lds_amd import gemm_rs as G
from tensor_gemm_reduce_lds_amd import inputs as I

_hip = None


def hip():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    return _hip


H2D, D2H = 1, 2


def d2h(ptr: int, nbytes: int, dtype) -> np.ndarray:
    out = np.empty(nbytes // np.dtype(dtype).itemsize, dtype=dtype)
    assert hip().hipMemcpy(out.ctypes.data, ptr, nbytes, D2H) == 0
    return out


def h2d(ptr: int, arr: np.ndarray, offset_bytes: int = 0) -> None:
    arr = np.ascontiguousarray(arr)
    assert hip().hipMemcpy(ptr + offset_bytes, arr.ctypes.data, arr.nbytes, H2D) == 0


def say(*a):
    """Name the case before each GPU step (flushed)."""
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(x: dict, w: I.Workload):
    import torch
    dev = torch.device("cuda", 0)

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev)
        return torch.from_numpy(a).to(dev)

    return {"A": up(x["A"]), "B": up(x["B"]), "C": up(x["C"])}


def new_out(w: I.Workload):
    import torch
    dt = torch.int16 if w.dtype == "bf16" else torch.float32
    return torch.empty((w.M, w.N), dtype=dt, device="cuda:0")


def out_to_f64(out, w: I.Workload) -> np.ndarray:
    a = out.cpu().numpy()
    if w.dtype == "bf16":
        return O.bf16_bits_to_f64(a.view(np.uint16))
    return a.astype(np.float64)


def out_bits(out) -> np.ndarray:
    a = out.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a.view(np.uint32)


def desc_fields(w: I.Workload, **over):
    f = dict(M=w.M, N=w.N, K=w.K, W=w.W,
             dtype=G.BF16 if w.dtype == "bf16" else G.F32,
             tile_m=w.tile_m, tile_n=w.tile_n,
             order=G.ORDER_TWO_LEVEL if w.order == "two_level" else G.ORDER_FLAT,
             groups=w.groups, has_c=int(w.has_c), ldc=w.ldc)
    f.update(over)
    return f


def oracle_kw(w: I.Workload, plan: G.Plan = None):
    return dict(dtype=O.BF16 if w.dtype == "bf16" else O.F32, alpha=w.alpha,
                beta=w.beta, ldc=w.ldc,
                order=O.TWO_LEVEL if w.order == "two_level" else O.FLAT,
                groups=w.groups)


def geometry(w: I.Workload, plan: G.Plan) -> O.Geometry:
    d = plan.desc
    return O.Geometry(w.M, w.N, w.K, w.W, plan.info.tile_m, plan.info.tile_n,
                      group_m=plan.info.group_m, swizzle=d.swizzle,
                      order=d.order, groups=d.groups, interleave=d.interleave,
                      staging_dtype=d.staging_dtype)


def sync():
    import torch
    torch.cuda.synchronize()


def run_checked(plan: G.Plan, dev, w: I.Workload, out, run_flags=G.RUN_ALL,
                alpha=None, beta=None):
    import torch
    alpha = w.alpha if alpha is None else alpha
    beta = w.beta if beta is None else beta
    s = torch.cuda.current_stream()
    plan.run(dev["A"], dev["B"], dev["C"], alpha, beta, out, s, run_flags)
    rc, detail = plan.status(s)
    assert rc == G.OK, (rc, detail)


def flags(plan: G.Plan) -> np.ndarray:
    W, T = plan.desc.W, plan.info.T
    return d2h(plan.info.flags, plan.info.flags_bytes, np.uint32).reshape(W, T)


def staging_slots(plan: G.Plan, geom: O.Geometry, dtype=np.float32) -> np.ndarray:
    """The used part of every staging slot, as [W(d)][W(r)][Mc][N] (slots
    are geom.slot elements apart; the rest of a slot is never written)."""
    W, used = geom.W, geom.Mc * geom.N
    assert plan.info.slot_elems == geom.slot
    assert plan.info.staging_bytes == W * W * geom.slot * np.dtype(dtype).itemsize
    st = d2h(plan.info.staging, plan.info.staging_bytes, dtype).reshape(W * W, geom.slot)
    return st[:, :used].reshape(W, W, geom.Mc, geom.N)


def put_staging(plan: G.Plan, geom: O.Geometry, S: np.ndarray) -> None:
    """Write S[d][r][Mc][N] into the staging slots (host to device)."""
    W, used = geom.W, geom.Mc * geom.N
    assert plan.info.slot_elems == geom.slot
    full = np.zeros((W * W, geom.slot), dtype=S.dtype)
    full[:, :used] = S.reshape(W * W, used)
    h2d(plan.info.staging, full)


def staging_rows(plan: G.Plan, geom: O.Geometry, d: int, r: int, il0: int, n: int):
    """Rows il0..il0+n of staging slot (d, r) as float32 [n][N]."""
    off = geom.staging_offset(d, r, d * geom.Mc + il0, 0) * 4
    return d2h(plan.info.staging + off, n * geom.N * 4, np.float32).reshape(n, geom.N)


def check_tolerance(got: np.ndarray, ref: np.ndarray, dtype: str):
    """The parity bar: bf16 out: max |g-r|/max(1,|r|) <= 2e-2 and
    rel-Frobenius <= 2e-3; fp32 out: both <= 1e-4."""
    mx = O.max_norm_err(got, ref)
    rf = O.rel_frobenius(got, ref)
    if dtype == "bf16":
        assert mx <= 2e-2, mx
        assert rf <= 2e-3, rf
    else:
        assert mx <= 1e-4, mx
        assert rf <= 1e-4, rf
    return mx, rf


def check_bf16_staging(got, ref, mag):
    """Bar for bfloat16 staging.  Elementwise, the rounding bound: each
    staged partial and the output are rounded to 8 significant bits, so
    |got - ref| <= 2^-8 |ref| + 2^-8 (1 + 2^-8) sum_r |D_r|, plus 1e-4
    sum_r |D_r| for the float accumulation and summation order.  A bound
    relative to |ref| alone cannot hold: when the W partials cancel, their
    rounding errors do not.  In aggregate, rel-Frobenius <= 3e-3: rounding
    each of W independent partials to 8 bits adds about the output
    rounding's own error (~1.7e-3 each for N(0,1) data, ~2.4e-3 together)."""
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + (2.0 ** -8 * (1 + 2.0 ** -8) + 1e-4) * mag + 1e-6
    assert np.all(err <= bound), float((err / bound).max())
    rf = O.rel_frobenius(got, ref)
    assert rf <= 3e-3, rf
    return float((err / bound).max()), rf
