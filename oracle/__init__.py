"""CPU oracle for the fused GEMM + reduce-scatter path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
calls it and shares no code with it: the index arithmetic here (tile map,
swizzle, staging offsets) and the numerics in ``gemm_rs_oracle.c`` are
written separately from the kernels, from the pages.

Contents
--------
* ``validate``       descriptor rules (which problems are invalid, which are
                     valid but unsupported).
* ``Geometry``       the tile -> chunk map and the per-rank tile order
                     (swizzle), plus staging offsets and flag predictions.
* ``staging_slot_elems``  the library's staging slot size (a restated
                     layout rule, like the UNSUPPORTED limits in
                     ``validate``).
* ``reference_*``    the fp64 result (parity target), in C.
* ``emulate_*``      a float pipeline emulation, bit-exact only where the
                     per-rank epilogue values are exact in float.
* ``reduce_emulate`` the ordered float sum alone, for host-written staging.
* ``bf16_rne``       float -> bfloat16 round-to-nearest-even.

Pins: every function here is checked in ``tests/test_oracle_pins.py``
against brute force, closed forms, library routines (numpy matmul, torch's
bfloat16 cast) or values the pages print.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

# ---- codes: the same numbers the C ABI uses (an interface, so they agree) --
OK, INVALID_ARG, UNSUPPORTED, HIP_ERROR, TIMEOUT, PROTOCOL = 0, -1, -2, -3, -4, -5
BF16, F32 = 0, 1
FLAT, TWO_LEVEL = 0, 1
REMOTE_FIRST, SELF_FIRST, IDENTITY, TILE_INTERLEAVED = 0, 1, 2, 3
STAGING_F32, STAGING_BF16 = 0, 1
RUN_GEMM, RUN_REDUCE, KEEP_FLAGS, TRACE_TILES = 1, 2, 4, 8
MAX_W = 64
K_STEP = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_rs_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_gemm_rs.so")
_lib = None


# --------------------------------------------------------------------------
# descriptor validation
# --------------------------------------------------------------------------
def validate(M, N, K, W, dtype, tile_m, tile_n, group_m=1, order=FLAT,
             groups=1, swizzle=REMOTE_FIRST, has_c=0, ldc=0,
             materialize_sub=0, supported_tiles: Optional[Sequence] = None,
             staging_dtype=STAGING_F32, interleave=0):
    """Return the status a plan must give for this descriptor.

    INVALID_ARG: the problem itself is ill-posed.  A reduce-scatter over W
    ranks hands each rank an equal block of M/W rows (page "flux精读",
    section 3 Design: the GEMM output is reduce-scattered across the TP
    group), so M % W != 0 is invalid; the two-level order needs W split into
    equal groups (page "flux实现：sm80 gemm+rs", section "2D Ring优化").
    UNSUPPORTED: a valid problem outside what the kernels implement: a tile
    shape not in ``supported_tiles``, N not a multiple of the tile width,
    K not a multiple of the 64-deep K step, a C row pitch that is not a
    multiple of 8 elements (16-byte rows), M, N or K of 2^31 or more,
    bfloat16 with K of 2^23 or more or N of 2^25 or more,
    a grid too large for 32-bit workgroup ids, or bfloat16 staging with
    float32 inputs or with the materialised two-level buffers.
    """
    ints = (M, N, K, W, dtype, tile_m, tile_n, group_m, order, groups,
            swizzle, has_c, ldc, materialize_sub, staging_dtype, interleave)
    if any(not isinstance(v, (int, np.integer)) for v in ints):
        return INVALID_ARG
    # K == 0 is the empty sum: every partial is 0, so out = beta*C
    if W < 1 or W > MAX_W or M < 1 or N < 1 or K < 0:
        return INVALID_ARG
    if M % W != 0:
        return INVALID_ARG
    if dtype not in (BF16, F32):
        return INVALID_ARG
    if group_m < 0 or tile_m < 0 or tile_n < 0:
        return INVALID_ARG
    if order not in (FLAT, TWO_LEVEL):
        return INVALID_ARG
    if order == TWO_LEVEL and (groups < 1 or W % groups != 0):
        return INVALID_ARG
    if swizzle not in (REMOTE_FIRST, SELF_FIRST, IDENTITY, TILE_INTERLEAVED):
        return INVALID_ARG
    # tiles per destination visit: 0 or 1 is one tile; more only means
    # something for the tile-interleaved order
    if interleave < 0 or (interleave > 1 and swizzle != TILE_INTERLEAVED):
        return INVALID_ARG
    if has_c not in (0, 1) or ldc < 0 or (has_c and ldc != 0 and ldc < N):
        return INVALID_ARG
    if materialize_sub not in (0, 1) or (materialize_sub and order != TWO_LEVEL):
        return INVALID_ARG
    if staging_dtype not in (STAGING_F32, STAGING_BF16):
        return INVALID_ARG
    if supported_tiles is not None and (tile_m, tile_n) not in set(
            tuple(t) for t in supported_tiles):
        return UNSUPPORTED
    if tile_m == 0 or tile_n == 0:
        return UNSUPPORTED
    if N % tile_n != 0 or K % K_STEP != 0:
        return UNSUPPORTED
    if has_c and ldc % 8 != 0:
        return UNSUPPORTED
    if staging_dtype == STAGING_BF16 and (dtype != BF16 or materialize_sub):
        return UNSUPPORTED
    if max(M, N, K) > 2**31 - 1:
        return UNSUPPORTED
    # bf16 kernel limit: 32-bit offsets inside one K step's operand windows
    if dtype == BF16 and (K >= 2**23 or N >= 2**25):
        return UNSUPPORTED
    tiles = -(-M // tile_m) * (N // tile_n)
    if tiles * W > 2**31 - 1:
        return UNSUPPORTED
    return OK


# --------------------------------------------------------------------------
# tile -> chunk map and swizzle
# --------------------------------------------------------------------------
def staging_slot_elems(Mc: int, N: int, elem_bytes: int) -> int:
    """Elements from one staging slot to the next.

    The library's staging layout, restated here so the tests can find a
    slot (not a rule of the pages, which leave the buffer layout open): a
    slot holds Mc x N partials, and once it holds 8 MiB or more its size is
    rounded up to a multiple of 512 KiB, the rest of it unused.
    """
    nbytes = Mc * N * elem_bytes
    if nbytes < 8 << 20:
        return Mc * N
    align = 512 << 10
    return -(-nbytes // align) * align // elem_bytes


class Geometry:
    """Tile grid, chunk ownership and per-rank tile order.

    The GEMM output [M, N] is cut into BM x BN tiles over the full grid; the
    communication unit is one tile, while the semantic chunk handed to a
    rank is M/W rows and need not match the tile shape (page "flux实现：sm80
    gemm+rs", section "gemmrs版本的swizzle如何编排", the ReduceScatterOp
    paragraph).  A tile can straddle two chunks: its rows are routed one by
    one, and its owner for scheduling is the chunk of its first row.
    """

    def __init__(self, M, N, K, W, tile_m, tile_n, group_m=1,
                 swizzle=REMOTE_FIRST, order=FLAT, groups=1, interleave=1,
                 staging_dtype=STAGING_F32):
        self.M, self.N, self.K, self.W = M, N, K, W
        self.BM, self.BN = tile_m, tile_n
        self.g = max(1, group_m)
        self.swizzle = swizzle
        self.q = max(1, interleave)
        self.order, self.groups = order, (groups if order == TWO_LEVEL else 1)
        self.Mc = M // W
        self.slot = staging_slot_elems(self.Mc, N, 2 if staging_dtype == STAGING_BF16 else 4)
        self.tiles_m = -(-M // tile_m)
        self.tiles_n = N // tile_n
        self.T = self.tiles_m * self.tiles_n

    # -- map --------------------------------------------------------------
    def chunk_of_row(self, i: int) -> int:
        """d(i): the rank that receives global row i."""
        return i // self.Mc

    def tile_rows(self, tm: int):
        """Half-open row range [lo, hi) of tile-row tm (last one ragged)."""
        return tm * self.BM, min(self.M, (tm + 1) * self.BM)

    def owner(self, tm: int) -> int:
        """Scheduling owner of tile-row tm: the chunk of its first row."""
        return self.chunk_of_row(tm * self.BM)

    def straddling_tile_rows(self) -> List[int]:
        out = []
        for tm in range(self.tiles_m):
            lo, hi = self.tile_rows(tm)
            if self.chunk_of_row(lo) != self.chunk_of_row(hi - 1):
                out.append(tm)
        return out

    def staging_offset(self, d: int, r: int, i: int, j: int) -> int:
        """Element offset of (row i, col j) from rank r in slot (d, r).

        Staging is destination-major: slot (d, r) is the piece of rank r's
        output that rank d receives (the per-destination reduce-scatter
        buffer the epilogue writes into, page "flux实现：sm80 gemm+rs",
        section "cutlass自定义epilogue–sm80", the StoreD paragraph), rows
        [Mc][N] row-major from the slot's start; slots are ``self.slot``
        elements apart (``staging_slot_elems``).
        """
        return (d * self.W + r) * self.slot + (i - d * self.Mc) * self.N + j

    def sub_offset(self, d: int, g: int, i: int, j: int) -> int:
        """Element offset of (row i, col j) of group g's partial sum in the
        materialised two-level buffer sub[d][G][Mc][N]: for destination d,
        one Mc x N block per group of ranks (the sub-node partial buffer of
        page "flux实现：sm80 gemm+rs", section "2D Ring优化")."""
        return ((d * self.groups + g) * self.Mc + (i - d * self.Mc)) * self.N + j

    # -- swizzle ----------------------------------------------------------
    def dest(self, r: int, s: int) -> int:
        """Destination chunk of rank r at step s.

        REMOTE_FIRST: remote chunks first, the local chunk last, and each
        rank starting at a different destination so no two ranks write the
        same chunk in the same step (page "flux实现：sm80 gemm+rs", section
        "gemmrs版本的swizzle如何编排"; page "通信 overlap 实现", Flux tile
        fusion section: rank-offset tile coordinates).
        SELF_FIRST: the rank-offset order as described on page "flux精读",
        section 4.1 (rank 1 writes chunks 1..7 then 0, rank 0 writes 0..7).
        IDENTITY: every rank in the same order 0..W-1 (the contention case
        the swizzle exists to avoid).
        TILE_INTERLEAVED: the remote-first rotation, visited one tile at a
        time (see ``seq``).
        """
        if self.swizzle in (REMOTE_FIRST, TILE_INTERLEAVED):
            return (r + 1 + s) % self.W
        if self.swizzle == SELF_FIRST:
            return (r + s) % self.W
        return s

    def chunk_tile_rows(self, d: int) -> List[int]:
        return [tm for tm in range(self.tiles_m) if self.owner(tm) == d]

    def chunk_tiles(self, d: int) -> List[int]:
        """Tiles of chunk d in their within-chunk order: sorted by
        (tile-row group, tile column, tile row) with groups of ``group_m``
        tile-rows counted from the chunk's first tile-row.  Tile id
        t = tm * tiles_n + tn."""
        rows = self.chunk_tile_rows(d)
        if not rows:
            return []
        tm0 = rows[0]
        tiles = [(tm, tn) for tm in rows for tn in range(self.tiles_n)]
        tiles.sort(key=lambda x: ((x[0] - tm0) // self.g, x[1], x[0]))
        return [tm * self.tiles_n + tn for tm, tn in tiles]

    def seq(self, r: int) -> List[int]:
        """Tile order of rank r.

        Chunk-major orders (REMOTE_FIRST, SELF_FIRST, IDENTITY): chunk by
        chunk in dest order, each chunk's tiles in their within-chunk order.
        TILE_INTERLEAVED (a reading of the tile-interleaved variant of the
        remote-first order: every destination in flight at once instead of
        one chunk per step): rank r visits the destinations dest(r, 0..W-1)
        in turn and takes the next q = ``interleave`` tiles of each on every
        visit (round j takes the chunk's tiles [j*q, (j+1)*q)); a chunk with
        fewer left gives what remains, a used-up chunk is skipped.  q = 1 is
        one tile per visit; q at least the largest chunk's tile count is the
        chunk-major remote-first order."""
        if self.swizzle != TILE_INTERLEAVED:
            out = []
            for s in range(self.W):
                out.extend(self.chunk_tiles(self.dest(r, s)))
            return out
        lists = [self.chunk_tiles(self.dest(r, s)) for s in range(self.W)]
        q = self.q
        rounds = -(-max(len(x) for x in lists) // q)
        out = []
        for j in range(rounds):
            for s in range(self.W):
                out.extend(lists[s][j * q:(j + 1) * q])
        return out

    def seq_table(self) -> np.ndarray:
        return np.array([self.seq(r) for r in range(self.W)], dtype=np.int32)

    def trace(self) -> np.ndarray:
        """Tile computed by workgroup b of the W*T grid: rank b % W, its
        (b // W)-th tile."""
        tab = self.seq_table()
        b = np.arange(self.W * self.T)
        return tab[b % self.W, b // self.W].astype(np.int32)

    # -- flags --------------------------------------------------------------
    def predict_flags(self, run_flags_history: Sequence[int]) -> np.ndarray:
        """flag[r][t] after a sequence of runs from the all-zero state.

        A producer sets its tile's flag to 1 after the tile's stores; the
        consumer waits for 1 and then puts it back to 0 (consume and reset,
        like the consumer side of the device barrier on page "flux实现：sm80
        gemm+rs", section "device side barrier"), unless KEEP_FLAGS asks it
        to leave them set.  Signals are 32-bit words allocated once (page
        "flux精读", section 4.2)."""
        f = np.zeros((self.W, self.T), dtype=np.uint32)
        for rf in run_flags_history:
            if rf & RUN_GEMM:
                f[:] = 1
            if rf & RUN_REDUCE and not rf & KEEP_FLAGS:
                f[:] = 0
        return f


# --------------------------------------------------------------------------
# C numerics
# --------------------------------------------------------------------------
def build(force: bool = False) -> str:
    """Compile gemm_rs_oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off",
                        "-fno-fast-math", "-shared", "-fPIC", "-std=c11",
                        "-Wall", "-o", tmp, _SRC], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    lib = ctypes.CDLL(build())
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
    common = [i64, i64, i64, i32, i32, vp, vp, vp, i32, i64, dbl, dbl]
    lib.oracle_partial_rows.argtypes = common + [i32, i64, i64, vp]
    lib.oracle_reference_rows.argtypes = common + [i32, i32, i64, i64, vp]
    lib.oracle_emulate_rows.argtypes = common + [i32, i32, i64, i64, i32, i32, vp]
    lib.oracle_reference_elems.argtypes = common + [i32, i32, i64, vp, vp, vp]
    lib.oracle_reduce_emulate.argtypes = [i32, i32, i32, i64, vp, i32, vp]
    lib.oracle_bf16_rne_array.argtypes = [i64, vp, vp]
    lib.oracle_bf16_rne_array.restype = None
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    for f in (lib.oracle_partial_rows, lib.oracle_reference_rows,
              lib.oracle_emulate_rows, lib.oracle_reference_elems,
              lib.oracle_reduce_emulate):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_threads(n: int) -> None:
    """OpenMP threads for the oracle's next calls (timing only)."""
    _load().oracle_set_threads(int(n))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _prep(A, B, C, dtype):
    want = np.uint16 if dtype == BF16 else np.float32
    A = np.ascontiguousarray(A, dtype=want)
    B = np.ascontiguousarray(B, dtype=want)
    C = None if C is None else np.ascontiguousarray(C, dtype=want)
    return A, B, C


def _common(A, B, C, dtype, alpha, beta, ldc):
    A, B, C = _prep(A, B, C, dtype)
    W, M, K = A.shape
    N = B.shape[2]
    assert B.shape == (W, K, N)
    has_c = 0 if C is None else 1
    if has_c:
        need = N if ldc == 0 else (M - 1) * ldc + N
        assert C.size >= need
    args = (M, N, K, W, dtype, _ptr(A), _ptr(B), _ptr(C), has_c, ldc,
            float(alpha), float(beta))
    return (A, B, C), args, (W, M, N, K)


def partial_rows(A, B, C=None, *, dtype, alpha=1.0, beta=0.0, ldc=0, r,
                 row_lo=0, row_hi=None):
    """Epilogue value D_r of rank r for rows [row_lo, row_hi), fp64."""
    keep, args, (W, M, N, K) = _common(A, B, C, dtype, alpha, beta, ldc)
    row_hi = M if row_hi is None else row_hi
    out = np.empty((row_hi - row_lo, N), dtype=np.float64)
    rc = _load().oracle_partial_rows(*args, r, row_lo, row_hi, _ptr(out))
    assert rc == 0, rc
    return out


def reference_rows(A, B, C=None, *, dtype, alpha=1.0, beta=0.0, ldc=0,
                   order=FLAT, groups=1, row_lo=0, row_hi=None):
    """Reduced result rows [row_lo, row_hi), fp64, no rounding."""
    keep, args, (W, M, N, K) = _common(A, B, C, dtype, alpha, beta, ldc)
    row_hi = M if row_hi is None else row_hi
    out = np.empty((row_hi - row_lo, N), dtype=np.float64)
    rc = _load().oracle_reference_rows(*args, order, groups, row_lo, row_hi,
                                       _ptr(out))
    assert rc == 0, rc
    return out


def emulate_rows(A, B, C=None, *, dtype, alpha=1.0, beta=0.0, ldc=0,
                 order=FLAT, groups=1, row_lo=0, row_hi=None,
                 staging_dtype=STAGING_F32):
    """Float-pipeline emulation of rows [row_lo, row_hi): uint16 bfloat16
    bits for dtype BF16, float32 for F32.  With STAGING_BF16 each rank's
    float epilogue value is rounded to bfloat16 (nearest even) before the
    ordered float sum, as a bfloat16 staging slot holds it."""
    keep, args, (W, M, N, K) = _common(A, B, C, dtype, alpha, beta, ldc)
    row_hi = M if row_hi is None else row_hi
    out_kind = 0 if dtype == BF16 else 1
    out = np.empty((row_hi - row_lo, N),
                   dtype=np.uint16 if out_kind == 0 else np.float32)
    rc = _load().oracle_emulate_rows(*args, order, groups, row_lo, row_hi,
                                     out_kind, int(staging_dtype == STAGING_BF16), _ptr(out))
    assert rc == 0, rc
    return out


def reference_elems(A, B, C=None, *, dtype, alpha=1.0, beta=0.0, ldc=0,
                    order=FLAT, groups=1, ii, jj):
    """Reduced result at elements (ii[e], jj[e]), fp64."""
    keep, args, _ = _common(A, B, C, dtype, alpha, beta, ldc)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    out = np.empty(ii.shape[0], dtype=np.float64)
    rc = _load().oracle_reference_elems(*args, order, groups, ii.shape[0],
                                        _ptr(ii), _ptr(jj), _ptr(out))
    assert rc == 0, rc
    return out


def reduce_emulate(S, *, order=FLAT, groups=1, out_bf16=True):
    """Ordered float sum of S[W][n] over W (flat or two-level), then
    bfloat16 RNE bits (out_bf16) or float32."""
    S = np.ascontiguousarray(S, dtype=np.float32)
    W, n = S.shape
    out = np.empty(n, dtype=np.uint16 if out_bf16 else np.float32)
    rc = _load().oracle_reduce_emulate(W, order, groups, n, _ptr(S),
                                       0 if out_bf16 else 1, _ptr(out))
    assert rc == 0, rc
    return out


def bf16_rne(x) -> np.ndarray:
    """float32 -> bfloat16 bits (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(x.shape[0], dtype=np.uint16)
    _load().oracle_bf16_rne_array(x.shape[0], _ptr(x), _ptr(out))
    return out


def bf16_bits_to_f64(h) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# error measures (the parity bar)
# --------------------------------------------------------------------------
def _same_shape(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    # no broadcasting: a result of the wrong shape is a failure, not a
    # smaller comparison
    if got.shape != ref.shape:
        raise ValueError("shape mismatch: got %s, ref %s" % (got.shape, ref.shape))
    return got, ref


def rel_frobenius(got, ref) -> float:
    """||got - ref||_F / ||ref||_F over all elements (the aggregate half of
    the accuracy bar).  A zero reference has no scale: the error is then
    ||got||_F itself (0 only for an all-zero result)."""
    got, ref = _same_shape(got, ref)
    den = np.sqrt(np.sum(ref * ref))
    num = np.sqrt(np.sum((got - ref) * (got - ref)))
    return float(num / (den if den > 0 else 1.0))


def max_norm_err(got, ref) -> float:
    """max |got - ref| / max(1, |ref|) over all elements (the elementwise
    half of the accuracy bar: absolute below |ref| = 1, relative above)."""
    got, ref = _same_shape(got, ref)
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref))))


# --------------------------------------------------------------------------
# all-gather + GEMM (include/gemm_ag.h)
# --------------------------------------------------------------------------
# pieces each tile-row of X is copied in (an implementation limit of the
# library's copy kernel, mirrored here only for the descriptor rules)
AG_COPY_PIECES = 16


def validate_ag(M, N, K, W, tile_m, tile_n, group_m=0, pad=0,
                supported_tiles: Optional[Sequence] = None):
    """Status a plan of the all-gather + GEMM must give.  INVALID_ARG: the
    gather hands every rank an equal row shard, so M % W != 0 is invalid
    (page "flux精读", section 3 Design: the input is all-gathered across
    the TP group); negative sizes or a non-zero pad.  UNSUPPORTED: the tile
    and K-step limits of the GEMM kernel, as in ``validate``."""
    ints = (M, N, K, W, tile_m, tile_n, group_m, pad)
    if any(not isinstance(v, (int, np.integer)) for v in ints):
        return INVALID_ARG
    if W < 1 or W > MAX_W or M < 1 or N < 1 or K < 1:
        return INVALID_ARG
    if M % W != 0:
        return INVALID_ARG
    if group_m < 0 or tile_m < 0 or tile_n < 0 or pad != 0:
        return INVALID_ARG
    if supported_tiles is not None and (tile_m, tile_n) not in set(
            tuple(t) for t in supported_tiles):
        return UNSUPPORTED
    if tile_m == 0 or tile_n == 0 or N % tile_n != 0 or K % K_STEP != 0:
        return UNSUPPORTED
    if max(M, N, K) > 2**31 - 1:
        return UNSUPPORTED
    if K >= 2**23 or N >= 2**25:
        return UNSUPPORTED
    if -(-M // tile_m) * (N // tile_n) * W > 2**31 - 1:
        return UNSUPPORTED
    # the gather is issued as AG_COPY_PIECES pieces per tile-row and rank,
    # counted in 32 bits
    if -(-M // tile_m) * W * AG_COPY_PIECES > 2**32 - 1:
        return UNSUPPORTED
    return OK


def ag_gather(X_shards: np.ndarray) -> np.ndarray:
    """The all-gathered input: shard d (rank d's M/W rows) becomes rows
    [d*M/W, (d+1)*M/W) of X (page "flux精读", section 3 Design)."""
    W, Mc, K = X_shards.shape
    return np.concatenate([X_shards[d] for d in range(W)], axis=0)


def ag_send_order(M, W, tile_m, r) -> List[int]:
    """Tile-rows of X in the order they are sent to rank r: its own chunk
    first, then chunks r+1, r+2, ... (mod W), each chunk's tile-rows in
    ascending order; a tile-row belongs to the chunk of its first row.  The
    GEMM's tiles wait in the same order (page "flux精读", section 3 Design:
    the wait order follows the send order)."""
    G = Geometry(M, tile_m, K_STEP, W, tile_m, tile_m, swizzle=SELF_FIRST)
    out = []
    for s in range(W):
        out.extend(G.chunk_tile_rows(G.dest(r, s)))
    return out


def ag_gemm_rows(X_shards, B, *, r, row_lo=0, row_hi=None) -> np.ndarray:
    """Rank r's output rows [row_lo, row_hi) of Y_r = X . B_r, fp64, where X
    is the gathered input (bfloat16 bit patterns in, as everywhere)."""
    X_shards = np.ascontiguousarray(X_shards)
    W, Mc, K = X_shards.shape
    # stacked row shards already are the gathered matrix, row for row (the
    # same rows as ag_gather, without a copy)
    X = X_shards.reshape(W * Mc, K)
    M = X.shape[0]
    row_hi = M if row_hi is None else row_hi
    return partial_rows(X[None], np.asarray(B)[r][None], dtype=BF16, r=0,
                        row_lo=row_lo, row_hi=row_hi)
