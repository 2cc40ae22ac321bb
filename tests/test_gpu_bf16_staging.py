"""bfloat16 staging (GEMM_RS_STAGING_BF16) on the GPU, through the C ABI.

In this mode every rank's epilogue value is rounded to bfloat16 (nearest
even) when it is staged; the reduce widens the slots back to float and sums
them in the same fixed order.  The second rounding has its own bar (see
``check_bf16_staging``); integer-valued inputs pin every staged slot and
every output bit against the oracle's emulation of exactly this pipeline."""
import ctypes

import numpy as np
import pytest

import oracle as O
from tensor_gemm_reduce_lds_amd import gemm_rs as G
from tensor_gemm_reduce_lds_amd import inputs as I

from gpu_util import (check_bf16_staging, d2h, desc_fields, flags, geometry, h2d, hip,
                      new_out, oracle_kw, out_bits, out_to_f64, run_checked, say, staging_slots,
                      to_device)

pytestmark = pytest.mark.gpu

W70 = I.WORKLOADS
BF = dict(staging_dtype=G.STAGING_BF16)


def staging16_rows(plan, geom, d, r, il0, n):
    """Rows il0..il0+n of bfloat16 staging slot (d, r) as uint16 [n][N]."""
    off = geom.staging_offset(d, r, d * geom.Mc + il0, 0) * 2
    return d2h(plan.info.staging + off, n * geom.N * 2, np.uint16).reshape(n, geom.N)


SMALL = [
    ("bf16_256x256_ragged", I.with_shape(W70["llama8b"], W=8, M=800, N=512, K=256,
                                         tile_m=256, tile_n=256), {}),
    ("bf16_256x128_w4", I.with_shape(W70["llama8b"], W=4, M=520, N=384, K=192,
                                     tile_m=256, tile_n=128), {}),
    ("bf16_128x128_fullc", I.with_shape(W70["llama70b"], W=8, M=320, N=256, K=320,
                                        tile_m=128, tile_n=128, ldc=256), {}),
    ("bf16_64x128_decode", I.with_shape(W70["decode"], M=64, N=512, K=256), {}),
    ("two_level_g2", I.with_shape(W70["ragged_2lvl"], M=8 * 40, N=256, K=128,
                                  tile_m=128, tile_n=128), {}),
    ("tile_interleaved", I.with_shape(W70["llama8b"], W=8, M=800, N=512, K=256,
                                      tile_m=256, tile_n=256),
     dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED)),
]


@pytest.mark.parametrize("name,w,over", SMALL, ids=[s[0] for s in SMALL])
def test_small_parity(name, w, over):
    x = I.make_inputs(w)
    say("bf16 staging", name)
    dev = to_device(x, w)
    with G.Plan(**desc_fields(w, **BF, **over)) as plan:
        geom = geometry(w, plan)
        assert plan.info.slot_elems == geom.slot
        assert plan.info.staging_bytes == w.W * w.W * geom.slot * 2
        out = new_out(w)
        run_checked(plan, dev, w, out)
        assert not flags(plan).any()
        got = out_to_f64(out, w)
    kw = oracle_kw(w)
    ref = O.reference_rows(x["A"], x["B"], x["C"], **kw)
    mag = sum(np.abs(O.partial_rows(x["A"], x["B"], x["C"], dtype=kw["dtype"],
                                    alpha=w.alpha, beta=w.beta, ldc=w.ldc, r=r))
              for r in range(w.W))
    used, rf = check_bf16_staging(got, ref, mag)
    say("  bound used %.3f rel_F %.3e" % (used, rf))


def _sample_rows(w, rng):
    Mc = w.M // w.W
    rows = set()
    for d in range(w.W):
        rows.update((d * Mc, d * Mc + Mc - 1, d * Mc + int(rng.integers(0, Mc))))
    return sorted(rows)


@pytest.mark.parametrize("name", ["llama8b", "ragged_2lvl", "llama70b"])
def test_integer_inputs_bit_exact(name):
    """Entries in {-1,0,1}: every partial is an integer, exact in the float
    accumulators, so each staged slot must equal bfloat16-RNE of the
    oracle's partial bit for bit (partials above 256 in magnitude do round)
    and the output must equal the oracle's bfloat16-staging emulation.
    Staging is filled with 0xFFFF (NaN) first: an unwritten slot shows."""
    w = W70[name]
    x = I.make_inputs(w, dist="ternary", c_dist="ternary")
    rng = np.random.default_rng(11)
    dev = to_device(x, w)
    say("bf16 staging integer exactness", name)
    kw = oracle_kw(w)
    with G.Plan(**desc_fields(w, **BF)) as plan:
        geom = geometry(w, plan)
        ptr, nbytes = plan.info.staging, plan.info.staging_bytes
        hip().hipMemset.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t]
        assert hip().hipMemset(ptr, 0xFF, nbytes) == 0
        out = new_out(w)
        run_checked(plan, dev, w, out, G.RUN_GEMM)
        st = staging_slots(plan, geom, np.uint16)
        assert not (st == 0xFFFF).any(), "staging elements left unwritten"
        del st
        rows = _sample_rows(w, rng)
        for i in rows:
            d = i // geom.Mc
            for r in range(w.W):
                part = O.partial_rows(x["A"], x["B"], x["C"], dtype=kw["dtype"],
                                      alpha=w.alpha, beta=w.beta, ldc=w.ldc, r=r,
                                      row_lo=i, row_hi=i + 1)[0].astype(np.float32)
                want = O.bf16_rne(part)
                got = staging16_rows(plan, geom, d, r, i - d * geom.Mc, 1)[0]
                assert np.array_equal(got, want), (i, r)
        run_checked(plan, dev, w, out, G.RUN_REDUCE)
        assert not flags(plan).any()
        bits = out_bits(out)
    for i in rows:
        em = O.emulate_rows(x["A"], x["B"], x["C"], row_lo=i, row_hi=i + 1,
                            staging_dtype=O.STAGING_BF16, **kw)
        assert np.array_equal(bits[i], em[0].view(bits.dtype)), i


@pytest.mark.parametrize("swizzle", [G.SWIZZLE_REMOTE_FIRST, G.SWIZZLE_IDENTITY])
def test_overlapped_reduce_matches_serial_bits(swizzle):
    import torch
    w = I.with_shape(W70["llama70b"], M=2048, N=1024, K=512)
    x = I.make_inputs(w)
    say("bf16 staging overlap", swizzle)
    dev = to_device(x, w)
    s = torch.cuda.current_stream()
    with G.Plan(**desc_fields(w, **BF)) as plan_rf:
        ref = new_out(w)
        run_checked(plan_rf, dev, w, ref)
    with G.Plan(**desc_fields(w, swizzle=swizzle, **BF)) as plan:
        got = new_out(w)
        for _ in range(2):
            plan.run(dev["A"], dev["B"], dev["C"], w.alpha, w.beta, got, s,
                     G.RUN_ALL | G.OVERLAP_REDUCE)
            rc, detail = plan.status(s)
            assert rc == G.OK, detail
            assert not flags(plan).any()
            assert np.array_equal(out_bits(got), out_bits(ref))


def test_reduce_only_widening_and_order():
    """Host-written bfloat16 slots: rank 0 holds 256 and rank 1 holds 260
    (0x4380, 0x4382) everywhere; the float sum 516 is exact in bfloat16
    (0x4401).  A second column pattern checks the widening of both halves
    of each 32-bit word: -1.5 (0xBFC0) and 3.0 (0x4040) sum to 1.5 (0x3FC0)."""
    import torch
    W, M, N = 2, 64, 128
    with G.Plan(M=M, N=N, K=64, W=W, tile_m=64, tile_n=128, **BF) as plan:
        Mc = M // W
        assert plan.info.slot_elems == Mc * N            # small slots: contiguous
        S = np.empty((W, W, Mc, N), dtype=np.uint16)     # S[d][r][il][j]
        S[:, 0] = 0x4380
        S[:, 1] = 0x4382
        S[:, 0, :, 1::2] = 0xBFC0
        S[:, 1, :, 1::2] = 0x4040
        h2d(plan.info.staging, S)
        h2d(plan.info.flags, np.ones(W * plan.info.T, dtype=np.uint32))
        out = torch.empty((M, N), dtype=torch.int16, device="cuda:0")
        plan.run(None, None, None, 1.0, 0.0, out, None, G.RUN_REDUCE)
        rc, detail = plan.status()
        assert rc == G.OK, detail
        bits = out_bits(out)
    assert (bits[:, 0::2] == 0x4401).all()
    assert (bits[:, 1::2] == 0x3FC0).all()
