"""All-gather fused into the GEMM prologue (include/gemm_ag.h), through the
C ABI, against the oracle.

The fused mode launches the GEMM before the copies (the copies run on the
plan's second stream), so a tile that did not wait for its signal would read
the gathered buffer before its rows arrived: the buffer is filled with NaN
before every fused run, and a single early read shows as NaN in the output."""
import ctypes

import numpy as np
import pytest

import oracle as O
from tensor_gemm_reduce_lds_amd import gemm_rs as G
from tensor_gemm_reduce_lds_amd import inputs as I

from gpu_util import check_tolerance, d2h, hip, say

pytestmark = pytest.mark.gpu


def _dev(x):
    import torch
    return {k: torch.from_numpy(v.view(np.int16)).to("cuda:0") for k, v in x.items()}


def _out(W, M, N):
    import torch
    return torch.empty((W, M, N), dtype=torch.int16, device="cuda:0")


def _f64(out):
    return I.bf16_bits_to_f32(out.cpu().numpy().view(np.uint16)).astype(np.float64)


def _poison(plan):
    info = plan.info
    hip().hipMemset.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t]
    assert hip().hipMemset(info.gathered, 0xFF, info.gathered_bytes) == 0


SMALL = [
    # ragged last tile-row and tile-rows that straddle chunks (Mc = 100)
    ("w8_ragged", dict(M=800, N=512, K=256, W=8)),
    # 256x128 tiles, W=4
    ("w4_256x128", dict(M=520, N=384, K=192, W=4, tile_m=256, tile_n=128)),
    # 64x128 tiles, one tile-row (chunks of 8 rows share it)
    ("decode_like", dict(M=64, N=512, K=256, W=8)),
    # W=1: the gather is a plain copy
    ("w1", dict(M=256, N=256, K=128, W=1)),
]


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name,shape", SMALL, ids=[s[0] for s in SMALL])
def test_small_parity(name, shape, fused):
    import torch
    M, N, K, W = shape["M"], shape["N"], shape["K"], shape["W"]
    x = I.make_ag_inputs(M, N, K, W)
    say("ag", name, "fused" if fused else "serial")
    dev = _dev(x)
    out = _out(W, M, N)
    s = torch.cuda.current_stream()
    flags = G.AG_RUN_ALL | (G.AG_FUSED if fused else 0)
    with G.AgPlan(**shape) as plan:
        _poison(plan)
        plan.run(dev["X"], dev["B"], out, s, flags)
        rc, detail = plan.status(s)
        assert rc == G.OK, detail
        got = _f64(out)
    assert not np.isnan(got).any()
    for r in range(W):
        ref = O.ag_gemm_rows(x["X"], x["B"], r=r)
        check_tolerance(got[r], ref, "bf16")


def test_fused_runs_gate_on_signals_and_repeat():
    """Three fused runs in a row, each on a NaN-filled gathered buffer: the
    signals' epoch advances, no tile reads early, and every run gives the
    serial order's bits; a GEMM-only run afterwards reuses the buffer."""
    import torch
    M, N, K, W = 2048, 1024, 512, 8
    x = I.make_ag_inputs(M, N, K, W)
    dev = _dev(x)
    s = torch.cuda.current_stream()
    ref, out = _out(W, M, N), _out(W, M, N)
    with G.AgPlan(M=M, N=N, K=K, W=W) as plan:
        plan.run(dev["X"], dev["B"], ref, s, G.AG_RUN_ALL)
        assert plan.status(s)[0] == G.OK
        e0 = plan.info.epoch
        for k in range(3):
            _poison(plan)
            plan.run(dev["X"], dev["B"], out, s, G.AG_RUN_ALL | G.AG_FUSED)
            rc, detail = plan.status(s)
            assert rc == G.OK, detail
            assert plan.info.epoch == e0 + k + 1
            assert torch.equal(out, ref)
        sig = d2h(plan.info.signals, W * plan.info.tiles_m * 4, np.uint32)
        assert (sig == plan.info.epoch).all()
        out.zero_()
        plan.run(None, dev["B"], out, s, G.AG_RUN_GEMM)
        assert plan.status(s)[0] == G.OK
        assert torch.equal(out, ref)


def test_integer_inputs_bit_exact_up_projection():
    """The Llama-3-70B-like up-projection shard (W=8, M=8192, K=8192,
    N=3584) with entries in {-1,0,1}: every output is an integer below 2^24,
    exact in the float accumulators, so each rank's output equals the
    oracle's bfloat16 rounding of the exact product bit for bit (sampled
    rows, every rank, fused mode on a NaN-filled buffer)."""
    import torch
    p = I.AG_WORKLOADS["llama70b_up"]
    M, N, K, W = p["M"], p["N"], p["K"], p["W"]
    x = I.make_ag_inputs(M, N, K, W, index=p["index"], dist="ternary")
    dev = _dev(x)
    s = torch.cuda.current_stream()
    out = _out(W, M, N)
    say("ag integer exactness", M, N, K, W)
    with G.AgPlan(M=M, N=N, K=K, W=W) as plan:
        _poison(plan)
        plan.run(dev["X"], dev["B"], out, s, G.AG_RUN_ALL | G.AG_FUSED)
        rc, detail = plan.status(s)
        assert rc == G.OK, detail
    bits = out.cpu().numpy().view(np.uint16)
    rng = np.random.default_rng(5)
    Mc = M // W
    rows = sorted({d * Mc for d in range(W)} | {d * Mc + Mc - 1 for d in range(W)} |
                  {int(v) for v in rng.integers(0, M, 8)})
    for r in range(W):
        for i in rows:
            want = O.bf16_rne(O.ag_gemm_rows(x["X"], x["B"], r=r, row_lo=i,
                                             row_hi=i + 1)[0].astype(np.float32))
            assert np.array_equal(bits[r, i], want), (r, i)


def test_wait_timeout_is_reported_and_recovers():
    """A GEMM told to wait for an epoch no copy publishes (a debug flag set
    from the host) times out in every workgroup's bounded wait, reports
    TIMEOUT with the rank and tile-row, and the next run is correct."""
    import torch
    M, N, K, W = 512, 256, 128, 4
    x = I.make_ag_inputs(M, N, K, W)
    dev = _dev(x)
    s = torch.cuda.current_stream()
    ref, out = _out(W, M, N), _out(W, M, N)
    with G.AgPlan(M=M, N=N, K=K, W=W, timeout_ms=5) as plan:
        plan.run(dev["X"], dev["B"], ref, s, G.AG_RUN_ALL)
        assert plan.status(s)[0] == G.OK
        plan.run(None, dev["B"], out, s, G.AG_RUN_GEMM | G.AG_EXPECT_NEXT)
        rc, detail = plan.status(s)
        assert rc == G.ERR_TIMEOUT
        assert detail[0] == G.ERR_TIMEOUT and 0 <= detail[1] < W
        assert 0 <= detail[2] < plan.info.tiles_m
        assert plan.status(s)[0] == G.OK          # cleared
        plan.run(dev["X"], dev["B"], out, s, G.AG_RUN_ALL | G.AG_FUSED)
        assert plan.status(s)[0] == G.OK
        assert torch.equal(out, ref)


def test_full_size_sampled_parity_fused():
    """The up-projection shard as the bench runs it (W=8, M=8192, K=8192,
    N=3584, 256x256 tiles, fused, N(0,1) and N(0,1/K) inputs) on a
    NaN-filled gathered buffer: sampled rows of every rank (each chunk's
    first and last row, straddling tile-rows, random rows) against the fp64
    oracle, to the bf16 output bar."""
    import torch
    p = I.AG_WORKLOADS["llama70b_up"]
    M, N, K, W = p["M"], p["N"], p["K"], p["W"]
    x = I.make_ag_inputs(M, N, K, W, index=p["index"])
    dev = _dev(x)
    s = torch.cuda.current_stream()
    out = _out(W, M, N)
    say("ag full-size sampled parity", M, N, K, W)
    with G.AgPlan(M=M, N=N, K=K, W=W) as plan:
        _poison(plan)
        plan.run(dev["X"], dev["B"], out, s, G.AG_RUN_ALL | G.AG_FUSED)
        rc, detail = plan.status(s)
        assert rc == G.OK, detail
    got = out.cpu().numpy().view(np.uint16)
    rng = np.random.default_rng(17)
    Mc = M // W
    rows = sorted({d * Mc for d in range(W)} | {d * Mc + Mc - 1 for d in range(W)} |
                  {int(v) for v in rng.integers(0, M, 6)})
    for r in range(W):
        g = I.bf16_bits_to_f32(got[r, rows]).astype(np.float64)
        ref = np.concatenate([O.ag_gemm_rows(x["X"], x["B"], r=r, row_lo=i, row_hi=i + 1)
                              for i in rows])
        assert not np.isnan(g).any()
        check_tolerance(g, ref, "bf16")
