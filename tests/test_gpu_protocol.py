"""GPU protocol tests: flag life cycle, split runs, back-to-back runs with no
host sync, timeouts and stale flags forced from the host (every kernel
still exits: waits are bounded), and the reduce order checked bit for bit
on staging contents written by the test."""
import numpy as np
import pytest

import oracle as O
from tensor_gemm_reduce_lds_amd import gemm_rs as G
from tensor_gemm_reduce_lds_amd import inputs as I

from gpu_util import (check_tolerance, desc_fields, flags, h2d, new_out, oracle_kw, out_bits,
                      out_to_f64, put_staging, run_checked, say, sync, to_device)

pytestmark = pytest.mark.gpu

SMALL = I.with_shape(I.WORKLOADS["llama70b"], W=8, M=800, N=512, K=128,
                     tile_m=256, tile_n=256)


def _setup(w=SMALL, **over):
    x = I.make_inputs(w)
    return x, to_device(x, w), G.Plan(**desc_fields(w, **over))


def test_flag_life_cycle_and_split_runs():
    say("flag life cycle")
    x, dev, plan = _setup()
    with plan:
        ref = new_out(SMALL)
        run_checked(plan, dev, SMALL, ref)
        assert not flags(plan).any()
        o = new_out(SMALL)
        run_checked(plan, dev, SMALL, o, G.RUN_ALL | G.KEEP_FLAGS)
        assert flags(plan).all()
        run_checked(plan, dev, SMALL, o)            # GEMM re-sets 1s, reduce clears
        assert not flags(plan).any()
        run_checked(plan, dev, SMALL, o, G.RUN_GEMM)
        assert flags(plan).all()
        o2 = new_out(SMALL)
        run_checked(plan, dev, SMALL, o2, G.RUN_REDUCE)
        assert not flags(plan).any()
        assert np.array_equal(out_bits(o2), out_bits(ref))


def test_back_to_back_runs_without_host_sync():
    import torch
    say("back to back")
    x, dev, plan = _setup()
    with plan:
        s = torch.cuda.current_stream()
        outs = [new_out(SMALL) for _ in range(3)]
        for o in outs:
            plan.run(dev["A"], dev["B"], dev["C"], SMALL.alpha, SMALL.beta, o, s)
        rc, detail = plan.status(s)
        assert rc == G.OK, detail
        b = [out_bits(o) for o in outs]
        assert np.array_equal(b[0], b[1]) and np.array_equal(b[0], b[2])
        assert not flags(plan).any()


def test_missing_producer_times_out_and_plan_recovers():
    say("timeout")
    x, dev, plan = _setup(timeout_ms=5)
    with plan:
        o = new_out(SMALL)
        run_checked(plan, dev, SMALL, o, G.RUN_GEMM)
        r0, t0 = 5, 7
        h2d(plan.info.flags, np.zeros(1, dtype=np.uint32), (r0 * plan.info.T + t0) * 4)
        plan.run(dev["A"], dev["B"], dev["C"], SMALL.alpha, SMALL.beta, o, None,
                 G.RUN_REDUCE)
        rc, detail = plan.status()
        assert rc == G.ERR_TIMEOUT
        assert detail == [G.ERR_TIMEOUT, r0, t0, 0]
        assert not flags(plan).any()                 # status re-zeroed them
        assert plan.status()[0] == G.OK              # and cleared the record
        ref = new_out(SMALL)
        run_checked(plan, dev, SMALL, ref)           # the plan runs again


def test_stale_flag_is_a_protocol_error():
    say("protocol")
    x, dev, plan = _setup()
    with plan:
        o = new_out(SMALL)
        run_checked(plan, dev, SMALL, o, G.RUN_GEMM)
        r1, t1 = 2, 3
        h2d(plan.info.flags, np.array([2], dtype=np.uint32), (r1 * plan.info.T + t1) * 4)
        plan.run(dev["A"], dev["B"], dev["C"], SMALL.alpha, SMALL.beta, o, None,
                 G.RUN_REDUCE)
        rc, detail = plan.status()
        assert rc == G.ERR_PROTOCOL and detail == [G.ERR_PROTOCOL, r1, t1, 2]
        assert not flags(plan).any()


# ----------------------------------------------- reduce on host-written staging
def _reduce_only(W, M, N, dtype, order, groups, S_rmn, tile=(64, 128),
                 materialize=0):
    """Write S (per rank r, output [M][N]) into the staging slots, set every
    flag, run REDUCE only, return output bits."""
    import torch
    if dtype == G.F32:
        tile = (64, 64)     # the only fp32 tile
    desc = dict(M=M, N=N, K=64, W=W, dtype=dtype, tile_m=tile[0], tile_n=tile[1],
                order=order, groups=groups, materialize_sub=materialize)
    with G.Plan(**desc) as plan:
        Mc = M // W
        # staging S[d][r][Mc][N] from S_rmn[r][d*Mc + il][j]
        st = S_rmn.reshape(W, W, Mc, N).transpose(1, 0, 2, 3)
        geom = O.Geometry(M, N, 64, W, tile[0], tile[1], order=order, groups=groups)
        put_staging(plan, geom, np.ascontiguousarray(st, dtype=np.float32))
        h2d(plan.info.flags, np.ones(W * plan.info.T, dtype=np.uint32))
        out = torch.empty((M, N), dtype=torch.int16 if dtype == G.BF16 else torch.float32,
                          device="cuda:0")
        plan.run(None, None, None, 1.0, 0.0, out, None, G.RUN_REDUCE)
        rc, detail = plan.status()
        assert rc == G.OK, detail
        assert not flags(plan).any()
        return out_bits(out)


@pytest.mark.parametrize("order,groups,want", [(O.FLAT, 1, 0.0),
                                               (O.TWO_LEVEL, 2, 3.0),
                                               (O.TWO_LEVEL, 4, 5.0)])
def test_reduce_order_closed_form(order, groups, want):
    say("reduce order", order, groups)
    v = np.array([2.0**24, 1, 1, 1, 1, 1, 1, -2.0**24], dtype=np.float32)
    W, M, N = 8, 64, 128
    S = np.broadcast_to(v[:, None, None], (W, M, N)).astype(np.float32)
    for materialize in ([0, 1] if order == O.TWO_LEVEL else [0]):
        bits = _reduce_only(W, M, N, G.F32, order, groups, S, materialize=materialize)
        assert np.all(bits.view(np.float32) == want)
        bits = _reduce_only(W, M, N, G.BF16, order, groups, S, materialize=materialize)
        assert np.all(bits == O.bf16_rne(np.array([want], np.float32))[0])


@pytest.mark.parametrize("dtype", [G.BF16, G.F32])
@pytest.mark.parametrize("order,groups,materialize", [(O.FLAT, 1, 0), (O.TWO_LEVEL, 2, 0),
                                                      (O.TWO_LEVEL, 4, 0),
                                                      (O.TWO_LEVEL, 2, 1)])
def test_reduce_random_staging_bit_exact(dtype, order, groups, materialize):
    say("reduce random", dtype, order, groups, materialize)
    rng = np.random.default_rng(21)
    W, M, N = 8, 8 * 40, 256
    S = (rng.standard_normal((W, M, N)) * np.exp(rng.uniform(-8, 8, (W, M, N)))).astype(
        np.float32)
    bits = _reduce_only(W, M, N, dtype, order, groups, S, tile=(128, 128),
                        materialize=materialize)
    want = O.reduce_emulate(S.reshape(W, M * N), order=order, groups=groups,
                            out_bf16=(dtype == G.BF16))
    assert np.array_equal(bits.ravel(), want.view(bits.dtype))


def test_output_rounding_ties_w1():
    say("rne ties")
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F808008], dtype=np.uint32)
    W, M, N = 1, 64, 128
    S = np.resize(ties, M * N).view(np.float32).reshape(1, M, N)
    bits = _reduce_only(W, M, N, G.BF16, O.FLAT, 1, S)
    assert bits.ravel()[:4].tolist() == [0x3F80, 0x3F82, 0xBF80, 0x3F81]
    assert np.array_equal(bits.ravel(), O.bf16_rne(S.ravel()))


# ------------------------------------------------ overlapped reduce (slices)
@pytest.mark.parametrize("swizzle", [G.SWIZZLE_REMOTE_FIRST, G.SWIZZLE_IDENTITY])
@pytest.mark.parametrize("name", ["llama8b", "ragged_2lvl", "decode",
                                  "llama70b_small"])
def test_overlapped_reduce_matches_serial_bits(name, swizzle):
    """The overlapped orders give the same bits as the serial remote-first
    order: the owner-fused reduce for the remote-first order (the last
    step's workgroups sum their tiles), chunk-by-chunk slices reduced on a
    second stream for the identity order; decode has unequal chunks and
    takes the serial path."""
    import torch
    if name == "llama70b_small":
        w = I.with_shape(I.WORKLOADS["llama70b"], M=2048, N=1024, K=512)
    else:
        w = I.WORKLOADS[name]
    say("overlap", name, "swizzle", swizzle)
    x, dev, plan = _setup(w, swizzle=swizzle)
    with plan:
        s = torch.cuda.current_stream()
        ref, got = new_out(w), new_out(w)
        if swizzle == G.SWIZZLE_REMOTE_FIRST:
            run_checked(plan, dev, w, ref)
        else:
            # the tile order does not change any element's arithmetic
            with G.Plan(**desc_fields(w)) as plan_rf:
                run_checked(plan_rf, dev, w, ref)
        for _ in range(2):   # twice: flags must come back to 0 in between
            plan.run(dev["A"], dev["B"], dev["C"], w.alpha, w.beta, got, s,
                     G.RUN_ALL | G.OVERLAP_REDUCE)
            rc, detail = plan.status(s)
            assert rc == G.OK, detail
            assert not flags(plan).any()
            assert np.array_equal(out_bits(got), out_bits(ref))
        plan.run(dev["A"], dev["B"], dev["C"], w.alpha, w.beta, got, s,
                 G.RUN_ALL | G.OVERLAP_REDUCE | G.KEEP_FLAGS)
        assert plan.status(s)[0] == G.OK
        assert flags(plan).all()


def _chunk_rows(w, rng, per_chunk=3):
    """Every chunk's first and last row plus random rows of each chunk."""
    Mc = w.M // w.W
    rows = set()
    for d in range(w.W):
        rows.update([d * Mc, d * Mc + Mc - 1])
        rows.update(d * Mc + int(v) for v in rng.integers(0, Mc, size=per_chunk - 2))
    return sorted(rows)


@pytest.mark.parametrize("name", ["llama70b", "ragged_2lvl"])
def test_identity_overlap_full_size_against_oracle(name):
    """The identity order's overlapped reduce (chunk groups reduced on the
    plan's second stream while the next group's GEMM runs), at full size in
    the launch configuration the benchmark times: sampled rows and 3000
    sampled elements against the oracle's fp64 reference, then integer
    inputs whose sampled rows must equal the oracle's emulation bit for
    bit."""
    import torch
    w = I.WORKLOADS[name]
    rng = np.random.default_rng(41)
    kw = oracle_kw(w)
    for dist in ("normal", "ternary"):
        x = I.make_inputs(w) if dist == "normal" else I.make_inputs(w, dist="ternary",
                                                                    c_dist="ternary")
        dev = to_device(x, w)
        say("identity overlap full", name, dist)
        with G.Plan(**desc_fields(w, swizzle=G.SWIZZLE_IDENTITY)) as plan:
            s = torch.cuda.current_stream()
            got = new_out(w)
            plan.run(dev["A"], dev["B"], dev["C"], w.alpha, w.beta, got, s,
                     G.RUN_ALL | G.OVERLAP_REDUCE)
            rc, detail = plan.status(s)
            assert rc == G.OK, detail
            assert not flags(plan).any()
        rows = _chunk_rows(w, rng)
        if dist == "normal":
            g = out_to_f64(got, w)
            ref = np.concatenate([O.reference_rows(x["A"], x["B"], x["C"], row_lo=i,
                                                   row_hi=i + 1, **kw) for i in rows])
            check_tolerance(g[rows], ref, w.dtype)
            ii = rng.integers(0, w.M, size=3000)
            jj = rng.integers(0, w.N, size=3000)
            mx, rf = check_tolerance(g[ii, jj], O.reference_elems(x["A"], x["B"], x["C"],
                                                                  ii=ii, jj=jj, **kw), w.dtype)
            say("  sampled max_norm_err %.3e rel_F %.3e" % (mx, rf))
        else:
            bits = out_bits(got)
            for i in rows:
                em = O.emulate_rows(x["A"], x["B"], x["C"], row_lo=i, row_hi=i + 1, **kw)
                assert np.array_equal(bits[i], em[0].view(bits.dtype)), i
        del dev, got
