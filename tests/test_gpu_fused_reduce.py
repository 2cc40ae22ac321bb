"""GPU parity of the owner-fused reduce (GEMM_RS_OVERLAP_REDUCE with the
remote-first order): the last tile-order step of every rank is its own
chunk, so those workgroups sum each tile's W partials themselves and write
the output; no separate reduce runs and the owner's partial is never
staged.  Checked against the oracle (reference tolerance on normal inputs,
bit-exact emulate mode and staged partials on integer-valued inputs),
against the serial path's bits, and for its flag and staging footprint."""
import ctypes

import numpy as np
import pytest

import oracle as O
from tensor_gemm_reduce_lds_amd import gemm_rs as G
from tensor_gemm_reduce_lds_amd import inputs as I

from gpu_util import (check_bf16_staging, check_tolerance, d2h, desc_fields, flags, geometry,
                      hip, new_out, oracle_kw, out_bits, out_to_f64, run_checked, say,
                      staging_slots, to_device)

pytestmark = pytest.mark.gpu

W70 = I.WORKLOADS
FUSED = G.RUN_ALL | G.OVERLAP_REDUCE

# small fused-eligible cases (W = 8, 256 x 256 tiles, every chunk owning the
# same number of tile-rows), each compared with the oracle in full
SMALL = [
    # bias row, one tile-row per chunk
    ("bias_row", I.with_shape(W70["llama70b"], M=2048, N=1024, K=512), {}),
    # full C matrix with alpha and beta
    ("full_c", I.with_shape(W70["llama70b"], M=2048, N=512, K=192, ldc=512,
                            alpha=1.25, beta=0.75, c_std=1.0), {}),
    # beta*C inexact in float (beta = 0.7, 0.3): the serial epilogue's paths
    # and the fused sum must all round x + beta*c the same way
    ("bias_row_beta", I.with_shape(W70["llama70b"], M=2048, N=512, K=256,
                                   alpha=1.0, beta=0.7, c_std=1.0), {}),
    ("full_c_beta", I.with_shape(W70["llama70b"], M=2048, N=512, K=192, ldc=512,
                                 alpha=0.9, beta=0.3, c_std=1.0), {}),
    # the same with bfloat16 staging and tiles straddling chunks (the
    # epilogue's ragged-row path): the staged value is rounded once more
    ("bf16_staging_bias_beta", I.with_shape(W70["llama70b"], M=4000, N=512, K=128,
                                            alpha=1.0, beta=0.7, c_std=1.0),
     dict(staging_dtype=G.STAGING_BF16)),
    # Mc = 500: two tile-rows per chunk, every second one straddles into the
    # next chunk, ragged last tile-row (4000 = 15*256 + 160); two-level G=2
    ("straddle_2lvl", I.with_shape(W70["ragged_2lvl"], M=4000, N=512, K=128), {}),
    ("straddle_g4", I.with_shape(W70["ragged_2lvl"], M=4000, N=256, K=128, groups=4), {}),
    ("straddle_flat", I.with_shape(W70["llama8b"], M=4000, N=256, K=192), {}),
    # bf16 staging: the owner's value is rounded as a staging slot would hold it
    ("bf16_staging", I.with_shape(W70["llama70b"], M=2048, N=512, K=256),
     dict(staging_dtype=G.STAGING_BF16)),
    ("bf16_staging_straddle", I.with_shape(W70["ragged_2lvl"], M=4000, N=256, K=128),
     dict(staging_dtype=G.STAGING_BF16)),
]


def _serial_and_fused(w, x, over, rounds=2):
    dev = to_device(x, w)
    with G.Plan(**desc_fields(w, **over)) as plan:
        ref = new_out(w)
        run_checked(plan, dev, w, ref)
        got = new_out(w)
        for _ in range(rounds):   # flags must come back to 0 in between
            run_checked(plan, dev, w, got, FUSED)
            assert not flags(plan).any()
        return out_bits(ref), out_bits(got), out_to_f64(got, w)


@pytest.mark.parametrize("name,w,over", SMALL, ids=[c[0] for c in SMALL])
def test_fused_small_full_parity(name, w, over):
    x = I.make_inputs(w)
    say("fused small", name)
    serial, fused, got = _serial_and_fused(w, x, over)
    assert np.array_equal(fused, serial)
    kw = oracle_kw(w)
    ref = O.reference_rows(x["A"], x["B"], x["C"], **kw)
    if over.get("staging_dtype") == G.STAGING_BF16:
        # the second rounding's own bar (bit-exact pins: integer inputs)
        mag = sum(np.abs(O.partial_rows(x["A"], x["B"], x["C"], dtype=kw["dtype"],
                                        alpha=w.alpha, beta=w.beta, ldc=w.ldc, r=r))
                  for r in range(w.W))
        used, rf = check_bf16_staging(got, ref, mag)
        say("  bound used %.3f rel_F %.3e" % (used, rf))
        return
    mx, rf = check_tolerance(got, ref, w.dtype)
    say("  max_norm_err %.3e rel_F %.3e" % (mx, rf))


@pytest.mark.parametrize("name", ["straddle_2lvl", "bias_row", "full_c",
                                  "bf16_staging_straddle"])
def test_fused_small_integer_exact(name):
    """Integer-valued inputs: every partial is exact in float, so the output
    equals the oracle's float-pipeline emulation bit for bit (with bfloat16
    staging: each partial rounded to bfloat16 first, the owner's included)."""
    w, over = {c[0]: (c[1], c[2]) for c in SMALL}[name]
    # K = 512 and entries up to 1 in magnitude: bfloat16 staging rounds the
    # partials above 256
    if over.get("staging_dtype") == G.STAGING_BF16:
        w = I.with_shape(w, K=512)
    x = I.make_inputs(w, dist="ternary", c_dist="ternary")
    say("fused small integer", name)
    serial, fused, _ = _serial_and_fused(w, x, over)
    em = O.emulate_rows(x["A"], x["B"], x["C"], **oracle_kw(w),
                        staging_dtype=over.get("staging_dtype", O.STAGING_F32))
    assert np.array_equal(fused, em.view(fused.dtype))
    assert np.array_equal(serial, fused)


def _sample_rows(w, rng, per_chunk=3):
    Mc = w.M // w.W
    rows = set()
    for d in range(w.W):
        rows.update([d * Mc, d * Mc + Mc - 1])
        for _ in range(per_chunk - 2):
            rows.add(d * Mc + int(rng.integers(0, Mc)))
    return sorted(rows)


@pytest.mark.parametrize("name", ["llama70b", "ragged_2lvl", "llama8b"])
def test_fused_full_size_sampled_parity(name):
    """The workloads at full size, in the launch configuration the
    benchmark times: sampled rows (every chunk's first and last) and 3000
    sampled elements against the oracle, and every bit against the serial
    path."""
    w = W70[name]
    rng = np.random.default_rng(31)
    x = I.make_inputs(w)
    say("fused full", name)
    serial, fused, got = _serial_and_fused(w, x, {}, rounds=1)
    assert np.array_equal(fused, serial)
    kw = oracle_kw(w)
    rows = _sample_rows(w, rng)
    ref_rows = np.concatenate([O.reference_rows(x["A"], x["B"], x["C"], row_lo=i,
                                                row_hi=i + 1, **kw) for i in rows])
    check_tolerance(got[rows], ref_rows, w.dtype)
    ii = rng.integers(0, w.M, size=3000)
    jj = rng.integers(0, w.N, size=3000)
    ref_e = O.reference_elems(x["A"], x["B"], x["C"], ii=ii, jj=jj, **kw)
    mx, rf = check_tolerance(got[ii, jj], ref_e, w.dtype)
    say("  sampled max_norm_err %.3e rel_F %.3e" % (mx, rf))


@pytest.mark.parametrize("name", ["llama70b", "ragged_2lvl"])
def test_fused_integer_inputs_staging_footprint(name):
    """Entries in {-1,0,1} at full size, staging filled with NaN first.
    After a fused run, a staged row (slot (d(i), r), row i) is written iff
    rank r is not the owner of row i's tile (the chunk of the tile's first
    row): the owner's partial never leaves registers.  Written rows equal
    the oracle's partials bit for bit; the output equals emulate mode on
    sampled rows and the serial path everywhere."""
    w = W70[name]
    x = I.make_inputs(w, dist="ternary", c_dist="ternary")
    rng = np.random.default_rng(17)
    dev = to_device(x, w)
    say("fused integer footprint", name)
    kw = oracle_kw(w)
    with G.Plan(**desc_fields(w)) as plan:
        geom = geometry(w, plan)
        ref = new_out(w)
        run_checked(plan, dev, w, ref)
        ptr, nbytes = plan.info.staging, plan.info.staging_bytes
        hip().hipMemset.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t]
        assert hip().hipMemset(ptr, 0xFF, nbytes) == 0
        out = new_out(w)
        run_checked(plan, dev, w, out, FUSED)
        assert not flags(plan).any()
        st = staging_slots(plan, geom)
        bits = out_bits(out)
        assert np.array_equal(bits, out_bits(ref))
    Mc = geom.Mc
    for d in range(w.W):
        rows = np.arange(d * Mc, (d + 1) * Mc)
        owner = np.array([geom.owner(i // geom.BM) for i in rows])
        for r in range(w.W):
            nan_rows = np.isnan(st[d, r]).all(axis=1)
            any_nan = np.isnan(st[d, r]).any(axis=1)
            assert np.array_equal(nan_rows, any_nan), (d, r)    # whole rows only
            assert np.array_equal(nan_rows, owner == r), (d, r)
    for i in _sample_rows(w, rng):
        d = i // Mc
        for r in range(w.W):
            if geom.owner(i // geom.BM) == r:
                continue
            want = O.partial_rows(x["A"], x["B"], x["C"], dtype=kw["dtype"], alpha=w.alpha,
                                  beta=w.beta, ldc=w.ldc, r=r, row_lo=i,
                                  row_hi=i + 1)[0].astype(np.float32)
            assert np.array_equal(st[d, r, i - d * Mc].view(np.uint32), want.view(np.uint32))
        em = O.emulate_rows(x["A"], x["B"], x["C"], row_lo=i, row_hi=i + 1, **kw)
        assert np.array_equal(bits[i], em[0].view(bits.dtype)), i


def test_fused_back_to_back_and_mixed_with_serial():
    """Fused and serial passes back to back on one stream with no host sync
    in between: each leaves the flags idle for the next."""
    import torch
    w = dict((c[0], c[1]) for c in SMALL)["straddle_2lvl"]
    x = I.make_inputs(w)
    dev = to_device(x, w)
    say("fused back to back")
    with G.Plan(**desc_fields(w)) as plan:
        s = torch.cuda.current_stream()
        outs = [new_out(w) for _ in range(4)]
        for k, o in enumerate(outs):
            plan.run(dev["A"], dev["B"], dev["C"], w.alpha, w.beta, o, s,
                     FUSED if k % 2 == 0 else G.RUN_ALL)
        rc, detail = plan.status(s)
        assert rc == G.OK, detail
        b = [out_bits(o) for o in outs]
        for k in range(1, 4):
            assert np.array_equal(b[0], b[k]), k
        assert not flags(plan).any()


def test_fused_trace_and_k0():
    """TRACE_TILES in the fused mode records every logical block's tile as
    the oracle orders them; with K = 0 the fused output is beta*C bit for
    bit."""
    import torch
    w = dict((c[0], c[1]) for c in SMALL)["bias_row"]
    x = I.make_inputs(w)
    dev = to_device(x, w)
    say("fused trace")
    with G.Plan(**desc_fields(w)) as plan:
        out = new_out(w)
        run_checked(plan, dev, w, out, FUSED | G.TRACE_TILES)
        tr = d2h(plan.info.trace, w.W * plan.info.T * 4, np.int32)
        assert np.array_equal(tr, geometry(w, plan).trace())
    w0 = I.with_shape(w, K=0, alpha=1.5, beta=0.75, c_std=1.0)
    x0 = I.make_inputs(w0)
    say("fused k0")
    C = torch.from_numpy(x0["C"].view(np.int16)).to("cuda:0")
    with G.Plan(**desc_fields(w0)) as plan:
        out = new_out(w0)
        s = torch.cuda.current_stream()
        plan.run(None, None, C, w0.alpha, w0.beta, out, s, FUSED)
        rc, detail = plan.status(s)
        assert rc == G.OK, detail
        assert not flags(plan).any()
        bits = out_bits(out)
    want = O.emulate_rows(x0["A"], x0["B"], x0["C"], **oracle_kw(w0))
    assert np.array_equal(bits, want.view(bits.dtype))


def test_ineligible_configurations_take_the_serial_path():
    """KEEP_FLAGS (the flags stay set, as the serial reduce leaves them),
    unequal chunks (the m <= 64 decode shard) and W != 8 run serially with
    the same bits."""
    cases = [("keep_flags", dict((c[0], c[1]) for c in SMALL)["bias_row"], G.KEEP_FLAGS),
             ("decode", W70["decode"], 0),
             ("w4", I.with_shape(W70["llama8b"], W=4, M=2048, N=512, K=128), 0)]
    for name, w, extra in cases:
        x = I.make_inputs(w)
        dev = to_device(x, w)
        say("ineligible", name)
        with G.Plan(**desc_fields(w)) as plan:
            ref, got = new_out(w), new_out(w)
            run_checked(plan, dev, w, ref)
            run_checked(plan, dev, w, got, FUSED | extra)
            assert np.array_equal(out_bits(got), out_bits(ref))
            if extra & G.KEEP_FLAGS:
                assert flags(plan).all()
            else:
                assert not flags(plan).any()


# ------------------------------------------------------ last-arriver reduce
LAST = G.RUN_ALL | G.LAST_ARRIVER


def _serial_and_last(w, x, over, rounds=2, poison=False):
    """Serial bits, then `rounds` last-arriver passes (staging filled with
    NaN before the first: a summing workgroup that read a partial before
    its producer's release would put NaN into the output)."""
    dev = to_device(x, w)
    with G.Plan(**desc_fields(w, **over)) as plan:
        ref = new_out(w)
        run_checked(plan, dev, w, ref)
        if poison:
            hip().hipMemset.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t]
            assert hip().hipMemset(plan.info.staging, 0xFF, plan.info.staging_bytes) == 0
        got = new_out(w)
        for _ in range(rounds):
            run_checked(plan, dev, w, got, LAST)
            assert not flags(plan).any()
        return out_bits(ref), out_bits(got), out_to_f64(got, w)


@pytest.mark.parametrize("swizzle", [G.SWIZZLE_REMOTE_FIRST, G.SWIZZLE_IDENTITY,
                                     G.SWIZZLE_TILE_INTERLEAVED])
@pytest.mark.parametrize("name,w,over", SMALL, ids=[c[0] for c in SMALL])
def test_last_arriver_small_full_parity(name, w, over, swizzle):
    """Any tile order: every tile is summed once, by whichever of its W
    producers counts in last, bit for bit as the serial reduce sums it."""
    x = I.make_inputs(w)
    say("last arriver small", name, swizzle)
    serial, got_bits, got = _serial_and_last(w, x, dict(over, swizzle=swizzle), poison=True)
    assert np.array_equal(got_bits, serial)
    kw = oracle_kw(w)
    ref = O.reference_rows(x["A"], x["B"], x["C"], **kw)
    if over.get("staging_dtype") == G.STAGING_BF16:
        mag = sum(np.abs(O.partial_rows(x["A"], x["B"], x["C"], dtype=kw["dtype"],
                                        alpha=w.alpha, beta=w.beta, ldc=w.ldc, r=r))
                  for r in range(w.W))
        check_bf16_staging(got, ref, mag)
    else:
        check_tolerance(got, ref, w.dtype)


@pytest.mark.parametrize("name", ["straddle_2lvl", "full_c", "bf16_staging_straddle"])
def test_last_arriver_small_integer_exact(name):
    w, over = {c[0]: (c[1], c[2]) for c in SMALL}[name]
    if over.get("staging_dtype") == G.STAGING_BF16:
        w = I.with_shape(w, K=512)
    x = I.make_inputs(w, dist="ternary", c_dist="ternary")
    say("last arriver integer", name)
    serial, got, _ = _serial_and_last(w, x, over)
    em = O.emulate_rows(x["A"], x["B"], x["C"], **oracle_kw(w),
                        staging_dtype=over.get("staging_dtype", O.STAGING_F32))
    assert np.array_equal(got, em.view(got.dtype))
    assert np.array_equal(serial, got)


@pytest.mark.parametrize("name", ["llama70b", "ragged_2lvl"])
def test_last_arriver_full_size_sampled_parity(name):
    """Full size, staging poisoned with NaN first: the output has no NaN,
    equals the serial bits everywhere and the oracle on sampled rows and
    elements."""
    w = W70[name]
    rng = np.random.default_rng(41)
    x = I.make_inputs(w)
    say("last arriver full", name)
    serial, got_bits, got = _serial_and_last(w, x, {}, rounds=1, poison=True)
    assert np.isfinite(got).all()
    assert np.array_equal(got_bits, serial)
    kw = oracle_kw(w)
    rows = _sample_rows(w, rng)
    ref_rows = np.concatenate([O.reference_rows(x["A"], x["B"], x["C"], row_lo=i,
                                                row_hi=i + 1, **kw) for i in rows])
    check_tolerance(got[rows], ref_rows, w.dtype)
    ii = rng.integers(0, w.M, size=3000)
    jj = rng.integers(0, w.N, size=3000)
    ref_e = O.reference_elems(x["A"], x["B"], x["C"], ii=ii, jj=jj, **kw)
    check_tolerance(got[ii, jj], ref_e, w.dtype)


def test_last_arriver_flag_life_cycle_and_mixed_runs():
    """KEEP_FLAGS leaves every flag at 1 (the counters still reset); the
    next serial GEMM re-sets them and its reduce clears them; last-arriver,
    owner-fused and serial passes alternate on one stream without a host
    sync and give the same bits; a combined OVERLAP_REDUCE | LAST_ARRIVER
    is refused."""
    import torch
    w = dict((c[0], c[1]) for c in SMALL)["straddle_2lvl"]
    x = I.make_inputs(w)
    dev = to_device(x, w)
    say("last arriver life cycle")
    with G.Plan(**desc_fields(w)) as plan:
        ref = new_out(w)
        run_checked(plan, dev, w, ref)
        o = new_out(w)
        run_checked(plan, dev, w, o, LAST | G.KEEP_FLAGS)
        assert flags(plan).all()
        assert np.array_equal(out_bits(o), out_bits(ref))
        run_checked(plan, dev, w, o)
        assert not flags(plan).any()
        s = torch.cuda.current_stream()
        outs = [new_out(w) for _ in range(6)]
        for k, oo in enumerate(outs):
            plan.run(dev["A"], dev["B"], dev["C"], w.alpha, w.beta, oo, s,
                     (LAST, FUSED, G.RUN_ALL)[k % 3])
        rc, detail = plan.status(s)
        assert rc == G.OK, detail
        for oo in outs:
            assert np.array_equal(out_bits(oo), out_bits(ref))
        assert not flags(plan).any()
        rc = G.gemm_rs_run(plan.handle, dev["A"], dev["B"], dev["C"], w.alpha, w.beta, o, s,
                           LAST | G.OVERLAP_REDUCE)
        assert rc == G.ERR_INVALID_ARG
