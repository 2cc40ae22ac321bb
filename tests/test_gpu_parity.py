"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases compare every output element; the five workloads at full size
are checked on sampled rows and elements the oracle computes one by one,
plus properties that hold at any size (integer-valued exactness of every
staging slot, alpha scaling, poison-filled staging)."""
import numpy as np
import pytest

import oracle as O
from tensor_gemm_reduce_lds_amd import gemm_rs as G
from tensor_gemm_reduce_lds_amd import inputs as I

from gpu_util import (check_tolerance, d2h, desc_fields, flags, geometry, h2d,
                      new_out, oracle_kw, out_bits, out_to_f64, run_checked, say,
                      staging_rows, staging_slots, sync, to_device)

pytestmark = pytest.mark.gpu

W70 = I.WORKLOADS

# (name, workload) small enough for a full oracle comparison; they span
# several tiles, ragged last tile-rows and tiles that straddle chunks.
SMALL = [
    ("tiny_f32", W70["tiny_f32"]),
    ("bf16_256x256_ragged", I.with_shape(W70["llama8b"], W=8, M=800, N=512, K=256,
                                         tile_m=256, tile_n=256)),
    ("bf16_256x128_w4", I.with_shape(W70["llama8b"], W=4, M=520, N=384, K=192,
                                     tile_m=256, tile_n=128)),
    ("bf16_128x128_fullc", I.with_shape(W70["llama70b"], W=8, M=320, N=256, K=320,
                                        tile_m=128, tile_n=128, ldc=256,
                                        alpha=1.25, beta=0.75, c_std=1.0)),
    ("bf16_64x128_bias", I.with_shape(W70["llama70b"], W=8, M=64, N=1024, K=512,
                                      tile_m=64, tile_n=128)),
    ("bf16_two_level", I.with_shape(W70["ragged_2lvl"], M=560, N=512, K=128,
                                    tile_m=256, tile_n=256)),
    ("bf16_w1", I.with_shape(W70["llama8b"], W=1, M=256, N=256, K=64,
                             tile_m=256, tile_n=256)),
    ("bf16_mc1", I.with_shape(W70["llama8b"], W=8, M=8, N=128, K=64,
                              tile_m=64, tile_n=128)),
]


def _run_small(w, seed=0, **over):
    x = I.make_inputs(w, seed=seed)
    say("case", w.name, w.W, w.M, w.N, w.K, over)
    dev = to_device(x, w)
    with G.Plan(**desc_fields(w, **over)) as plan:
        out = new_out(w)
        run_checked(plan, dev, w, out)
        got = out_to_f64(out, w)
        assert not flags(plan).any()
        bits = out_bits(out)
    ref = O.reference_rows(x["A"], x["B"], x["C"], **oracle_kw(w))
    return got, ref, bits


@pytest.mark.parametrize("name,w", SMALL, ids=[s[0] for s in SMALL])
def test_small_full_parity(name, w):
    got, ref, _ = _run_small(w)
    mx, rf = check_tolerance(got, ref, w.dtype)
    say("  max_norm_err %.3e rel_F %.3e" % (mx, rf))


def test_materialised_two_level_matches_register_two_level():
    w = dict(SMALL)["bf16_two_level"]
    _, ref, bits_reg = _run_small(w)
    got, _, bits_mat = _run_small(w, materialize_sub=1)
    check_tolerance(got, ref, w.dtype)
    assert np.array_equal(bits_reg, bits_mat)


@pytest.mark.parametrize("groups", [2, 4])
def test_materialised_sub_buffer_layout(groups):
    """The materialised two-level mode writes each group's partial sum to
    sub[d][g][Mc][N].  With entries in {-1,0,1} every partial and every
    group sum is exact in float, so the buffer must hold, at the oracle's
    sub_offset(d, g, i, j), the sum of the oracle's partials of the ranks in
    group g, element for element (straddling tiles, ragged last tile-row)."""
    w = I.with_shape(W70["ragged_2lvl"], M=560, N=512, K=128, groups=groups,
                     tile_m=256, tile_n=256)
    x = I.make_inputs(w, dist="ternary", c_dist="ternary")
    dev = to_device(x, w)
    say("sub buffer layout", groups)
    kw = oracle_kw(w)
    with G.Plan(**desc_fields(w, materialize_sub=1)) as plan:
        out = new_out(w)
        run_checked(plan, dev, w, out)
        geom = geometry(w, plan)
        sub = d2h(plan.info.sub, plan.info.sub_bytes, np.float32)
        assert plan.info.sub_bytes == groups * w.M * w.N * 4
        bits = out_bits(out)
    parts = [O.partial_rows(x["A"], x["B"], x["C"], dtype=kw["dtype"], alpha=w.alpha,
                            beta=w.beta, ldc=w.ldc, r=r) for r in range(w.W)]
    L = w.W // groups
    jj = np.arange(w.N)
    for g in range(groups):
        want = sum(parts[r] for r in range(g * L, (g + 1) * L))
        for i in range(w.M):
            off = geom.sub_offset(geom.chunk_of_row(i), g, i, 0)
            assert off == geom.sub_offset(geom.chunk_of_row(i), g, i, jj[-1]) - (w.N - 1)
            got = sub[off:off + w.N].astype(np.float64)
            assert np.array_equal(got, want[i]), (g, i)
    em = O.emulate_rows(x["A"], x["B"], x["C"], **kw)
    assert np.array_equal(bits, em.view(bits.dtype))


@pytest.mark.parametrize("over", [dict(swizzle=G.SWIZZLE_SELF_FIRST),
                                  dict(swizzle=G.SWIZZLE_IDENTITY),
                                  dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED),
                                  dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED, group_m=3),
                                  dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED, interleave=3),
                                  dict(group_m=2), dict(group_m=3)])
def test_tile_order_does_not_change_bits(over):
    w = dict(SMALL)["bf16_256x256_ragged"]
    _, _, base = _run_small(w)
    _, _, other = _run_small(w, **over)
    assert np.array_equal(base, other)


# ---------------------------------------------------------------- tile order
ORDER_CASES = [
    ("tiny_f32", {}), ("llama8b", {}), ("llama70b", {}), ("decode", {}),
    ("ragged_2lvl", {}), ("llama70b", dict(group_m=4)),
    ("ragged_2lvl", dict(group_m=3)), ("llama8b", dict(swizzle=G.SWIZZLE_SELF_FIRST)),
    ("llama8b", dict(swizzle=G.SWIZZLE_IDENTITY)),
    # tile-interleaved: equal chunks, ragged chunks (straddling tiles, the
    # binary-searched tail), and decode (chunks without tiles)
    ("llama70b", dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED)),
    ("ragged_2lvl", dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED, group_m=3)),
    ("decode", dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED)),
    ("tiny_f32", dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED)),
    # q tiles per destination visit: equal chunks (closed form), ragged
    # chunks (binary-searched tail), and q beyond a chunk's tile count
    ("llama70b", dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED, interleave=16)),
    ("llama70b", dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED, interleave=32)),
    ("ragged_2lvl", dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED, group_m=3, interleave=5)),
    ("ragged_2lvl", dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED, interleave=100)),
    ("decode", dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED, interleave=3)),
    ("tiny_f32", dict(swizzle=G.SWIZZLE_TILE_INTERLEAVED, interleave=3)),
]


@pytest.mark.parametrize("name,over", ORDER_CASES)
def test_tile_order_matches_oracle_bit_exact(name, over):
    w = W70[name]
    say("tile order", name, over)
    with G.Plan(**desc_fields(w, **over)) as plan:
        got = plan.tile_order()
        want = geometry(w, plan).trace()
    assert np.array_equal(got, want)


@pytest.mark.parametrize("staging", [G.STAGING_F32, G.STAGING_BF16])
@pytest.mark.parametrize("name", ["llama8b", "llama70b", "decode", "ragged_2lvl"])
def test_staging_slot_layout_matches_rule(name, staging):
    """The plan's slot size and staging size follow the layout rule the
    oracle restates (padded slots only where a slot holds 8 MiB or more:
    the 1000-row chunks of the ragged shard)."""
    w = W70[name]
    say("staging layout", name, staging)
    with G.Plan(**desc_fields(w, staging_dtype=staging)) as plan:
        geom = geometry(w, plan)
        eb = 2 if staging == G.STAGING_BF16 else 4
        assert plan.info.slot_elems == geom.slot == O.staging_slot_elems(geom.Mc, w.N, eb)
        assert plan.info.staging_bytes == w.W * w.W * geom.slot * eb
        if name == "ragged_2lvl":
            assert geom.slot > geom.Mc * w.N


@pytest.mark.parametrize("swizzle", [G.SWIZZLE_REMOTE_FIRST, G.SWIZZLE_TILE_INTERLEAVED])
@pytest.mark.parametrize("case", ["bf16_256x256_ragged", "llama8b"])
def test_gemm_trace_matches_oracle(case, swizzle):
    """Every logical block (rank r's k-th tile) is run exactly once and takes
    the oracle's tile.  The launch hands each XCD one eighth of every rank's
    order, rank after rank (one tile per rank and XCD in the small case, 32
    in the 8B-like shard); the trace is indexed by logical block."""
    w = dict(SMALL)[case] if case in dict(SMALL) else W70[case]
    x = I.make_inputs(w)
    dev = to_device(x, w)
    say("gemm trace", w.name, "swizzle", swizzle)
    with G.Plan(**desc_fields(w, group_m=2, swizzle=swizzle)) as plan:
        out = new_out(w)
        run_checked(plan, dev, w, out, G.RUN_ALL | G.TRACE_TILES)
        tr = d2h(plan.info.trace, w.W * plan.info.T * 4, np.int32)
        assert np.array_equal(tr, geometry(w, plan).trace())


# -------------------------------------------------------- full-size workloads
FULL = ["llama8b", "llama70b", "decode", "ragged_2lvl"]


def _sample_rows(w, rng, per_chunk=2):
    Mc = w.M // w.W
    rows = set()
    for d in range(w.W):
        rows.add(d * Mc)
        rows.add(d * Mc + Mc - 1)
        for _ in range(per_chunk - 2):
            rows.add(d * Mc + int(rng.integers(0, Mc)))
    return sorted(rows)


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_parity(name):
    w = W70[name]
    rng = np.random.default_rng(100)
    x = I.make_inputs(w)
    say("full", name)
    dev = to_device(x, w)
    with G.Plan(**desc_fields(w)) as plan:
        out = new_out(w)
        run_checked(plan, dev, w, out)
        got = out_to_f64(out, w)
        assert not flags(plan).any()
    del dev
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
    assert np.isfinite(got).all()


def test_alpha_half_is_exact_half():
    # power-of-two scaling commutes with fp32 adds and bf16 rounding, so a
    # deterministic kernel gives exactly half the alpha=1 output
    w = W70["ragged_2lvl"]
    x = I.make_inputs(w)
    dev = to_device(x, w)
    say("alpha half", w.name)
    with G.Plan(**desc_fields(w)) as plan:
        o1, oh = new_out(w), new_out(w)
        run_checked(plan, dev, w, o1, alpha=1.0)
        run_checked(plan, dev, w, oh, alpha=0.5)
        a1, ah = out_to_f64(o1, w), out_to_f64(oh, w)
    assert np.array_equal(ah, 0.5 * a1)


@pytest.mark.parametrize("name", FULL)
def test_integer_inputs_bit_exact_everywhere(name):
    """Entries in {-1,0,1}: every partial is a small integer, exact in the
    fp32 MFMA accumulators and staging, so staging slots must equal the
    oracle's partials bit for bit and the output must equal emulate mode.
    Staging is filled with NaN first: any element the GEMM fails to write
    shows up."""
    w = W70[name]
    x = I.make_inputs(w, dist="ternary", c_dist="ternary")
    rng = np.random.default_rng(7)
    dev = to_device(x, w)
    say("integer exactness", name)
    kw = oracle_kw(w)
    with G.Plan(**desc_fields(w)) as plan:
        geom = geometry(w, plan)
        ptr, nbytes = plan.info.staging, plan.info.staging_bytes
        import ctypes
        from gpu_util import hip
        hip().hipMemset.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t]
        assert hip().hipMemset(ptr, 0xFF, nbytes) == 0
        out = new_out(w)
        run_checked(plan, dev, w, out, G.RUN_GEMM)
        assert flags(plan).all()
        st = staging_slots(plan, geom)
        assert not np.isnan(st).any(), "staging elements left unwritten"
        del st
        rows = _sample_rows(w, rng, per_chunk=3)
        for i in rows:
            d = i // geom.Mc
            for r in range(w.W):
                want = O.partial_rows(x["A"], x["B"], x["C"], dtype=kw["dtype"],
                                      alpha=w.alpha, beta=w.beta, ldc=w.ldc, r=r,
                                      row_lo=i, row_hi=i + 1)[0].astype(np.float32)
                got = staging_rows(plan, geom, d, r, i - d * geom.Mc, 1)[0]
                assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (i, r)
        run_checked(plan, dev, w, out, G.RUN_REDUCE)
        assert not flags(plan).any()
        bits = out_bits(out)
    for i in rows:
        em = O.emulate_rows(x["A"], x["B"], x["C"], row_lo=i, row_hi=i + 1, **kw)
        assert np.array_equal(bits[i], em[0].view(bits.dtype)), i


# ------------------------------------------------------------- edge cases
EDGE = [
    # non-power-of-two W: the reduce's runtime-W path
    ("w3", I.with_shape(W70["llama8b"], W=3, M=3 * 100, N=256, K=128,
                        tile_m=128, tile_n=128), {}),
    # many ranks: 64 slots per element, Mc = 2 (every tile straddles chunks)
    ("w64", I.with_shape(W70["llama8b"], W=64, M=128, N=128, K=64,
                         tile_m=64, tile_n=128), {}),
    # two-level with 1, 4 and 8 groups (G=1 and G=W are the flat order)
    ("g1", I.with_shape(W70["ragged_2lvl"], M=8 * 40, N=256, K=128, groups=1,
                        tile_m=128, tile_n=128), {}),
    ("g4", I.with_shape(W70["ragged_2lvl"], M=8 * 40, N=256, K=128, groups=4,
                        tile_m=128, tile_n=128), {}),
    ("g8_mat", I.with_shape(W70["ragged_2lvl"], M=8 * 40, N=256, K=128, groups=8,
                            tile_m=128, tile_n=128), dict(materialize_sub=1)),
    ("g4_mat_decode", I.with_shape(W70["ragged_2lvl"], M=64, N=512, K=256, groups=4,
                                   tile_m=64, tile_n=128), dict(materialize_sub=1)),
    # fp32 with several tiles and a ragged last tile-row (M = 4*50)
    ("f32_ragged", I.with_shape(W70["tiny_f32"], W=4, M=200, N=192, K=128), {}),
    # fp32 with a full C matrix and alpha/beta
    ("f32_fullc", I.with_shape(W70["tiny_f32"], W=2, M=128, N=128, K=64, has_c=True,
                               ldc=128, alpha=0.5, beta=2.0, c_std=1.0), {}),
    # group_m far beyond the tile-row count (clamped: same order)
    ("group_big", I.with_shape(W70["llama8b"], W=8, M=800, N=512, K=64,
                               tile_m=256, tile_n=256), dict(group_m=1000)),
    # single K step
    ("k64", I.with_shape(W70["llama70b"], W=8, M=512, N=512, K=64,
                         tile_m=256, tile_n=256), {}),
]


@pytest.mark.parametrize("name,w,over", EDGE, ids=[e[0] for e in EDGE])
def test_edge_full_parity(name, w, over):
    got, ref, _ = _run_small(w, **over)
    mx, rf = check_tolerance(got, ref, w.dtype)
    say("  max_norm_err %.3e rel_F %.3e" % (mx, rf))


def test_edge_tile_orders_bit_exact():
    for name, w, over in EDGE:
        for swz, q in ((G.SWIZZLE_REMOTE_FIRST, 0), (G.SWIZZLE_TILE_INTERLEAVED, 0),
                       (G.SWIZZLE_TILE_INTERLEAVED, 3)):
            with G.Plan(**desc_fields(w, **dict(over, swizzle=swz, interleave=q))) as plan:
                assert np.array_equal(plan.tile_order(), geometry(w, plan).trace()), \
                    (name, swz, q)


@pytest.mark.parametrize("dtype,ldc", [("bf16", 0), ("bf16", 256), ("f32", 0)])
def test_k0_empty_sum_is_beta_c(dtype, ldc):
    """K = 0: the empty sum.  Every partial is 0, so the output is beta*C
    (added once, by the chunk owner), bit for bit as the oracle's float
    pipeline gives it; A and B are never read and are passed as NULL."""
    import torch
    base = W70["llama70b"] if dtype == "bf16" else W70["tiny_f32"]
    w = I.with_shape(base, W=8, M=512, N=256, K=64, has_c=True, ldc=ldc,
                     alpha=1.5, beta=0.75, c_std=1.0,
                     tile_m=256 if dtype == "bf16" else 64,
                     tile_n=256 if dtype == "bf16" else 64)
    x = I.make_inputs(w)
    C = x["C"]
    A0 = x["A"][:, :, :0]
    B0 = x["B"][:, :0, :]
    say("k0", dtype, ldc)
    Cd = torch.from_numpy(C.view(np.int16) if C.dtype == np.uint16 else C).to("cuda:0")
    with G.Plan(**desc_fields(w, K=0)) as plan:
        out = new_out(w)
        s = torch.cuda.current_stream()
        plan.run(None, None, Cd, w.alpha, w.beta, out, s)
        rc, detail = plan.status(s)
        assert rc == G.OK, (rc, detail)
        assert not flags(plan).any()
        bits = out_bits(out)
    kw = oracle_kw(w)
    want = O.emulate_rows(A0, B0, C, **kw)
    assert np.array_equal(bits, want.view(bits.dtype))
    ref = O.reference_rows(A0, B0, C, **kw)
    Cf = O.bf16_bits_to_f64(C) if dtype == "bf16" else C.astype(np.float64)
    np.testing.assert_array_equal(ref, 0.75 * (np.broadcast_to(Cf, (w.M, w.N)) if ldc == 0
                                               else Cf[:, :w.N]))


@pytest.mark.parametrize("tile", [(256, 128), (128, 128)])
def test_llama70b_other_tiles_sampled(tile):
    """The 70B-like shard with the smaller tile shapes (sampled elements)."""
    w = I.with_shape(W70["llama70b"], tile_m=tile[0], tile_n=tile[1])
    rng = np.random.default_rng(5)
    x = I.make_inputs(w)
    say("70b tile", tile)
    dev = to_device(x, w)
    with G.Plan(**desc_fields(w)) as plan:
        out = new_out(w)
        run_checked(plan, dev, w, out)
        got = out_to_f64(out, w)
    del dev
    ii = rng.integers(0, w.M, size=2000)
    jj = rng.integers(0, w.N, size=2000)
    ref = O.reference_elems(x["A"], x["B"], x["C"], ii=ii, jj=jj, **oracle_kw(w))
    check_tolerance(got[ii, jj], ref, w.dtype)


def test_staging_of_4gib_uses_64bit_slot_loads():
    """A staging of 2^32 bytes (W=8, M=16384, N=8192) is past what the
    reduce's 32-bit buffer offsets reach, so the reduce reads the slots
    through 64-bit pointers, and the epilogue's slot offsets pass 2^31
    elements: integer inputs must give the oracle's emulated bits on every
    chunk's first and last row and on random rows, and Gaussian inputs the
    parity bar on sampled elements."""
    w = I.with_shape(W70["llama70b"], M=16384, K=128)
    rng = np.random.default_rng(9)
    kw = oracle_kw(w)
    for dist in ("ternary", "normal"):
        x = I.make_inputs(w, dist=dist, c_dist=dist) if dist == "ternary" else I.make_inputs(w)
        say("4 GiB staging", dist)
        dev = to_device(x, w)
        with G.Plan(**desc_fields(w)) as plan:
            assert plan.info.staging_bytes == 1 << 32
            out = new_out(w)
            run_checked(plan, dev, w, out)
            assert not flags(plan).any()
            bits = out_bits(out) if dist == "ternary" else None
            got = out_to_f64(out, w) if dist == "normal" else None
        del dev, out
        if dist == "ternary":
            for i in _sample_rows(w, rng, per_chunk=3):
                em = O.emulate_rows(x["A"], x["B"], x["C"], row_lo=i, row_hi=i + 1, **kw)
                assert np.array_equal(bits[i], em[0].view(bits.dtype)), i
        else:
            ii = rng.integers(0, w.M, size=2000)
            jj = rng.integers(0, w.N, size=2000)
            ref = O.reference_elems(x["A"], x["B"], x["C"], ii=ii, jj=jj, **kw)
            check_tolerance(got[ii, jj], ref, w.dtype)
