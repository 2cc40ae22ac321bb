"""Pins for the CPU oracle: brute force, closed forms, library routines and
the values the pages print.  CPU only (no GPU marker)."""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from tensor_gemm_reduce_lds_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_f32(rng, shape, lo=-1.0, hi=1.0):
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


# ---------------------------------------------------------------- bf16 RNE
def test_bf16_rne_ties_and_near_ties():
    # 0x3F808000 sits exactly between 0x3F80 and 0x3F81: ties to even (0x3F80)
    # 0x3F818000 sits between 0x3F81 and 0x3F82: ties to even (0x3F82)
    # 0xBF808000 is the negative tie: ties to even magnitude (0xBF80)
    # 0x3F808008 is just above the tie: rounds up (0x3F81)
    bits = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F808008,
                     0x3F807FFF, 0x00000000, 0x80000000], dtype=np.uint32)
    got = O.bf16_rne(bits.view(np.float32))
    assert got.tolist() == [0x3F80, 0x3F82, 0xBF80, 0x3F81, 0x3F80, 0, 0x8000]


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # add specials: +-inf, largest finite (rounds to inf), denormals, ties
    extra = np.array([0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x00000001,
                      0x00008000, 0x00018000, 0x7F7F8000, 0x7F7F7FFF],
                     dtype=np.uint32)
    bits = np.concatenate([bits, extra])
    x = bits.view(np.float32)
    got = O.bf16_rne(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN stays NaN
    back = (got[nan].astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(back))


# -------------------------------------------------------- reference values
def _brute_force(A, B, C, alpha, beta, ldc):
    """Exact rational arithmetic, straight from the definition:
    out[i][j] = alpha * sum_r sum_k A_r[i][k] B_r[k][j] + beta * C[i][j]."""
    W, M, K = A.shape
    N = B.shape[2]
    out = np.empty((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for r in range(W):
                for k in range(K):
                    s += Fraction(float(A[r, i, k])) * Fraction(float(B[r, k, j]))
            v = Fraction(alpha) * s
            if C is not None:
                c = C[j] if ldc == 0 else C[i, j]
                v += Fraction(beta) * Fraction(float(c))
            out[i, j] = v
    return out


@pytest.mark.parametrize("ldc_mode", ["none", "broadcast", "full"])
def test_reference_brute_force_tiny(ldc_mode):
    rng = np.random.default_rng(2)
    W, M, K, N = 2, 4, 5, 3
    A = _rand_f32(rng, (W, M, K))
    B = _rand_f32(rng, (W, K, N))
    C, ldc = None, 0
    if ldc_mode == "broadcast":
        C = _rand_f32(rng, (N,))
    elif ldc_mode == "full":
        C, ldc = _rand_f32(rng, (M, N)), N
    alpha, beta = 0.75, -1.25
    got = O.reference_rows(A, B, C, dtype=O.F32, alpha=alpha, beta=beta, ldc=ldc)
    exact = _brute_force(A, B, C, alpha, beta, ldc)
    for i, j in itertools.product(range(M), range(N)):
        assert abs(Fraction(got[i, j]) - exact[i, j]) <= Fraction(1, 10**12)
    # the element-wise entry point gives the same numbers
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    e = O.reference_elems(A, B, C, dtype=O.F32, alpha=alpha, beta=beta,
                          ldc=ldc, ii=ii.ravel(), jj=jj.ravel())
    np.testing.assert_allclose(e, got.ravel(), rtol=1e-13, atol=1e-13)


def test_reference_exact_on_small_integers():
    # integer inputs: fp64 is exact, so the oracle must equal integer math
    rng = np.random.default_rng(3)
    W, M, K, N = 3, 6, 7, 5
    A = rng.integers(-3, 4, size=(W, M, K)).astype(np.float32)
    B = rng.integers(-3, 4, size=(W, K, N)).astype(np.float32)
    got = O.reference_rows(A, B, dtype=O.F32)
    Ai, Bi = A.astype(np.int64), B.astype(np.int64)
    ref = sum(Ai[r] @ Bi[r] for r in range(W))
    assert np.array_equal(got, ref.astype(np.float64))


def test_sum_of_partials_equals_full_gemm():
    # sum_r A_r B_r == [A_0 .. A_{W-1}] (along K) @ [B_0; ..; B_{W-1}] (along K)
    rng = np.random.default_rng(4)
    W, M, K, N = 4, 8, 16, 12
    A = _rand_f32(rng, (W, M, K))
    B = _rand_f32(rng, (W, K, N))
    alpha = 1.5
    got = O.reference_rows(A, B, dtype=O.F32, alpha=alpha)
    A_full = np.concatenate([A[r] for r in range(W)], axis=1).astype(np.float64)
    B_full = np.concatenate([B[r] for r in range(W)], axis=0).astype(np.float64)
    np.testing.assert_allclose(got, alpha * (A_full @ B_full), rtol=1e-12, atol=1e-12)


def test_w1_bf16_is_plain_gemm():
    rng = np.random.default_rng(5)
    M, K, N = 16, 64, 24
    A = I.to_bf16_bits(rng.standard_normal((1, M, K)).astype(np.float32))
    B = I.to_bf16_bits(rng.standard_normal((1, K, N)).astype(np.float32))
    got = O.reference_rows(A, B, dtype=O.BF16)
    Af = I.bf16_bits_to_f32(A[0]).astype(np.float64)
    Bf = I.bf16_bits_to_f32(B[0]).astype(np.float64)
    np.testing.assert_allclose(got, Af @ Bf, rtol=1e-12, atol=1e-12)


def test_partials_are_rank_products():
    rng = np.random.default_rng(6)
    W, M, K, N = 4, 8, 8, 6
    A = _rand_f32(rng, (W, M, K))
    B = _rand_f32(rng, (W, K, N))
    for r in range(W):
        got = O.partial_rows(A, B, dtype=O.F32, alpha=-2.0, r=r)
        ref = -2.0 * (A[r].astype(np.float64) @ B[r].astype(np.float64))
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("ldc", [0, 6])
def test_bias_added_once_by_chunk_owner(ldc):
    W, M, K, N = 4, 8, 3, 6     # Mc = 2
    A = np.zeros((W, M, K), dtype=np.float32)
    B = np.ones((W, K, N), dtype=np.float32)
    rng = np.random.default_rng(7)
    C = _rand_f32(rng, (N,) if ldc == 0 else (M, ldc))
    beta = 0.5
    Cm = np.broadcast_to(C, (M, N)) if ldc == 0 else C[:, :N]
    out = O.reference_rows(A, B, C, dtype=O.F32, beta=beta, ldc=ldc)
    np.testing.assert_array_equal(out, beta * Cm.astype(np.float64))
    for r in range(W):
        p = O.partial_rows(A, B, C, dtype=O.F32, beta=beta, ldc=ldc, r=r)
        for i in range(M):
            expect = beta * Cm[i].astype(np.float64) if i // 2 == r else 0.0
            np.testing.assert_array_equal(p[i], np.broadcast_to(expect, (N,)))


def test_alpha0_beta1_returns_c_bits():
    rng = np.random.default_rng(8)
    W, M, K, N = 4, 8, 64, 16
    A = I.to_bf16_bits(rng.standard_normal((W, M, K)).astype(np.float32))
    B = I.to_bf16_bits(rng.standard_normal((W, K, N)).astype(np.float32))
    C = I.to_bf16_bits(rng.standard_normal((N,)).astype(np.float32))
    got = O.emulate_rows(A, B, C, dtype=O.BF16, alpha=0.0, beta=1.0, ldc=0)
    assert np.array_equal(got, np.broadcast_to(C, (M, N)))


@pytest.mark.parametrize("ldc", [0, 16])
def test_k0_empty_sum_is_beta_c(ldc):
    """K = 0: every partial product is the empty sum 0, so the output is
    beta*C, counted once (closed form), and in the float pipeline the
    bfloat16 rounding of the float beta*C (other ranks add exact zeros)."""
    rng = np.random.default_rng(9)
    W, M, N = 4, 8, 16
    A = np.zeros((W, M, 0), dtype=np.uint16)
    B = np.zeros((W, 0, N), dtype=np.uint16)
    C = I.to_bf16_bits(rng.standard_normal((N,) if ldc == 0 else (M, ldc)).astype(np.float32))
    Cf = O.bf16_bits_to_f64(C)
    Cm = np.broadcast_to(Cf, (M, N)) if ldc == 0 else Cf[:, :N]
    beta = 0.75
    ref = O.reference_rows(A, B, C, dtype=O.BF16, alpha=1.5, beta=beta, ldc=ldc)
    np.testing.assert_array_equal(ref, beta * Cm)
    for order, groups in ((O.FLAT, 1), (O.TWO_LEVEL, 2)):
        got = O.emulate_rows(A, B, C, dtype=O.BF16, alpha=1.5, beta=beta, ldc=ldc,
                             order=order, groups=groups)
        want = O.bf16_rne((beta * Cm).astype(np.float32)).reshape(M, N)
        assert np.array_equal(got, want)
    # no C: all zeros
    z = O.reference_rows(A, B, None, dtype=O.BF16, alpha=1.5)
    assert not z.any()


# ------------------------------------------------------------ reduce order
def _order_case(dtype):
    # rank r's partial at every element is v[r]: A_r = v[r] (K = 1), B_r = 1
    v = np.array([2.0**24, 1, 1, 1, 1, 1, 1, -2.0**24], dtype=np.float32)
    W, M, K, N = 8, 8, 1, 4
    A = np.broadcast_to(v[:, None, None], (W, M, K)).astype(np.float32)
    B = np.ones((W, K, N), dtype=np.float32)
    if dtype == O.BF16:
        A, B = I.to_bf16_bits(A), I.to_bf16_bits(B)
    return v, A, B


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
def test_reduce_order_closed_form(dtype):
    # float: 2^24 + 1 == 2^24 (tie to even), so the flat ascending sum loses
    # every +1 and ends at 0; the two-level order keeps 1+1+1 in group 1 and
    # ends at 3; the exact sum is 6.
    v, A, B = _order_case(dtype)
    ref = O.reference_rows(A, B, dtype=dtype)
    assert np.all(ref == 6.0)
    flat = O.emulate_rows(A, B, dtype=dtype, order=O.FLAT)
    two = O.emulate_rows(A, B, dtype=dtype, order=O.TWO_LEVEL, groups=2)
    if dtype == O.BF16:
        flat, two = O.bf16_bits_to_f64(flat), O.bf16_bits_to_f64(two)
    assert np.all(flat == 0.0) and np.all(two == 3.0)
    S = np.broadcast_to(v[:, None], (8, 5)).astype(np.float32)
    assert np.all(O.reduce_emulate(S, order=O.FLAT) == 0)
    assert np.all(O.reduce_emulate(S, order=O.TWO_LEVEL, groups=2) == 0x4040)
    assert np.all(O.reduce_emulate(S, order=O.TWO_LEVEL, groups=2,
                                   out_bf16=False) == 3.0)
    # G = 1 and G = W are both the flat ascending order
    assert np.all(O.reduce_emulate(S, order=O.TWO_LEVEL, groups=1) == 0)
    assert np.all(O.reduce_emulate(S, order=O.TWO_LEVEL, groups=8) == 0)
    # G = 4: (2^24+1) + (1+1) + (1+1) + (1-2^24) -> 2^24 + 2 + 2 - (2^24-1) = 5
    assert np.all(O.reduce_emulate(S, order=O.TWO_LEVEL, groups=4,
                                   out_bf16=False) == 5.0)


def test_emulate_equals_rounded_reference_on_integers():
    w = I.with_shape(I.WORKLOADS["llama8b"], M=64, N=128, K=128, W=8)
    x = I.make_inputs(w, seed=11, dist="ternary")
    ref = O.reference_rows(x["A"], x["B"], dtype=O.BF16)
    em = O.emulate_rows(x["A"], x["B"], dtype=O.BF16)
    assert np.array_equal(em, O.bf16_rne(ref.astype(np.float32)).reshape(em.shape))


def test_emulate_close_to_reference_on_floats():
    w = I.with_shape(I.WORKLOADS["llama8b"], M=32, N=64, K=128)
    x = I.make_inputs(w, seed=12)
    ref = O.reference_rows(x["A"], x["B"], dtype=O.BF16)
    em = O.bf16_bits_to_f64(O.emulate_rows(x["A"], x["B"], dtype=O.BF16))
    assert O.max_norm_err(em.reshape(ref.shape), ref) < 2**-8


# ---------------------------------------------------------- tile map, swizzle
def _geom_cases():
    cases = [
        (I.WORKLOADS["tiny_f32"], 64, 64),
        (I.WORKLOADS["llama8b"], 256, 256),
        (I.WORKLOADS["llama70b"], 256, 256),
        (I.WORKLOADS["decode"], 64, 128),
        (I.WORKLOADS["ragged_2lvl"], 256, 256),
    ]
    return [(w.M, w.N, w.K, w.W, bm, bn) for w, bm, bn in cases]


def _random_geoms(n=60):
    rng = np.random.default_rng(13)
    out = []
    for _ in range(n):
        W = int(rng.integers(1, 9))
        Mc = int(rng.integers(1, 70))
        bm = int(rng.choice([8, 16, 32, 64]))
        bn = int(rng.choice([8, 16]))
        tn = int(rng.integers(1, 5))
        out.append((W * Mc, bn * tn, 64, W, bm, bn))
    return out


@pytest.mark.parametrize("swz", [O.REMOTE_FIRST, O.SELF_FIRST, O.IDENTITY])
@pytest.mark.parametrize("g", [1, 2, 3])
def test_seq_is_permutation(swz, g):
    for (M, N, K, W, bm, bn) in _geom_cases() + _random_geoms():
        G = O.Geometry(M, N, K, W, bm, bn, group_m=g, swizzle=swz)
        tab = G.seq_table()
        assert tab.shape == (W, G.T)
        for r in range(W):
            assert sorted(tab[r].tolist()) == list(range(G.T))
            # tiles come chunk by chunk in dest order
            owners = [G.owner(t // G.tiles_n) for t in tab[r]]
            steps = {G.dest(r, s): s for s in range(W)}
            s_of = [steps[d] for d in owners]
            assert s_of == sorted(s_of)
        tr = G.trace()
        assert sorted(tr.tolist()) == sorted(list(range(G.T)) * W)


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8, 16, 64])
def test_dest_is_latin_square_remote_first(W):
    G = O.Geometry(W * 4, 64, 64, W, 4, 64)
    D = np.array([[G.dest(r, s) for s in range(W)] for r in range(W)])
    for s in range(W):
        assert sorted(D[:, s]) == list(range(W))   # distinct targets per step
    for r in range(W):
        assert sorted(D[r]) == list(range(W))      # every chunk once per rank
        assert D[r, W - 1] == r                    # local chunk last
        if W > 1:
            assert D[r, 0] != r                    # remote chunk first


def test_self_first_matches_page_example():
    rows = {}
    with open(os.path.join(GOLDEN, "swizzle_rank_offset_w8.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(":")
                rows[int(k)] = [int(x) for x in v.split()]
    G = O.Geometry(8 * 256, 256, 64, 8, 256, 256, swizzle=O.SELF_FIRST)
    for r, want in rows.items():
        assert [G.dest(r, s) for s in range(8)] == want
    # the default order is the same rotation shifted by one step: local last
    R = O.Geometry(8 * 256, 256, 64, 8, 256, 256, swizzle=O.REMOTE_FIRST)
    for r, want in rows.items():
        assert [R.dest(r, s) for s in range(8)] == want[1:] + want[:1]


def test_tile_interleaved_hand_examples():
    # W=2, two chunks of one tile-row each, 2 tile-columns: chunk 0 holds
    # tiles [0, 1], chunk 1 holds [2, 3].  Rank 0 visits chunk 1 then chunk
    # 0, one tile per visit; rank 1 visits chunk 0 then chunk 1.
    G = O.Geometry(4, 4, 64, 2, 2, 2, swizzle=O.TILE_INTERLEAVED)
    assert G.seq(0) == [2, 0, 3, 1]
    assert G.seq(1) == [0, 2, 1, 3]
    assert G.trace().tolist() == [2, 0, 0, 2, 3, 1, 1, 3]
    # unequal chunks: M=6, W=2 (Mc=3), 2-row tiles: tile-rows 0 and 1 start
    # in chunk 0, tile-row 2 in chunk 1; one tile-column.  Chunk 0 = [0, 1],
    # chunk 1 = [2]; once chunk 1 is used up only chunk 0 is left.
    G = O.Geometry(6, 16, 64, 2, 2, 16, swizzle=O.TILE_INTERLEAVED)
    assert [G.chunk_tiles(d) for d in range(2)] == [[0, 1], [2]]
    assert G.seq(0) == [2, 0, 1]
    assert G.seq(1) == [0, 2, 1]


@pytest.mark.parametrize("g", [1, 2, 4])
def test_tile_interleaved_properties(g):
    """Every rank's order is a permutation that keeps each chunk's own tile
    order; with equal chunks the k-th tile of rank r lies in chunk
    (r + 1 + k) mod W, so in every step the W ranks write W different
    chunks and every chunk receives one tile per rank in every W steps."""
    for (M, N, K, W, bm, bn) in _geom_cases() + _random_geoms():
        G = O.Geometry(M, N, K, W, bm, bn, group_m=g, swizzle=O.TILE_INTERLEAVED)
        tab = G.seq_table()
        counts = [len(G.chunk_tiles(d)) for d in range(W)]
        for r in range(W):
            assert sorted(tab[r].tolist()) == list(range(G.T))
            for d in range(W):
                mine = [t for t in tab[r] if G.owner(t // G.tiles_n) == d]
                assert mine == G.chunk_tiles(d)
        if len(set(counts)) == 1:
            for r in range(W):
                for k in range(G.T):
                    assert G.owner(tab[r, k] // G.tiles_n) == (r + 1 + k) % W
            for k in range(G.T):
                assert sorted(G.owner(t // G.tiles_n) for t in tab[:, k]) == list(range(W))


def test_tile_interleaved_blocks_hand_examples():
    # W=2, one tile-row per chunk, 4 tile-columns: chunk 0 = [0, 1, 2, 3],
    # chunk 1 = [4, 5, 6, 7].  Rank 0 visits chunk 1 then chunk 0, rank 1
    # chunk 0 then chunk 1, taking q tiles per visit.
    G = O.Geometry(4, 8, 64, 2, 2, 2, swizzle=O.TILE_INTERLEAVED, interleave=2)
    assert [G.chunk_tiles(d) for d in range(2)] == [[0, 1, 2, 3], [4, 5, 6, 7]]
    assert G.seq(0) == [4, 5, 0, 1, 6, 7, 2, 3]
    assert G.seq(1) == [0, 1, 4, 5, 2, 3, 6, 7]
    assert G.trace().tolist() == [4, 0, 5, 1, 0, 4, 1, 5, 6, 2, 7, 3, 2, 6, 3, 7]
    # q = 3: the second round has one tile left in each chunk
    G = O.Geometry(4, 8, 64, 2, 2, 2, swizzle=O.TILE_INTERLEAVED, interleave=3)
    assert G.seq(0) == [4, 5, 6, 0, 1, 2, 7, 3]
    assert G.seq(1) == [0, 1, 2, 4, 5, 6, 3, 7]
    # unequal chunks [0, 1] and [2] with q = 2
    G = O.Geometry(6, 16, 64, 2, 2, 16, swizzle=O.TILE_INTERLEAVED, interleave=2)
    assert G.seq(0) == [2, 0, 1]
    assert G.seq(1) == [0, 1, 2]


@pytest.mark.parametrize("q", [1, 2, 3, 16])
def test_tile_interleaved_blocks_properties(q):
    """Every order is a permutation that keeps each chunk's own order; with
    equal chunks of a multiple of q tiles, rank r's k-th tile lies in chunk
    (r + 1 + k // q) mod W; q of at least the largest chunk is the
    chunk-major remote-first order; q = 1 is one tile per visit."""
    for (M, N, K, W, bm, bn) in _geom_cases() + _random_geoms():
        for g in (1, 3):
            G = O.Geometry(M, N, K, W, bm, bn, group_m=g, swizzle=O.TILE_INTERLEAVED,
                           interleave=q)
            tab = G.seq_table()
            counts = [len(G.chunk_tiles(d)) for d in range(W)]
            for r in range(W):
                assert sorted(tab[r].tolist()) == list(range(G.T))
                for d in range(W):
                    mine = [t for t in tab[r] if G.owner(t // G.tiles_n) == d]
                    assert mine == G.chunk_tiles(d)
            if len(set(counts)) == 1 and counts[0] % q == 0:
                for r in range(W):
                    for k in range(G.T):
                        assert G.owner(tab[r, k] // G.tiles_n) == (r + 1 + k // q) % W
            big = O.Geometry(M, N, K, W, bm, bn, group_m=g, swizzle=O.TILE_INTERLEAVED,
                             interleave=max(counts))
            rf = O.Geometry(M, N, K, W, bm, bn, group_m=g, swizzle=O.REMOTE_FIRST)
            assert np.array_equal(big.seq_table(), rf.seq_table())


def test_identity_swizzle_same_order_everywhere():
    G = O.Geometry(8 * 512, 1024, 64, 8, 256, 256, swizzle=O.IDENTITY)
    tab = G.seq_table()
    assert all(np.array_equal(tab[0], tab[r]) for r in range(8))
    assert tab[0].tolist() == list(range(G.T))


def test_tiny_worked_example():
    # W=2, M=128, N=256, 64x64 tiles: tiles_m=2, tiles_n=4, T=8, Mc=64.
    # tile-row 0 belongs to chunk 0, tile-row 1 to chunk 1.
    # rank 0: remote chunk 1 first (tiles 4..7), then local chunk 0 (0..3);
    # rank 1: remote chunk 0 first (0..3), then chunk 1 (4..7).
    G = O.Geometry(128, 256, 512, 2, 64, 64)
    assert G.T == 8 and G.Mc == 64
    assert G.seq(0) == [4, 5, 6, 7, 0, 1, 2, 3]
    assert G.seq(1) == [0, 1, 2, 3, 4, 5, 6, 7]
    assert G.trace().tolist() == [4, 0, 5, 1, 6, 2, 7, 3, 0, 4, 1, 5, 2, 6, 3, 7]


def test_group_m_order_hand_example():
    # W=1, 4 tile-rows x 3 tile-columns, groups of 2 tile-rows:
    # (tm,tn) order (0,0)(1,0)(0,1)(1,1)(0,2)(1,2)(2,0)(3,0)(2,1)(3,1)(2,2)(3,2)
    G = O.Geometry(4 * 16, 3 * 16, 64, 1, 16, 16, group_m=2)
    assert G.seq(0) == [0, 3, 1, 4, 2, 5, 6, 9, 7, 10, 8, 11]
    # a ragged last group (3 tile-rows, g=2): the lone last row goes alone
    G = O.Geometry(3 * 16, 2 * 16, 64, 1, 16, 16, group_m=2)
    assert G.seq(0) == [0, 2, 1, 3, 4, 5]


def test_ragged_straddle_rows():
    w = I.WORKLOADS["ragged_2lvl"]
    G = O.Geometry(w.M, w.N, w.K, w.W, 256, 256)
    assert G.Mc == 1000 and G.tiles_m == 32
    assert G.straddling_tile_rows() == [3, 7, 11, 15, 19, 23, 27]
    assert G.tile_rows(31) == (7936, 8000)
    assert [G.chunk_of_row(i) for i in (999, 1000, 7999)] == [0, 1, 7]


def test_decode_degenerate_order():
    # M=64 with 64-row tiles: one tile-row, owned by chunk 0; every rank's
    # order is the same 64 tiles, and chunks 1..7 own no tile-row
    w = I.WORKLOADS["decode"]
    G = O.Geometry(w.M, w.N, w.K, w.W, 64, 128)
    assert G.T == 64 and G.straddling_tile_rows() == [0]
    for r in range(8):
        assert G.seq(r) == list(range(64))
    assert [len(G.chunk_tile_rows(d)) for d in range(8)] == [1] + [0] * 7


def test_staging_offsets_are_a_bijection():
    for (M, N, K, W, bm, bn) in _random_geoms(25):
        G = O.Geometry(M, N, K, W, bm, bn)
        seen = np.zeros(W * M * N, dtype=np.int32)
        # every element of every rank's output, walked tile by tile
        for r in range(W):
            for t in range(G.T):
                tm, tn = divmod(t, G.tiles_n)
                lo, hi = G.tile_rows(tm)
                for i in range(lo, hi):
                    d = G.chunk_of_row(i)
                    for j in range(tn * bn, (tn + 1) * bn):
                        seen[G.staging_offset(d, r, i, j)] += 1
        assert np.all(seen == 1)


def test_staging_offset_hand_values():
    # W=2, M=4 (Mc=2), N=3: S[d][r][il][j]
    G = O.Geometry(4, 3, 64, 2, 2, 3)
    assert G.staging_offset(0, 0, 0, 0) == 0
    assert G.staging_offset(0, 1, 1, 2) == (1 * 2 + 1) * 3 + 2
    assert G.staging_offset(1, 0, 2, 0) == (2 * 2 + 0) * 3
    assert G.staging_offset(1, 1, 3, 2) == 4 * 2 * 3 - 1


def test_staging_slot_size_hand_values():
    # below 8 MiB a slot is exactly Mc*N elements
    assert O.staging_slot_elems(2, 3, 4) == 6
    assert O.staging_slot_elems(8, 8192, 4) == 8 * 8192
    assert O.staging_slot_elems(255, 8192, 4) == 255 * 8192          # 7.97 MiB
    # 8 MiB and 32 MiB are already multiples of 512 KiB
    assert O.staging_slot_elems(256, 8192, 4) == 256 * 8192
    assert O.staging_slot_elems(1024, 8192, 4) == 1024 * 8192
    # 1000 rows of 8192 fp32 = 32,768,000 B = 62.5 x 512 KiB -> 63 x 512 KiB
    # = 33,030,144 B = 8,257,536 floats (1008 rows)
    assert O.staging_slot_elems(1000, 8192, 4) == 8257536
    # the same rows in bfloat16: 16,384,000 B = 31.25 x 512 KiB -> 32 x
    # 512 KiB = 16 MiB = 8,388,608 halves (1024 rows)
    assert O.staging_slot_elems(1000, 8192, 2) == 8388608
    # the rounding adds less than 512 KiB and never shrinks a slot
    for Mc, N, eb in [(1000, 8192, 4), (513, 4096, 4), (4097, 1000, 2), (3, 2**21, 4)]:
        s = O.staging_slot_elems(Mc, N, eb)
        assert Mc * N <= s and (s - Mc * N) * eb < 512 << 10
        if Mc * N * eb >= 8 << 20:
            assert (s * eb) % (512 << 10) == 0


def test_padded_staging_offsets():
    # M=8000, W=8: Mc=1000, slots 8,257,536 floats apart (1008 rows of
    # 8192); row il of slot (d, r) starts il*8192 after the slot's start
    G = O.Geometry(8000, 8192, 64, 8, 256, 256)
    assert G.slot == 8257536
    assert G.staging_offset(0, 0, 0, 0) == 0
    assert G.staging_offset(0, 1, 0, 0) == 8257536
    assert G.staging_offset(0, 0, 999, 8191) == 999 * 8192 + 8191
    # row 1000 is chunk 1's first row: slot (1, 0) = the 8th slot
    assert G.staging_offset(1, 0, 1000, 5) == 8 * 8257536 + 5
    assert G.staging_offset(7, 7, 7999, 8191) == 63 * 8257536 + 999 * 8192 + 8191
    # every used element has its own offset and the slots never overlap
    last = [G.staging_offset(d, r, d * 1000 + 999, 8191) for d in range(8) for r in range(8)]
    first = [G.staging_offset(d, r, d * 1000, 0) for d in range(8) for r in range(8)]
    assert first == [k * 8257536 for k in range(64)]
    assert all(l < f for l, f in zip(last, first[1:]))
    # bfloat16 staging pads to 1024 rows
    Gb = O.Geometry(8000, 8192, 64, 8, 256, 256, staging_dtype=O.STAGING_BF16)
    assert Gb.staging_offset(1, 2, 1001, 3) == (8 + 2) * 8388608 + 8192 + 3


def test_sub_offsets_are_a_bijection():
    # sub[d][G][Mc][N]: every (destination, group, chunk row, column) has
    # its own element, and together they fill G*M*N elements exactly once
    for (M, N, W, G) in [(8, 3, 4, 2), (12, 5, 4, 4), (16, 2, 8, 2), (6, 4, 2, 1)]:
        geo = O.Geometry(M, N, 64, W, 64, N, order=O.TWO_LEVEL, groups=G)
        seen = np.zeros(G * M * N, dtype=np.int32)
        for i in range(M):
            d = geo.chunk_of_row(i)
            for g in range(G):
                for j in range(N):
                    seen[geo.sub_offset(d, g, i, j)] += 1
        assert np.all(seen == 1), (M, N, W, G)


def test_sub_offset_hand_values():
    # W=4, G=2, M=8 (Mc=2), N=3: block (d, g) starts at (d*2 + g)*Mc*N
    geo = O.Geometry(8, 3, 64, 4, 64, 3, order=O.TWO_LEVEL, groups=2)
    assert geo.sub_offset(0, 0, 0, 0) == 0
    assert geo.sub_offset(0, 1, 0, 0) == 6          # second group of chunk 0
    assert geo.sub_offset(1, 0, 2, 0) == 12         # chunk 1 starts after 2 groups
    assert geo.sub_offset(1, 1, 3, 2) == 23         # ((1*2+1)*2 + 1)*3 + 2
    assert geo.sub_offset(3, 1, 7, 2) == 2 * 8 * 3 - 1


def test_flag_prediction():
    G = O.Geometry(128, 256, 512, 2, 64, 64)
    assert not G.predict_flags([3]).any()
    assert G.predict_flags([1]).all()
    assert G.predict_flags([3 | O.KEEP_FLAGS]).all()
    assert not G.predict_flags([1, 2]).any()
    assert not G.predict_flags([3, 3, 3]).any()


# ---------------------------------------------------------------- validate
TILES = [(256, 256), (64, 64)]


@pytest.mark.parametrize("kw,code", [
    (dict(), O.OK),
    (dict(W=0), O.INVALID_ARG),
    (dict(W=65), O.INVALID_ARG),
    (dict(M=1000, W=3), O.INVALID_ARG),
    (dict(M=0), O.INVALID_ARG),
    (dict(N=0), O.INVALID_ARG),
    (dict(K=-64), O.INVALID_ARG),
    (dict(K=0), O.OK),
    (dict(dtype=7), O.INVALID_ARG),
    (dict(order=2), O.INVALID_ARG),
    (dict(order=O.TWO_LEVEL, groups=3), O.INVALID_ARG),
    (dict(order=O.TWO_LEVEL, groups=0), O.INVALID_ARG),
    (dict(order=O.TWO_LEVEL, groups=2), O.OK),
    (dict(swizzle=4), O.INVALID_ARG),
    (dict(has_c=1, ldc=100), O.INVALID_ARG),
    (dict(has_c=1, ldc=0), O.OK),
    (dict(has_c=1, ldc=1024), O.OK),
    (dict(has_c=1, ldc=1028), O.UNSUPPORTED),
    (dict(materialize_sub=1), O.INVALID_ARG),
    (dict(materialize_sub=1, order=O.TWO_LEVEL, groups=2), O.OK),
    (dict(group_m=-1), O.INVALID_ARG),
    (dict(tile_m=128, tile_n=128), O.UNSUPPORTED),
    (dict(N=1000), O.UNSUPPORTED),
    (dict(K=100), O.UNSUPPORTED),
    (dict(K=2**23 - 64), O.OK),
    (dict(K=2**23), O.UNSUPPORTED),
    (dict(N=2**25 - 256), O.OK),
    (dict(N=2**25), O.UNSUPPORTED),
    (dict(swizzle=O.TILE_INTERLEAVED), O.OK),
    (dict(swizzle=O.TILE_INTERLEAVED, interleave=32), O.OK),
    (dict(interleave=1), O.OK),
    (dict(interleave=2), O.INVALID_ARG),
    (dict(swizzle=O.TILE_INTERLEAVED, interleave=-1), O.INVALID_ARG),
    (dict(staging_dtype=O.STAGING_BF16), O.OK),
    (dict(staging_dtype=2), O.INVALID_ARG),
    (dict(staging_dtype=O.STAGING_BF16, dtype=O.F32, tile_m=64, tile_n=64), O.UNSUPPORTED),
    (dict(staging_dtype=O.STAGING_BF16, materialize_sub=1, order=O.TWO_LEVEL,
          groups=2), O.UNSUPPORTED),
])
def test_validate_table(kw, code):
    base = dict(M=2048, N=1024, K=512, W=8, dtype=O.BF16, tile_m=256,
                tile_n=256)
    base.update(kw)
    assert O.validate(**base, supported_tiles=TILES) == code


# ------------------------------------------------------ bfloat16 staging mode
def test_bf16_staging_hand_example():
    """W=2, K=2, one row per chunk.  Row 0's partials are 256+1 = 257 (rank 0)
    and 256+5 = 261 (rank 1).  Staged in bfloat16 they become 256 and 260
    (both ties, rounded to even), summing to 516 = 0x4401; staged in float
    the sum 518 rounds (tie, to even) to 520 = 0x4402 on output."""
    bf = lambda v: O.bf16_rne(np.array(v, np.float32)).reshape(np.shape(v))
    A = np.stack([bf([[256, 1], [1, 0]]), bf([[256, 5], [2, 0]])])   # [W][M][K]
    B = np.stack([bf([[1], [1]]), bf([[1], [1]])])                  # [W][K][N]
    f32 = O.emulate_rows(A, B, dtype=O.BF16)
    b16 = O.emulate_rows(A, B, dtype=O.BF16, staging_dtype=O.STAGING_BF16)
    assert f32[:, 0].tolist() == [0x4402, int(bf([3.0])[0])]
    assert b16[:, 0].tolist() == [0x4401, int(bf([3.0])[0])]


def test_bf16_staging_equals_f32_staging_when_partials_are_exact():
    """Integer inputs whose every partial lies in [-256, 256] are exact in
    bfloat16, so rounding them on staging changes nothing."""
    rng = np.random.default_rng(7)
    W, M, N, K = 4, 8, 16, 64
    vals = rng.integers(-1, 2, size=(W, M, K)).astype(np.float32)
    wts = rng.integers(-1, 2, size=(W, K, N)).astype(np.float32)
    A, B = O.bf16_rne(vals).reshape(vals.shape), O.bf16_rne(wts).reshape(wts.shape)
    for r in range(W):
        assert np.abs(O.partial_rows(A, B, dtype=O.BF16, r=r)).max() <= 256
    a = O.emulate_rows(A, B, dtype=O.BF16)
    b = O.emulate_rows(A, B, dtype=O.BF16, staging_dtype=O.STAGING_BF16)
    assert np.array_equal(a, b)


def test_bf16_staging_within_rounding_bound():
    """|out - ref| <= 2^-8 |ref| + 2^-8 (1 + 2^-8) sum_r |D_r| (+ float sums):
    each staged partial and the output are rounded to 8 significant bits
    by round-to-nearest-even."""
    x = I.make_inputs(I.with_shape(I.WORKLOADS["llama8b"], M=64, N=128, K=256))
    A, B = x["A"], x["B"]
    W = A.shape[0]
    out = O.bf16_bits_to_f64(O.emulate_rows(A, B, dtype=O.BF16,
                                            staging_dtype=O.STAGING_BF16))
    ref = O.reference_rows(A, B, dtype=O.BF16)
    mag = sum(np.abs(O.partial_rows(A, B, dtype=O.BF16, r=r)) for r in range(W))
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -8 * (1 + 2.0 ** -8) * mag + 1e-6 * mag
    assert np.all(np.abs(out - ref) <= bound)
    # and the second rounding is visible: not every output equals the
    # float-staged one
    f32 = O.bf16_bits_to_f64(O.emulate_rows(A, B, dtype=O.BF16))
    assert np.any(out != f32)


# ------------------------------------------------------ all-gather + GEMM
def test_ag_gather_and_send_order_hand_examples():
    shards = np.arange(2 * 3 * 2).reshape(2, 3, 2)
    assert O.ag_gather(shards).tolist() == [[0, 1], [2, 3], [4, 5], [6, 7], [8, 9], [10, 11]]
    # M=8, W=2, 2-row tiles: chunk 0 = tile-rows {0,1}, chunk 1 = {2,3}
    assert O.ag_send_order(8, 2, 2, 0) == [0, 1, 2, 3]
    assert O.ag_send_order(8, 2, 2, 1) == [2, 3, 0, 1]
    # M=6 (Mc=3): tile-row 1 (rows 2-3) starts in chunk 0, so chunk 0 sends
    # tile-rows {0,1} and chunk 1 only {2}
    assert O.ag_send_order(6, 2, 2, 0) == [0, 1, 2]
    assert O.ag_send_order(6, 2, 2, 1) == [2, 0, 1]


def test_ag_send_order_is_a_permutation_own_chunk_first():
    for (M, N, K, W, bm, bn) in _random_geoms(20):
        G = O.Geometry(M, N, K, W, bm, bn)
        for r in range(W):
            order = O.ag_send_order(M, W, bm, r)
            assert sorted(order) == list(range(G.tiles_m))
            own = G.chunk_tile_rows(r)
            assert order[:len(own)] == own


def test_ag_gemm_rows_exact_integers():
    """Y_r = gather(X) . B_r against an integer matmul done here in int64
    (entries in {-1,0,1} and small integers: exact in bfloat16 and fp64)."""
    rng = np.random.default_rng(3)
    W, Mc, K, N = 4, 5, 64, 24
    Xi = rng.integers(-1, 2, size=(W, Mc, K))
    Bi = rng.integers(-3, 4, size=(W, K, N))
    to_bits = lambda a: O.bf16_rne(a.astype(np.float32)).reshape(a.shape)
    Xfull = np.concatenate(list(Xi), axis=0).astype(np.int64)
    for r in range(W):
        got = O.ag_gemm_rows(to_bits(Xi), to_bits(Bi), r=r)
        want = Xfull @ Bi[r].astype(np.int64)
        assert np.array_equal(got, want.astype(np.float64)), r
    # a row range
    got = O.ag_gemm_rows(to_bits(Xi), to_bits(Bi), r=2, row_lo=7, row_hi=12)
    assert np.array_equal(got, (Xfull @ Bi[2].astype(np.int64))[7:12].astype(np.float64))


@pytest.mark.parametrize("kw,code", [
    (dict(), O.OK),
    (dict(W=0), O.INVALID_ARG),
    (dict(M=1000, W=3), O.INVALID_ARG),
    (dict(pad=1), O.INVALID_ARG),
    (dict(group_m=-1), O.INVALID_ARG),
    (dict(N=1000), O.UNSUPPORTED),
    (dict(K=100), O.UNSUPPORTED),
    (dict(K=2**23), O.UNSUPPORTED),
    (dict(N=2**25), O.UNSUPPORTED),
    (dict(tile_m=128, tile_n=64), O.UNSUPPORTED),
])
def test_validate_ag_table(kw, code):
    base = dict(M=2048, N=1024, K=512, W=8, tile_m=256, tile_n=256)
    base.update(kw)
    assert O.validate_ag(**base, supported_tiles=[(256, 256), (256, 128)]) == code


# ------------------------------------------------------- the parity measures
def test_error_measures_hand_values():
    # got = [1, 2], ref = [1, 3]: difference [0, -1]
    got, ref = np.array([1.0, 2.0]), np.array([1.0, 3.0])
    assert O.rel_frobenius(got, ref) == pytest.approx(1 / np.sqrt(10), rel=1e-15)
    assert O.max_norm_err(got, ref) == pytest.approx(1 / 3, rel=1e-15)
    # 2-D input: all elements count, not a row or column
    g2 = np.array([[1.0, 2.0], [3.0, 4.0]])
    r2 = np.array([[1.0, 2.0], [3.0, 6.0]])
    assert O.rel_frobenius(g2, r2) == pytest.approx(2 / np.sqrt(50), rel=1e-15)
    assert O.max_norm_err(g2, r2) == pytest.approx(2 / 6, rel=1e-15)
    # identical inputs
    assert O.rel_frobenius(r2, r2) == 0.0 and O.max_norm_err(r2, r2) == 0.0


def test_max_norm_err_floor_below_one():
    # |ref| < 1: the error is absolute (divided by 1, not by |ref|)
    assert O.max_norm_err(np.array([0.5]), np.array([0.25])) == pytest.approx(0.25)
    assert O.max_norm_err(np.array([1e-3]), np.array([0.0])) == pytest.approx(1e-3)
    # |ref| > 1: relative
    assert O.max_norm_err(np.array([9.0]), np.array([8.0])) == pytest.approx(1 / 8)
    assert O.max_norm_err(np.array([-9.0]), np.array([-8.0])) == pytest.approx(1 / 8)
    # the maximum over elements, mixing both regimes
    got = np.array([0.5, 9.0, 100.5])
    ref = np.array([0.25, 8.0, 100.0])
    assert O.max_norm_err(got, ref) == pytest.approx(0.25)
    assert O.max_norm_err(np.zeros(0), np.zeros(0)) == 0.0


def test_rel_frobenius_zero_reference():
    # no scale to divide by: the error is the result's own norm
    assert O.rel_frobenius(np.zeros(4), np.zeros(4)) == 0.0
    assert O.rel_frobenius(np.array([3.0, 4.0]), np.zeros(2)) == pytest.approx(5.0)


@pytest.mark.parametrize("fn", [O.rel_frobenius, O.max_norm_err])
def test_error_measures_reject_shape_mismatch(fn):
    # broadcasting a [N] reference against an [M, N] result would compare
    # less than the whole output: a mismatch must raise
    with pytest.raises(ValueError):
        fn(np.zeros((4, 3)), np.zeros(3))
    with pytest.raises(ValueError):
        fn(np.zeros((3, 4)), np.zeros((4, 3)))
    with pytest.raises(ValueError):
        fn(np.zeros(5), np.zeros(4))


def test_bf16_output_floor_hand_case():
    # 1 + 2^-9 is a quarter ulp above 1.0 in bfloat16 (ulp 2^-7): it rounds
    # to 1.0, an error of 2^-9; 3.0 is exact
    ref = np.array([1.0 + 2.0**-9, 3.0])
    got = O.bf16_bits_to_f64(O.bf16_rne(ref.astype(np.float32)))
    assert got.tolist() == [1.0, 3.0]
    want = 2.0**-9 / np.sqrt((1 + 2.0**-9) ** 2 + 9.0)
    assert O.rel_frobenius(got, ref) == pytest.approx(want, rel=1e-12)
    assert O.max_norm_err(got, ref) == pytest.approx(2.0**-9 / (1 + 2.0**-9), rel=1e-12)


def test_bf16_output_floor_on_gaussian_outputs():
    """The accuracy floor of any bfloat16 output: rel_F(bf16_RNE(ref), ref)
    on N(0, 8) data (W = 8 partials of unit variance).  Rounding to nearest
    with 8 significant bits errs by at most 2^-8 of |x| (a strict bound),
    and with the error spread evenly over +-half an ulp of the binade
    [2^e, 2^(e+1)) its mean square is 2^(2e-16)/3, so rel_F lies between
    2^-8/(2*sqrt(3)) (all mantissas near 2) and 2^-8/sqrt(3) (all near 1).
    Truncation instead of rounding would double it; a dropped square root
    would put it near 3e-6.  The floor sits below the 2e-3 bar, which is
    why the staged partials are kept in float32."""
    rng = np.random.default_rng(8)
    ref = (rng.standard_normal(1 << 20) * np.sqrt(8.0)).astype(np.float32).astype(np.float64)
    got = O.bf16_bits_to_f64(O.bf16_rne(ref.astype(np.float32)))
    floor = O.rel_frobenius(got, ref)
    assert floor <= 2.0**-8
    assert 2.0**-8 / (2 * np.sqrt(3)) <= floor <= 2.0**-8 / np.sqrt(3)
    assert floor < 2e-3
    assert O.max_norm_err(got, ref) <= 2.0**-8
