"""The no-allocation entry point (gemm_rs_run_noalloc) on the GPU, through
the C ABI: its output against gemm_rs_run's on the same inputs (bit for
bit: the same kernels on the same data) and against the oracle's bar, on
calls in a row that reuse the one static scratch array with a smaller
problem each time."""
import numpy as np
import pytest
import torch

import oracle as O
from tensor_gemm_reduce_lds_amd import gemm_rs as G
from tensor_gemm_reduce_lds_amd import inputs as I

from gpu_util import (check_tolerance, desc_fields, new_out, oracle_kw, out_bits, out_to_f64,
                      run_checked, say, to_device)

pytestmark = pytest.mark.gpu

W70 = I.WORKLOADS


def _plan_bits(w, dev, over):
    with G.Plan(**desc_fields(w, **over)) as plan:
        out = new_out(w)
        run_checked(plan, dev, w, out)
        return out_bits(out)


def _noalloc(w, dev, over, run_flags=G.RUN_ALL):
    s = torch.cuda.current_stream()
    out = new_out(w)
    status = torch.full((4,), -7, dtype=torch.int32, device="cuda:0")
    rc = G.gemm_rs_run_noalloc(G.make_desc(**desc_fields(w, **over)), dev["A"], dev["B"],
                               dev["C"], w.alpha, w.beta, out, s, run_flags, status)
    assert rc == G.OK, G.gemm_rs_strerror(rc)
    s.synchronize()
    assert status.cpu().tolist() == [0, 0, 0, 0]     # cleared, no asynchronous error
    return out


CASES = [
    # the m <= 64 decode shard at full size (16 MiB of staging), then a
    # smaller problem with a bias row, then a smaller one still with the
    # owner-fused reduce and a two-level order
    ("decode", W70["decode"], {}, G.RUN_ALL),
    ("bias_small", I.with_shape(W70["llama70b"], M=512, N=1024, K=256), {}, G.RUN_ALL),
    ("fused_2lvl", I.with_shape(W70["ragged_2lvl"], M=2048, N=256, K=128), {},
     G.RUN_ALL | G.OVERLAP_REDUCE),
    ("bf16_staging", I.with_shape(W70["llama8b"], M=256, N=512, K=128),
     dict(staging_dtype=G.STAGING_BF16), G.RUN_ALL),
    # the one-launch last-arriver pass (write-through staging stores into
    # the array, release and count per producer, the last one sums)
    ("last_arriver", I.with_shape(W70["llama70b"], M=1024, N=512, K=128),
     dict(tile_m=256, tile_n=256), G.RUN_ALL | G.LAST_ARRIVER),
]


def test_noalloc_matches_run_on_calls_in_a_row():
    rng = np.random.default_rng(3)
    for name, w, over, flags in CASES:
        x = I.make_inputs(w)
        dev = to_device(x, w)
        say("noalloc", name, w.W, w.M, w.N, w.K, over, flags)
        want = _plan_bits(w, dev, over)
        got = _noalloc(w, dev, over, flags)
        assert np.array_equal(out_bits(got), want), name
        kw = oracle_kw(w)
        rows = sorted(set([0, w.M - 1] + [int(v) for v in rng.integers(0, w.M, size=6)]))
        ref = np.concatenate([O.reference_rows(x["A"], x["B"], x["C"], row_lo=i, row_hi=i + 1,
                                               **kw) for i in rows])
        if over.get("staging_dtype") == G.STAGING_BF16:
            continue       # its own bar; the bits equal gemm_rs_run's above
        check_tolerance(out_to_f64(got, w)[rows], ref, w.dtype)


def test_noalloc_rejects_what_does_not_fit_or_apply():
    s = torch.cuda.current_stream()
    big = W70["llama70b"]
    rc = G.gemm_rs_run_noalloc(G.make_desc(**desc_fields(big)), None, None, None, 1.0, 0.0,
                               None, s)
    assert rc == G.ERR_SCRATCH
    small = I.with_shape(W70["llama8b"], M=256, N=512, K=128)
    x = I.make_inputs(small)
    dev = to_device(x, small)
    out = new_out(small)
    for flags in (G.RUN_GEMM, G.RUN_REDUCE, G.RUN_ALL | G.KEEP_FLAGS,
                  G.RUN_ALL | G.TRACE_TILES):
        rc = G.gemm_rs_run_noalloc(G.make_desc(**desc_fields(small)), dev["A"], dev["B"], None,
                                   1.0, 0.0, out, s, flags)
        assert rc == G.ERR_INVALID_ARG, flags
    # after the rejected calls the array still serves a correct pass
    got = _noalloc(small, dev, {})
    assert np.array_equal(out_bits(got), _plan_bits(small, dev, {}))
