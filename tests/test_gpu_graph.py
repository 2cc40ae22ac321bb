"""A pass captured in a HIP graph: gemm_rs_run (the serial order, the
owner-fused reduce and the two-level order) and gemm_rs_run_noalloc are
captured once on a side stream and the graph is replayed several times, with
eager work and synchronisations between the replays.  Every replay gives the
eager pass's output bit for bit and leaves the flags idle: the run path
enqueues kernels only (no memset, no host synchronisation, no allocation)."""
import numpy as np
import pytest
import torch

from tensor_gemm_reduce_lds_amd import gemm_rs as G
from tensor_gemm_reduce_lds_amd import inputs as I

from gpu_util import desc_fields, flags, new_out, out_bits, run_checked, say, to_device

pytestmark = pytest.mark.gpu

W70 = I.WORKLOADS
CASES = [
    ("serial", I.with_shape(W70["llama70b"], M=2048, N=1024, K=512), G.RUN_ALL),
    ("owner_fused", I.with_shape(W70["llama70b"], M=2048, N=1024, K=512),
     G.RUN_ALL | G.OVERLAP_REDUCE),
    ("two_level_ragged", I.with_shape(W70["ragged_2lvl"], M=4000, N=512, K=256), G.RUN_ALL),
]
REPLAYS = 3


def _poison(out):
    # an eager fill kernel between replays: a replay that skipped a tile
    # would leave this pattern in the output
    out.fill_(-1)


@pytest.mark.parametrize("name,w,run_flags", CASES, ids=[c[0] for c in CASES])
def test_plan_pass_replays_match_eager(name, w, run_flags):
    x = I.make_inputs(w)
    dev = to_device(x, w)
    say("graph capture", name)
    with G.Plan(**desc_fields(w)) as plan:
        ref = new_out(w)
        run_checked(plan, dev, w, ref, run_flags)     # eager pass first
        want = out_bits(ref)
        side = torch.cuda.Stream()
        out = new_out(w)
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            plan.run(dev["A"], dev["B"], dev["C"], w.alpha, w.beta, out, side, run_flags)
        for k in range(REPLAYS):
            _poison(out)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            rc, detail = plan.status(torch.cuda.current_stream())
            assert rc == G.OK, (k, rc, detail)
            assert np.array_equal(out_bits(out), want), k
            assert not flags(plan).any(), k
            # eager work on the plan between replays
            run_checked(plan, dev, w, ref, G.RUN_ALL)
        del graph


def test_noalloc_pass_replays_match_eager():
    w = I.with_shape(W70["llama70b"], M=1024, N=1024, K=256)
    x = I.make_inputs(w)
    dev = to_device(x, w)
    say("graph capture noalloc")
    desc = G.make_desc(**desc_fields(w))
    status = torch.full((4,), -7, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.current_stream()
    ref = new_out(w)
    rc = G.gemm_rs_run_noalloc(desc, dev["A"], dev["B"], dev["C"], w.alpha, w.beta, ref, s,
                               G.RUN_ALL, status)
    assert rc == G.OK, G.gemm_rs_strerror(rc)
    s.synchronize()
    assert status.cpu().tolist() == [0, 0, 0, 0]
    want = out_bits(ref)
    side = torch.cuda.Stream()
    out = new_out(w)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        rc = G.gemm_rs_run_noalloc(desc, dev["A"], dev["B"], dev["C"], w.alpha, w.beta, out,
                                   side, G.RUN_ALL, status)
    assert rc == G.OK, G.gemm_rs_strerror(rc)
    for k in range(REPLAYS):
        _poison(out)
        status.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert status.cpu().tolist() == [0, 0, 0, 0], k
        assert np.array_equal(out_bits(out), want), k
        # an eager no-allocation call of another size between replays
        w2 = I.with_shape(w, M=512, N=512, K=128)
        x2 = I.make_inputs(w2)
        dev2 = to_device(x2, w2)
        o2 = new_out(w2)
        rc = G.gemm_rs_run_noalloc(G.make_desc(**desc_fields(w2)), dev2["A"], dev2["B"],
                                   dev2["C"], w2.alpha, w2.beta, o2, s, G.RUN_ALL, None)
        assert rc == G.OK, G.gemm_rs_strerror(rc)
        s.synchronize()
    del graph
