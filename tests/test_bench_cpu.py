"""CPU checks of bench.py's bookkeeping: algorithmic byte counts and the
roofline each workload is priced against (no GPU needed)."""
import bench
from tensor_gemm_reduce_lds_amd import inputs as I


def test_algorithmic_bytes_70b_like():
    # A + B (bf16) + fp32 staging + one bias row; reduce: staging + bf16 out
    w = I.WORKLOADS["llama70b"]
    gemm, red = bench.algorithmic_bytes(w, 2)
    assert gemm == 8 * 8192 * 3584 * 2 * 2 + 8 * 8192 * 8192 * 4 + 8192 * 2 == 3087024128
    assert red == 8 * 8192 * 8192 * 4 + 8192 * 8192 * 2 == 2281701376
    assert w.flops == 3848290697216


def test_algorithmic_bytes_other_workloads():
    w = I.WORKLOADS["llama8b"]
    assert bench.algorithmic_bytes(w, 2) == (771751936, 570425344)
    w = I.WORKLOADS["decode"]
    assert bench.algorithmic_bytes(w, 2) == (490209280, 17825792)
    w = I.WORKLOADS["ragged_2lvl"]
    assert bench.algorithmic_bytes(w, 2) == (3025666048, 2228224000)
    w = I.WORKLOADS["tiny_f32"]
    assert bench.algorithmic_bytes(w, 4) == (1835008, 393216)


def test_roofline_bound_follows_intensity():
    peak = bench.PEAK_BF16_TFLOPS
    w = I.WORKLOADS["llama70b"]
    g, _ = bench.algorithmic_bytes(w, 2)
    r = bench.gemm_roofline(w.flops, g, 3.2, peak, None)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert abs(r["achieved"] - w.flops / 3.2e-3 / 1e12) < 0.01
    assert abs(r["frac"] - r["achieved"] / peak) < 1e-4
    w = I.WORKLOADS["decode"]
    g, _ = bench.algorithmic_bytes(w, 2)
    r = bench.gemm_roofline(w.flops, g, 0.1, peak, None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - g / 0.1e-3 / 1e9) < 0.1


def test_stored_traffic_matches_kernel_digest():
    # the committed counter summary is used only for the kernel it was taken on
    t = bench.stored_traffic()
    with open(bench.TRAFFIC_FILE) as f:
        text = f.read()
    if "kernel_source_digest: %s" % bench.kernel_source_digest() in text:
        assert t is not None and t > 3.0e9
    else:
        assert t is None
