"""The all-gather's fused mode needs the copy kernel to run beside gated
GEMM workgroups that occupy every CU while they wait for its signals.  A
copy wave therefore has to fit in the registers each GEMM tile
configuration leaves free on a SIMD at that configuration's maximum
occupancy.  This reads the compiler's resource report for both device
sources (built with the library's flags) and checks the budget for every
GEMM instantiation (CPU only: hipcc cross-compiles for gfx950)."""
import os
import re
import shutil
import subprocess

import pytest

from tensor_gemm_reduce_lds_amd import build as B

VGPRS_PER_SIMD_LANE = 512      # unified VGPR + AGPR file per SIMD lane (gfx950)
LDS_PER_CU = 160 * 1024
SIMDS_PER_CU = 4
GRANULE = 8


def _report(src):
    cmd = [B.HIPCC] + B.CFLAGS + ["--cuda-device-only", "-c", "-o", os.devnull,
                                  "-Rpass-analysis=kernel-resource-usage", src]
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, p.stderr[-2000:]
    kernels, cur = {}, None
    for line in p.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|LDS Size \[bytes/block\]|Occupancy \[waves/SIMD\]|"
                      r"ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).split(" ")[0]] = int(m.group(2))
    return kernels


def _params(name):
    """Template arguments of a gemm_bf16_kernel instantiation: BM, BN, BK,
    STAGES, WGM, WGN, FW (0: plain epilogue, W: owner-fused reduce) and U2
    (1: the K loop unrolled by two steps)."""
    return tuple(map(int, re.search(
        r"ILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELb(\d)EE", name).groups()))


def _gemms():
    return {k: v for k, v in _report(os.path.join(B.CSRC, "gemm_bf16.hip")).items()
            if "gemm_bf16_kernel" in k}


def _plain_gemms():
    # the instantiations the all-gather and the overlapped slices run beside
    # (the rolled K loop; the unrolled one is only launched alone)
    return {k: v for k, v in _gemms().items() if _params(k)[6] == 0 and _params(k)[7] == 0}


def _alloc(vgprs, agprs):
    # AGPRs start at the next multiple of 4 after the VGPRs; the total is
    # allocated in granules
    total = (-(-vgprs // 4) * 4 + agprs) if agprs else vgprs
    return -(-total // GRANULE) * GRANULE


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC),
                    reason="hipcc not available")
def test_copy_wave_fits_beside_every_gemm_configuration():
    copy = [v for k, v in _report(os.path.join(B.CSRC, "gemm_ag.hip")).items()
            if "ag_copy_kernel" in k]
    assert len(copy) == 1
    copy_alloc = _alloc(copy[0]["VGPRs"], copy[0].get("AGPRs", 0))
    assert copy[0].get("LDS", 0) == 0
    gemms = _plain_gemms()
    assert len(gemms) == 4
    for name, r in gemms.items():
        bm, bn, bk, stages, wgm, wgn, _, _ = _params(name)
        lds = stages * (bm + bn) * bk * 2 + r.get("LDS", 0)
        wgs_per_cu = LDS_PER_CU // lds
        waves_by_lds = -(-wgs_per_cu * wgm * wgn // SIMDS_PER_CU)
        waves = min(r["Occupancy"], waves_by_lds)
        gemm_alloc = _alloc(r["VGPRs"], r.get("AGPRs", 0))
        free = VGPRS_PER_SIMD_LANE - waves * gemm_alloc
        assert copy_alloc <= free, (bm, bn, waves, gemm_alloc, copy_alloc)


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC),
                    reason="hipcc not available")
def test_overlap_reduce_slices_fit_beside_every_gemm_configuration():
    """The overlapped reduce launches its slices (the one-row instantiations)
    while GEMM workgroups hold the CUs; a slice wave that does not fit
    beside them waits for them to retire and the overlap is lost (a
    throughput property: the slices never wait on anything a GEMM
    workgroup waits for)."""
    red = {k: v for k, v in _report(os.path.join(B.CSRC, "reduce.hip")).items()
           # template <W, L, bf16 out, bf16 staging, ROWS2, BUF>: ROWS2 = BUF = false
           if "reduce_kernel" in k and k.endswith("Lb0ELb0EEEvNS_10ReduceArgsE")}
    assert red, "one-row reduce instantiations not found"
    need = max(_alloc(v["VGPRs"], v.get("AGPRs", 0)) for v in red.values())
    gemms = _plain_gemms()
    for name, r in gemms.items():
        bm, bn, bk, stages, wgm, wgn, _, _ = _params(name)
        lds = stages * (bm + bn) * bk * 2 + r.get("LDS", 0)
        waves = min(r["Occupancy"], -(-(LDS_PER_CU // lds) * wgm * wgn // SIMDS_PER_CU))
        free = VGPRS_PER_SIMD_LANE - waves * _alloc(r["VGPRs"], r.get("AGPRs", 0))
        assert need <= free, (bm, bn, need, free)


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC),
                    reason="hipcc not available")
def test_fused_reduce_variant_keeps_the_plain_occupancy():
    """The owner-fused reduce epilogue holds a row's remote partials in
    registers: it must not spill or drop below the plain kernel's two
    workgroup waves per SIMD."""
    gemms = _gemms()
    fused = {k: v for k, v in gemms.items() if _params(k)[6] > 0}
    assert fused, "no owner-fused instantiation"
    for name, r in fused.items():
        plain = [v for k, v in gemms.items() if _params(k)[:6] == _params(name)[:6]
                 and _params(k)[6:] == (0, 0)]
        assert len(plain) == 1
        assert r.get("ScratchSize", 0) == 0, name
        assert r["Occupancy"] >= plain[0]["Occupancy"], (name, r, plain[0])


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC),
                    reason="hipcc not available")
def test_unrolled_loop_keeps_the_plain_occupancy():
    """The K loop unrolled by two steps (stage offsets in the DS reads'
    immediate fields) exists for the 256 x 256 plain kernel only and keeps
    its two workgroup waves per SIMD."""
    gemms = _gemms()
    unrolled = {k: v for k, v in gemms.items() if _params(k)[7] == 1}
    assert [_params(k)[:7] for k in unrolled] == [(256, 256, 64, 2, 2, 4, 0)]
    for name, r in unrolled.items():
        plain = [v for k, v in gemms.items() if _params(k)[:6] == _params(name)[:6]
                 and _params(k)[6:] == (0, 0)]
        assert len(plain) == 1
        assert r["Occupancy"] >= plain[0]["Occupancy"], (name, r, plain[0])
