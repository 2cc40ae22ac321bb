"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, and rejects bad descriptors before any HIP call with
the same status the oracle's rules give."""
import ctypes
import os
import subprocess

import pytest

import oracle as O
from tensor_gemm_reduce_lds_amd import gemm_rs as G

BF16_TILES = [(256, 256), (256, 128), (128, 128), (64, 128)]
F32_TILES = [(64, 64)]


def test_library_exports_every_header_function():
    names = G.header_functions()
    assert names == sorted(["gemm_rs_plan", "gemm_rs_run", "gemm_rs_run_noalloc",
                            "gemm_rs_destroy",
                            "gemm_rs_query", "gemm_rs_tile_order",
                            "gemm_rs_status", "gemm_rs_strerror",
                            "gemm_ag_plan", "gemm_ag_run", "gemm_ag_query",
                            "gemm_ag_status", "gemm_ag_destroy"])
    lib = G.load_library()
    for n in names:
        assert hasattr(lib, n), n


STRUCTS = [("d", "gemm_rs_desc_t", G.gemm_rs_desc_t), ("i", "gemm_rs_info_t", G.gemm_rs_info_t),
           ("ad", "gemm_ag_desc_t", G.gemm_ag_desc_t), ("ai", "gemm_ag_info_t", G.gemm_ag_info_t)]


def _c_layout(tmp_path):
    """sizeof/offsetof of the public structs as gcc lays them out."""
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "gemm_rs.h"',
           '#include "gemm_ag.h"', "int main(void) {"]
    for key, cname, cls in STRUCTS:
        src.append('  printf("%s %%zu\\n", sizeof(%s));' % (key, cname))
        for f, _ in cls._fields_:
            src.append('  printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (key, f, cname, f))
    src.append("  return 0; }")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(G.HEADER), str(c), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    return dict(line.split() for line in out.splitlines())


def test_struct_layout_matches_c_compiler(tmp_path):
    lay = _c_layout(tmp_path)
    for key, cname, cls in STRUCTS:
        assert int(lay[key]) == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(lay[key + "." + f]) == getattr(cls, f).offset, (cname, f)


def test_strerror_and_null_handles():
    assert G.gemm_rs_strerror(0) == "ok"
    assert "timed out" in G.gemm_rs_strerror(G.ERR_TIMEOUT)
    assert G.gemm_rs_strerror(12345) == "unknown status"
    rc, h = G.gemm_rs_plan(None)
    assert rc == G.ERR_INVALID_ARG and h is None
    assert G.gemm_rs_run(None, None, None, None, 1.0, 0.0, None) == G.ERR_INVALID_ARG
    assert G.gemm_rs_destroy(None) == G.OK
    assert G.gemm_rs_query(None)[0] == G.ERR_INVALID_ARG
    assert G.gemm_rs_status(None)[0] == G.ERR_INVALID_ARG


BAD = [
    dict(W=0), dict(W=65), dict(M=1000, W=3), dict(M=0), dict(K=-64), dict(N=0), dict(dtype=7),
    dict(order=2), dict(order=1, groups=3), dict(order=1, groups=0), dict(swizzle=4),
    dict(swizzle=-1),
    dict(has_c=1, ldc=100), dict(has_c=2), dict(ldc=-8), dict(materialize_sub=1),
    dict(materialize_sub=2, order=1, groups=2), dict(group_m=-1), dict(tile_m=-64),
    dict(tile_m=128, tile_n=64), dict(tile_m=32, tile_n=32), dict(N=1000),
    dict(K=100), dict(has_c=1, ldc=1028), dict(dtype=1, tile_m=128, tile_n=128),
    dict(M=2**31, W=1), dict(K=2**31 + 64),
    dict(staging_dtype=2), dict(staging_dtype=1, dtype=1, tile_m=64, tile_n=64),
    dict(staging_dtype=1, materialize_sub=1, order=1, groups=2),
    dict(interleave=-1, swizzle=3), dict(interleave=2),
    dict(K=2**23), dict(N=2**25), dict(N=2**25 + 256),
]


@pytest.mark.parametrize("kw", BAD)
def test_bad_descriptors_rejected_like_oracle(kw):
    base = dict(M=2048, N=1024, K=512, W=8, dtype=0, tile_m=256, tile_n=256)
    base.update(kw)
    tiles = F32_TILES if base["dtype"] == 1 else BF16_TILES
    want = O.validate(**base, supported_tiles=tiles)
    assert want != O.OK
    rc, h = G.gemm_rs_plan(G.make_desc(**base))
    assert rc == want and h is None


def test_ag_null_handles_and_flags():
    rc, h = G.gemm_ag_plan(None)
    assert rc == G.ERR_INVALID_ARG and h is None
    assert G.gemm_ag_run(None, None, None, None) == G.ERR_INVALID_ARG
    assert G.gemm_ag_query(None)[0] == G.ERR_INVALID_ARG
    assert G.gemm_ag_status(None)[0] == G.ERR_INVALID_ARG
    assert G.gemm_ag_destroy(None) == G.OK


AG_BAD = [dict(W=0), dict(W=65), dict(M=1000, W=3), dict(M=0), dict(K=0), dict(pad=1),
          dict(group_m=-1), dict(tile_m=-64), dict(tile_m=128, tile_n=64), dict(N=1000),
          dict(K=100), dict(M=2**31, W=1), dict(K=2**23), dict(N=2**25),
          # 2^23 tile-rows x 64 ranks x 16 copy pieces overflows 32 bits
          dict(M=2**29, N=128, K=64, W=64, tile_m=64, tile_n=128)]


@pytest.mark.parametrize("kw", AG_BAD)
def test_bad_ag_descriptors_rejected_like_oracle(kw):
    base = dict(M=2048, N=1024, K=512, W=8, tile_m=256, tile_n=256)
    base.update(kw)
    want = O.validate_ag(**base, supported_tiles=BF16_TILES)
    assert want != O.OK
    rc, h = G.gemm_ag_plan(G.make_ag_desc(**base))
    assert rc == want and h is None


def test_noalloc_rejects_before_any_hip_call():
    """gemm_rs_run_noalloc checks its descriptor, flags and workspace size
    on the host before it touches a device."""
    assert G.gemm_rs_run_noalloc(None, None, None, None, 1.0, 0.0, None) == G.ERR_INVALID_ARG
    base = dict(M=64, N=1024, K=512, W=8, dtype=0, tile_m=64, tile_n=128)
    for kw in BAD[:10]:
        d = dict(base, **kw)
        tiles = F32_TILES if d["dtype"] == 1 else BF16_TILES
        want = O.validate(**d, supported_tiles=tiles)
        assert G.gemm_rs_run_noalloc(G.make_desc(**d), None, None, None, 1.0, 0.0,
                                     None) == want, kw
    # the 70B-like shard's 2 GiB of staging does not fit in 64 MiB
    big = G.make_desc(M=8192, N=8192, K=3584, W=8)
    assert G.gemm_rs_run_noalloc(big, None, None, None, 1.0, 0.0, None) == G.ERR_SCRATCH
    # 64 MiB holds W*M*N*4 = 8*256*8192*4 = 64 MiB only without the flag words
    edge = G.make_desc(M=256, N=8192, K=64, W=8)
    assert G.gemm_rs_run_noalloc(edge, None, None, None, 1.0, 0.0, None) == G.ERR_SCRATCH
    sub = G.make_desc(M=64, N=1024, K=64, W=8, order=1, groups=2, materialize_sub=1)
    assert G.gemm_rs_run_noalloc(sub, None, None, None, 1.0, 0.0, None) == G.ERR_UNSUPPORTED
    d = G.make_desc(**base)
    for flags in (G.RUN_GEMM, G.RUN_REDUCE, G.RUN_ALL | G.KEEP_FLAGS, G.RUN_ALL | G.TRACE_TILES,
                  G.RUN_ALL | 64):
        assert G.gemm_rs_run_noalloc(d, None, None, None, 1.0, 0.0, None, None,
                                     flags) == G.ERR_INVALID_ARG, flags
    assert G.gemm_rs_strerror(G.ERR_SCRATCH).startswith("workspace larger than")
