"""The benchmark's measurement library (libfar_ceiling.so, include/far_ceiling.h) without
a GPU: it loads, exports what the header declares, and rejects bad arguments before
launching anything (every call here fails validation)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "far_ceiling.h")
LIB = os.path.join(ROOT, "residual_add_rmsnorm_fp32_amd", "libfar_ceiling.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: build with __graft_entry__.build()")
    import bench
    return bench.Ceiling().lib


def test_exports_every_declared_function(lib):
    names = set(re.findall(r"^int (far_ceiling_\w+)\(", open(HEADER).read(), re.M))
    assert names == {"far_ceiling_rows", "far_ceiling_flat", "far_ceiling_empty", "far_ceiling_sleep",
                     "far_ceiling_stamp"}
    for n in names:
        assert hasattr(lib, n)


def _ptrs(n):
    return (ctypes.c_void_p * n)(*[0x7F0000000000 + i * (1 << 20) for i in range(n)])


def test_rows_argument_checks(lib):
    ok = dict(inputs=_ptrs(3), n=3, out_full=0x7E0000000000, out2=None, half=1, out_row=None,
              rows=16, row_bytes=4096, w=4, n_packs=1, rpb=1, grid=16)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.far_ceiling_rows(a["inputs"], a["n"], a["out_full"], a["out2"], a["half"], a["out_row"],
                                    a["rows"], a["row_bytes"], a["w"], a["n_packs"], a["rpb"], a["grid"], None)
    assert call(n=0) == 1
    assert call(n=10, inputs=_ptrs(10)) == 1
    assert call(out_full=None) == 1
    assert call(rows=0) == 1
    assert call(row_bytes=4100) == 1                 # not whole 16-byte packs
    assert call(w=1) == 1                            # 64 lanes x 1 pack < 256 packs
    assert call(w=16, rpb=2) == 1                    # 2048 lanes
    assert call(n_packs=6) == 1
    assert call(n=9, inputs=_ptrs(9), n_packs=3) == 1  # 27 loads per lane
    assert call(grid=0) == 1
    assert call(grid=(1 << 20) + 1) == 1


def test_flat_empty_sleep_argument_checks(lib):
    p = _ptrs(2)
    assert lib.far_ceiling_flat(p, 2, 0x7E0000000000, None, 0, 15, 1, 256, 8, None) == 1       # not packs
    assert lib.far_ceiling_flat(p, 2, 0x7E0000000000, None, 0, 1 << 32, 1, 256, 8, None) == 1  # >= 4 GiB
    assert lib.far_ceiling_flat(p, 2, 0x7E0000000000, None, 0, 4096, 1, 100, 8, None) == 1     # block
    assert lib.far_ceiling_flat(p, 2, 0x7E0000000000, None, 0, 4096, 13, 256, 8, None) == 1    # unroll
    assert lib.far_ceiling_empty(0, 64, None) == 1
    assert lib.far_ceiling_empty(4, 65, None) == 1
    assert lib.far_ceiling_sleep(-1, None) == 1
    assert lib.far_ceiling_sleep(100001, None) == 1
    assert lib.far_ceiling_stamp(None, 0, None) == 1
    assert lib.far_ceiling_stamp(0x7E0000000000, -1, None) == 1
