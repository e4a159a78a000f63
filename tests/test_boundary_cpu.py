"""The C ABI without a GPU: the library loads, exports what include/far.h declares,
and rejects every bad argument before touching the device. No kernel is launched:
each call here either fails validation or has T == 0.
"""

import ctypes
import os
import re

import pytest

from residual_add_rmsnorm_fp32_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "far.h")

OK, NULLP, SHAPE, DTYPE, NPART, QARGS, ALIAS, HIP, PLAN, WS, SCRATCH = range(11)


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def test_exports_every_declared_function(lib):
    text = open(HEADER).read()
    names = set(re.findall(r"^\s*(?:far_status_t|const char \*|int|int64_t)\s*\n?\s*(far_\w+)\s*\(", text, re.M))
    names |= set(re.findall(r"\b(far_\w+)\(\s*\n", text))
    declared = {n for n in names if n not in ("far_plan_t",)}
    assert {"far_fused_add_rmsnorm", "far_fused_add_rmsnorm_ex", "far_plan", "far_workspace_bytes",
            "far_status_string", "far_version", "far_fused_add_rmsnorm_noalloc"} <= declared
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in far.h but not exported"


def test_status_strings(lib):
    assert len(B.STATUS_NAMES) == 11
    for code, name in B.STATUS_NAMES.items():
        assert B.far_status_string(code).startswith(name)
    assert "UNKNOWN" in B.far_status_string(99)
    assert B.far_version() == 10000


def test_plan_struct_matches_header():
    # far_plan_t: six int32 then one int64
    assert ctypes.sizeof(B.far_plan_t) == 32


def test_constants_match_header():
    text = open(HEADER).read()
    for name in ("FAR_MAX_PARTIALS", "FAR_MAX_WAVES_PER_ROW", "FAR_MAX_PACKS_PER_LANE"):
        m = re.search(r"#define\s+%s\s+(\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(B, name), name


# ------------------------------------------------------------------ planning

SHAPES = [(1, 8), (1, 4096), (16, 2048), (80, 4096), (64, 8192), (2048, 5120),
          (16384, 3584), (3, 12), (4097, 8200), (7, 32768), (2, 40960), (2, 40968),
          (100000, 64), (5, 4), (2048, 5124), (80, 4100), (1, 1), (9, 40959), (2, 40961)]


@pytest.mark.parametrize("T,H", SHAPES)
@pytest.mark.parametrize("P", [1, 2, 8])
def test_auto_plan_is_consistent(T, H, P):
    p = B.far_plan(T, H, P, 0, 0)
    packs = -(-H // 8)  # the last one partial when H % 8 != 0
    if packs > B.FAR_MAX_WAVES_PER_ROW * 64 * B.FAR_MAX_PACKS_PER_LANE:
        assert p["variant"] == "generic"
        # one workgroup per row, about four elements per lane, 64..1024 lanes
        lanes = min(1024, -(-(-(-H // 4)) // 64) * 64)
        assert p["grid_blocks"] == min(T, MAX_GRID) and p["block_threads"] == lanes
        assert p["waves_per_row"] * 64 == lanes
        return
    assert p["variant"] == "vector"
    w, n, r = p["waves_per_row"], p["packs_per_lane"], p["rows_per_block"]
    assert 1 <= w <= B.FAR_MAX_WAVES_PER_ROW and 1 <= n <= B.FAR_MAX_PACKS_PER_LANE and r >= 1
    assert w * 64 * n >= packs, "row does not fit the team"
    assert (w - 1) * 64 * n < packs, "team has a wave with no pack"
    assert p["block_threads"] == r * w * 64 <= 1024
    # one workgroup per group of r rows, or half as many looping over two groups each
    groups = -(-T // r)
    assert p["grid_blocks"] in (min(groups, MAX_GRID), min(-(-groups // 2), MAX_GRID))


MAX_GRID = 1 << 20  # workgroups per launch, at most (the kernels loop over rows beyond)


@pytest.mark.parametrize("T,H", [(1 << 27, 8), (1 << 27, 4), ((1 << 31) - 1, 8), ((1 << 31) - 1, 2)])
def test_plan_for_huge_batches_of_short_rows_fits_one_dispatch(T, H):
    """A dispatch holds fewer than 2^32 lanes: with 2^27 rows of one (whole or partial)
    pack a team per row would exceed that, so the grid is capped and the kernels loop
    over rows."""
    p = B.far_plan(T, H, 2, 0, 0)
    assert 1 <= p["grid_blocks"] <= MAX_GRID
    assert p["grid_blocks"] * p["block_threads"] < 1 << 32


def test_plan_regimes():
    # decode (few rows): each row spread over several waves, one row per workgroup
    for T in (1, 16, 80):
        p = B.far_plan(T, 4096, 8, 0, 0)
        assert p["waves_per_row"] >= 4 and p["rows_per_block"] == 1, p
    assert B.far_plan(64, 8192, 4, 0, 1)["waves_per_row"] <= 8
    # prefill (many rows): one row per workgroup at two packs per lane
    p8 = B.far_plan(16384, 3584, 8, 1, 0)
    assert (p8["waves_per_row"], p8["packs_per_lane"], p8["rows_per_block"], p8["grid_blocks"]) == (4, 2, 1, 16384)
    # a grid of one row per workgroup would need 1.25 rounds of the chip's resident waves:
    # half as many workgroups, each looping over two rows
    p2 = B.far_plan(2048, 5120, 2, 0, 2)
    assert (p2["waves_per_row"], p2["packs_per_lane"], p2["rows_per_block"], p2["grid_blocks"]) == (5, 2, 1, 1024)
    # 1.5 rounds (6-wave teams for 641 packs) still loops; 2.5 rounds does not
    assert B.far_plan(2048, 5124, 2, 0, 2)["grid_blocks"] == 1024
    assert B.far_plan(4096, 5120, 2, 0, 2)["grid_blocks"] == 4096
    assert B.far_plan(2048, 8192, 2, 0, 0)["grid_blocks"] == 2048
    # many partials: an even team of three-pack lanes rather than an odd one of two
    p8o = B.far_plan(2048, 5120, 8, 0, 2)
    assert (p8o["waves_per_row"], p8o["packs_per_lane"]) == (4, 3)
    # rows of at most 64 packs: eight rows per workgroup
    ps = B.far_plan(16384, 512, 2, 0, 0)
    assert (ps["waves_per_row"], ps["packs_per_lane"], ps["rows_per_block"]) == (1, 1, 8)


def test_plan_empty_and_errors(lib):
    assert B.far_plan(0, 4096, 2, 0, 0)["variant"] == "empty"
    out = B.far_plan_t()
    assert lib.far_plan(4, 4096, 0, 0, 0, ctypes.byref(out)) == NPART
    assert lib.far_plan(4, 4096, 9, 0, 0, ctypes.byref(out)) == NPART
    assert lib.far_plan(4, 4096, 2, 2, 0, ctypes.byref(out)) == DTYPE
    assert lib.far_plan(4, 4096, 2, 0, 5, ctypes.byref(out)) == QARGS
    assert lib.far_plan(-1, 4096, 2, 0, 0, ctypes.byref(out)) == SHAPE
    assert lib.far_plan(4, 0, 2, 0, 0, ctypes.byref(out)) == SHAPE
    assert lib.far_plan(4, (1 << 30) + 1, 2, 0, 0, ctypes.byref(out)) == SHAPE
    assert lib.far_plan(4, 4096, 2, 0, 0, None) == NULLP


# ------------------------------------------------------------------ validation
# Fake, well-separated, 256-byte aligned "device" addresses: validation never
# dereferences them, and every call below fails before a launch.

T, H = 4, 64
TB = T * H * 2
BASE = 0x7F0000000000
STRIDE = 1 << 20


def addr(i, off=0):
    return BASE + i * STRIDE + off


def call(lib, P=2, partials=None, residual=addr(10), gamma=addr(11), t=T, h=H, dtype=0,
         quant=0, scale=None, norm_out=addr(20), residual_out=addr(21), quant_out=None,
         scale_out=None, plan=None, workspace=None, workspace_bytes=0, ex=False, noalloc=False):
    if partials is None:
        partials = [addr(i) for i in range(P)]
    arr = (ctypes.c_void_p * max(len(partials), 1))(*partials) if partials != "null" else None
    args = [arr, P, residual, gamma, t, h, dtype, 1e-6, 0.0, quant, scale, norm_out,
            residual_out, quant_out, scale_out, None]
    if noalloc:
        return lib.far_fused_add_rmsnorm_noalloc(*args)
    if plan is None and not ex:
        return lib.far_fused_add_rmsnorm(*args)
    return lib.far_fused_add_rmsnorm_ex(*args, ctypes.byref(plan) if plan is not None else None,
                                        workspace, workspace_bytes)


def test_scalar_errors(lib):
    assert call(lib, P=0, partials=[addr(0)]) == NPART
    assert call(lib, P=9, partials=[addr(i) for i in range(9)]) == NPART
    assert call(lib, dtype=5) == DTYPE
    assert call(lib, quant=7) == QARGS
    assert call(lib, quant=5) == QARGS
    assert call(lib, t=-1) == SHAPE
    assert call(lib, h=0) == SHAPE
    assert call(lib, h=(1 << 30) + 8) == SHAPE


def _bad_plan():
    p = B.far_plan_t()
    p.variant, p.waves_per_row, p.rows_per_block, p.packs_per_lane = 1, 1, 1, 0  # invalid depth
    return p


def test_null_pointers(lib):
    assert call(lib, partials="null") == NULLP
    assert call(lib, partials=[addr(0), None]) == NULLP
    assert call(lib, gamma=None) == NULLP
    assert call(lib, norm_out=None) == NULLP          # required without quantisation
    # residual and residual_out are optional (no-residual and residual-discarding
    # forms): they pass the pointer checks and stop only at the (invalid) forced plan
    assert call(lib, residual=None, plan=_bad_plan()) == PLAN
    assert call(lib, residual_out=None, plan=_bad_plan()) == PLAN
    assert call(lib, residual=None, residual_out=None, plan=_bad_plan()) == PLAN
    assert call(lib, quant=2, norm_out=None, residual_out=None, quant_out=addr(31),
                scale_out=addr(32), plan=_bad_plan()) == PLAN


def test_empty_batch_is_ok_without_launch(lib):
    # T == 0: FAR_OK and nothing launched (so this is safe without a GPU), even with
    # null tensor pointers (empty torch tensors may have a null data pointer)
    assert call(lib, t=0, residual=None, gamma=None, norm_out=None, residual_out=None) == OK


def test_quant_argument_rules(lib):
    # none: no scale / quant_out / scale_out
    assert call(lib, scale=addr(30)) == QARGS
    assert call(lib, quant_out=addr(31)) == QARGS
    assert call(lib, scale_out=addr(32)) == QARGS
    # static: scale and quant_out required, no scale_out
    assert call(lib, quant=1, quant_out=addr(31)) == QARGS
    assert call(lib, quant=1, scale=addr(30)) == QARGS
    assert call(lib, quant=1, scale=addr(30), quant_out=addr(31), scale_out=addr(32)) == QARGS
    # dynamic: quant_out and scale_out required, no scale
    assert call(lib, quant=2, quant_out=addr(31)) == QARGS
    assert call(lib, quant=2, scale_out=addr(32)) == QARGS
    assert call(lib, quant=2, quant_out=addr(31), scale_out=addr(32), scale=addr(30)) == QARGS


def test_alias_rules(lib):
    # outputs identical to an input or to each other
    assert call(lib, norm_out=addr(0)) == ALIAS
    assert call(lib, norm_out=addr(10)) == ALIAS
    assert call(lib, norm_out=addr(21)) == ALIAS                      # = residual_out
    assert call(lib, norm_out=addr(11)) == ALIAS                      # = gamma
    # partial overlaps
    assert call(lib, norm_out=addr(0, TB - 2)) == ALIAS
    assert call(lib, residual_out=addr(10, 128)) == ALIAS             # shifted residual
    assert call(lib, residual_out=addr(11, -TB + 2)) == ALIAS          # runs into gamma
    assert call(lib, quant=2, norm_out=None, quant_out=addr(31), scale_out=addr(31, T * H - 4)) == ALIAS
    assert call(lib, quant=1, norm_out=None, scale=addr(31, 8), quant_out=addr(31)) == ALIAS


def test_residual_out_never_over_gamma_or_scale(lib):
    """residual_out may coincide only with the residual or a partial. With T == 1 a row
    tensor has exactly gamma's size, and with T * H == 2 exactly the static scale's, so
    an exact-match rule on sizes alone would let the new residual overwrite tensors
    that every row reads."""
    assert call(lib, t=1, residual_out=addr(11)) == ALIAS                  # = gamma, T = 1
    assert call(lib, t=1, residual_out=addr(11), plan=_bad_plan()) == ALIAS
    assert call(lib, t=2, residual_out=addr(11)) == ALIAS                  # = gamma, T = 2
    # [1, 2] bf16 tensors are 4 bytes, as large as the static scale
    assert call(lib, t=1, h=2, quant=1, norm_out=None, scale=addr(30), quant_out=addr(31),
                residual_out=addr(30)) == ALIAS
    # the allowed forms still pass the alias check at T == 1 (they stop at the bad plan)
    assert call(lib, t=1, residual_out=addr(10), plan=_bad_plan()) == PLAN
    assert call(lib, t=1, residual_out=addr(0), plan=_bad_plan()) == PLAN


def test_allowed_in_place_forms_pass_validation(lib):
    # residual_out == residual and residual_out == partials[0] are allowed; with a forced
    # plan that cannot fit, the call stops at the plan check, i.e. after the alias check
    bad = B.far_plan_t()
    bad.variant = 1
    bad.waves_per_row = 1
    bad.packs_per_lane = 1   # 64 lanes x 1 pack < 8 packs needed? H=64 -> 8 packs: fits
    bad.rows_per_block = 1
    bad.packs_per_lane = 0   # invalid depth
    assert call(lib, residual_out=addr(10), plan=bad) == PLAN
    assert call(lib, residual_out=addr(0), plan=bad) == PLAN
    assert call(lib, residual_out=addr(1), plan=bad) == PLAN          # exactly a partial


def test_plan_errors(lib):
    def plan(**kw):
        p = B.far_plan_t()
        p.variant, p.waves_per_row, p.rows_per_block, p.packs_per_lane = 1, 1, 1, 1
        for k, v in kw.items():
            setattr(p, k, v)
        return p
    assert call(lib, h=64 * 8 * 2, plan=plan()) == PLAN                # 128 packs > 64 lanes
    assert call(lib, plan=plan(waves_per_row=17)) == PLAN
    assert call(lib, plan=plan(packs_per_lane=B.FAR_MAX_PACKS_PER_LANE + 1)) == PLAN
    assert call(lib, plan=plan(rows_per_block=0)) == PLAN
    assert call(lib, plan=plan(waves_per_row=16, rows_per_block=2)) == PLAN   # 2048 lanes
    assert call(lib, plan=plan(variant=0)) == PLAN
    assert call(lib, plan=plan(variant=3)) == PLAN
    assert call(lib, h=64 * 8 + 4, plan=plan()) == PLAN                # 64 whole packs + a partial one
    # a tensor at an odd byte address cannot take the vector variant (element-aligned
    # ones can: 16-byte accesses need no alignment on this hardware)
    assert call(lib, residual=addr(10, 1), plan=plan()) == PLAN
    assert call(lib, norm_out=addr(20, 3), plan=plan()) == PLAN


def test_binding_requires_device_tensors():
    import torch
    x = torch.zeros(2, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        B.far_fused_add_rmsnorm([x], x, x[0], 1e-6, 0.0, None, None, x.clone(), x.clone(), None, None)


def test_binding_rejects_wrong_dtype_before_device():
    import torch
    x = torch.zeros(2, 8, dtype=torch.float32)
    with pytest.raises((TypeError, ValueError)):
        B.fused_add_rmsnorm([x], x, x[0], 1e-6)


def test_group_and_tensor_modes_arguments(lib):
    G = -(-H // B.FAR_FP8_GROUP)
    q = dict(norm_out=None, quant_out=addr(31), scale_out=addr(32))
    # group: like the per-token mode, scale_out is [T, G]
    assert call(lib, quant=3, quant_out=addr(31)) == QARGS
    assert call(lib, quant=3, scale=addr(30), **q) == QARGS
    assert call(lib, quant=3, norm_out=None, quant_out=addr(31), scale_out=addr(31, T * H - 4)) == ALIAS
    assert call(lib, quant=3, plan=_bad_plan(), **q) == PLAN
    # tensor: needs a workspace of 8 * T bytes, which overlaps nothing
    assert B.far_workspace_bytes(T, H, "tensor") == 8 * T
    assert B.far_workspace_bytes(T, H, "dynamic") == 0
    assert B.far_workspace_bytes(-1, H, "tensor") == -1
    assert call(lib, quant=4, **q) == WS                                  # plain entry point
    assert call(lib, quant=4, ex=True, workspace=addr(40), workspace_bytes=8 * T - 1, **q) == WS
    assert call(lib, quant=4, ex=True, workspace=addr(31), workspace_bytes=8 * T, **q) == ALIAS
    assert call(lib, quant=4, plan=_bad_plan(), workspace=addr(40), workspace_bytes=8 * T, **q) == PLAN
    # T == 0 needs nothing
    assert call(lib, quant=4, t=0, **q) == OK
    assert G == 1


def test_missing_library_fails_loudly(tmp_path):
    """No fallback: without the HIP library every entry point raises."""
    import importlib
    import residual_add_rmsnorm_fp32_amd.binding as binding
    fresh = importlib.reload(binding)
    try:
        with pytest.raises(fresh.FarLibraryMissing):
            fresh.load_library(str(tmp_path / "libfar.so"))
    finally:
        importlib.reload(binding)


def test_noalloc_validates_before_touching_the_device(lib):
    """The no-allocation entry point rejects a per-tensor batch beyond its scratch
    (8 * T > 2 MiB) and every bad argument before any HIP call, so these run without a
    GPU; T == 0 is OK with nothing launched."""
    assert B.FAR_NOALLOC_SCRATCH_BYTES == 2 * 1024 * 1024
    text = open(HEADER).read()
    assert re.search(r"#define\s+FAR_NOALLOC_SCRATCH_BYTES\s+\(2 \* 1024 \* 1024\)", text)
    q = dict(norm_out=None, quant_out=addr(31), scale_out=addr(32))
    limit_t = B.FAR_NOALLOC_SCRATCH_BYTES // 8
    assert call(lib, quant=4, t=limit_t + 1, noalloc=True, **q) == SCRATCH
    # at the limit the scratch suffices: the call gets as far as the alias check
    assert call(lib, quant=4, t=limit_t, noalloc=True, norm_out=None, quant_out=addr(31),
                scale_out=addr(31, 8)) == ALIAS
    # the same argument rules as the other entry points
    assert call(lib, P=9, partials=[addr(i) for i in range(9)], noalloc=True) == NPART
    assert call(lib, gamma=None, noalloc=True) == NULLP
    assert call(lib, t=1, residual_out=addr(11), noalloc=True) == ALIAS
    assert call(lib, quant=4, noalloc=True, scale=addr(30), **q) == QARGS
    assert call(lib, quant=4, t=0, noalloc=True, **q) == OK
    assert "scratch" in B.far_status_string(SCRATCH)
