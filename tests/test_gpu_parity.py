"""HIP path vs the CPU oracle, element by element, through the C ABI (needs a GPU)."""

import itertools
import sys

import numpy as np
import pytest
import torch

import compare as cmp
import gpu_util as G
from residual_add_rmsnorm_fp32_amd import binding as B
from residual_add_rmsnorm_fp32_amd import workloads as wk

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


# ------------------------------------------------------------------ the named workloads

@pytest.mark.parametrize("quant", ["group", "tensor"])
def test_c4_shape_group_and_tensor_scales(quant):
    """The prefill workload's inputs with per-group (128) and per-tensor dynamic scales."""
    wl = wk.WORKLOADS["c4"]
    inp = wk.make_inputs(wl)
    _say(f"[parity] c4 inputs, {quant} scales, plan {B.far_plan(wl.T, wl.H, wl.P, G.TORCH_DT[wl.dtype], quant)}")
    gpu = G.run_gpu(inp, wl.dtype, wl.eps, wl.weight_bias, quant, want_norm=True)
    ref = G.run_oracle(inp, wl.dtype, wl.eps, wl.weight_bias, quant)
    stats = G.compare(gpu, ref, wl.dtype, quant, inp, tag=f"c4 {quant}")
    _say(f"[parity] c4 {quant}: {stats}")
    gpu2 = G.run_gpu(inp, wl.dtype, wl.eps, wl.weight_bias, quant, want_norm=False)
    for k in ("quant_out", "new_residual", "scale_out"):
        assert np.array_equal(gpu2[k], gpu[k]), k


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_workload_full(name):
    wl = wk.WORKLOADS[name]
    _say(f"[parity] workload {name}: P={wl.P} T={wl.T} H={wl.H} {wl.dtype} quant={wl.quant}")
    inp = wk.make_inputs(wl)
    gpu = G.run_gpu(inp, wl.dtype, wl.eps, wl.weight_bias, wl.quant, want_norm=True)
    ref = G.run_oracle(inp, wl.dtype, wl.eps, wl.weight_bias, wl.quant)
    stats = G.compare(gpu, ref, wl.dtype, wl.quant, inp, tag=name)
    _say(f"[parity] {name}: {stats}")
    assert stats["new_residual"]["cancellation_excused"] == 0
    # every element's terms lie within the window where the sum is exact, so the new
    # residual is the oracle's bit for bit
    assert stats["new_residual"]["max_ulp"] == 0
    if wl.quant != "none":
        # the timed configuration writes no norm_out: the codes must not depend on it
        gpu2 = G.run_gpu(inp, wl.dtype, wl.eps, wl.weight_bias, wl.quant, want_norm=False)
        assert np.array_equal(gpu2["quant_out"], gpu["quant_out"])
        assert np.array_equal(gpu2["new_residual"], gpu["new_residual"])
        if wl.quant == "dynamic":
            assert np.array_equal(gpu2["scale_out"], gpu["scale_out"])


@pytest.mark.parametrize("T", [1, 8, 32])
def test_c2_token_sweep(T):
    wl = wk.WORKLOADS["c2"]
    _say(f"[parity] c2 sweep T={T}")
    inp = wk.make_inputs(wl, T=T)
    gpu = G.run_gpu(inp, wl.dtype, wl.eps, wl.weight_bias, wl.quant)
    ref = G.run_oracle(inp, wl.dtype, wl.eps, wl.weight_bias, wl.quant)
    stats = G.compare(gpu, ref, wl.dtype, wl.quant, inp, tag=f"c2 T={T}")
    assert stats["new_residual"]["cancellation_excused"] == 0
    assert stats["new_residual"]["max_ulp"] == 0


def test_c5_full_size_every_row():
    """[4, 4096, 3584] fp16, P = 8, weight_bias = 1, passed 3-D; every one of the 16384
    rows of new_residual and norm_out is compared with the oracle (in row chunks)."""
    wl = wk.WORKLOADS["c5"]
    _say("[parity] c5 full size, 3-D input, every row against the oracle")
    inp = wk.make_inputs(wl)
    gpu = G.run_gpu(inp, wl.dtype, wl.eps, wl.weight_bias, wl.quant, shape=wl.view_shape)
    assert gpu["new_residual"].shape == (wl.T, wl.H) and gpu["norm_out"].shape == (wl.T, wl.H)
    stats = G.compare_rows_chunked(gpu, inp, wl.dtype, wl.eps, wl.weight_bias, wl.quant, tag="c5")
    assert len(stats) * 512 >= wl.T
    worst = {k: max(s[k]["max_ulp"] for s in stats) for k in ("new_residual", "norm_out")}
    excused = sum(s["new_residual"]["cancellation_excused"] for s in stats)
    _say(f"[parity] c5: {wl.T} rows, max ulp {worst}, cancellation excused {excused}")
    assert excused == 0
    # fp16 terms are summed exactly (binary64) and rounded once: the oracle's codes
    assert worst["new_residual"] == 0


def _codes_of(values, dtype):
    return wk.to_codes(np.asarray(values, np.float64), dtype)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_sum_rounds_once_across_binades(dtype):
    """Rows whose terms span many binades. 1 + u/2 + tiny (u the storage ulp at 1) lies
    just above a rounding midpoint, so the new residual is 1 + u; a binary32 sum drops
    the tiny term and lands on the midpoint itself, which rounds to even (1.0). fp16
    terms are summed in binary64 and must give the oracle's codes exactly; bf16 terms
    are summed in binary32 (exact only within about 12 binades, here exceeded on
    purpose) and stay within the one-ulp tolerance."""
    u = 2.0 ** -10 if dtype == "fp16" else 2.0 ** -7
    tiny = 2.0 ** -24 if dtype == "fp16" else 2.0 ** -40
    H = 64
    rows = [
        [1.0, u / 2, tiny, 0.0],          # just above the midpoint -> 1 + u
        [1.0, u / 2, -tiny, 0.0],         # just below -> 1
        [-1.0, -u / 2, -tiny, 0.0],       # mirrored -> -(1 + u)
        [2.0, u, tiny, -tiny],            # exact midpoint of the 2-binade (tie to even)
        [1.5, u / 2, tiny, tiny],         # above the midpoint above 1.5
        [3.0, -u, tiny, 0.0],             # below 3 - u (between codes)
    ]
    T, P = len(rows), 3
    partials = np.zeros((P, T, H))
    residual = np.zeros((T, H))
    for t, (a, b, c, d) in enumerate(rows):
        partials[0, t, :], partials[1, t, :], partials[2, t, :], residual[t, :] = a, b, c, d
    inp = {"partials": np.stack([_codes_of(partials[p], dtype) for p in range(P)]),
           "residual": _codes_of(residual, dtype),
           "gamma": _codes_of(np.ones(H), dtype)}
    gpu = G.run_gpu(inp, dtype, 1e-6, 0.0, "none")
    ref = G.run_oracle(inp, dtype, 1e-6, 0.0, "none")
    stats = G.compare(gpu, ref, dtype, "none", inp, tag=f"binades {dtype}")
    _say(f"[parity] sum across binades {dtype}: {stats}")
    if dtype == "fp16":
        assert np.array_equal(gpu["new_residual"], ref["new_residual"])
        # the first row really needs the exact sum: the oracle rounds it up to 1 + u
        assert cmp.decode(ref["new_residual"][0, 0], dtype) == 1.0 + u


@pytest.mark.parametrize("T,H,quant,variant", [((1 << 20) + 3, 4, "dynamic", "generic"),
                                               ((1 << 23) + 3, 4, "dynamic", "vector"),
                                               ((1 << 23) + 5, 8, "none", "vector")])
def test_more_rows_than_one_grid_holds(T, H, quant, variant):
    """Beyond 2^20 workgroups the grid is capped and both kernels loop over rows: the
    generic kernel (one workgroup per row) past 2^20 rows, the vector kernel (eight
    one-pack rows per workgroup, whole or partial) past 2^23."""
    forced = {"variant": "generic"} if variant == "generic" else None
    plan = B.far_plan(T, H, 1, G.TORCH_DT["bf16"], quant)
    _say(f"[parity] T={T} H={H} {quant} {variant} auto plan={plan}")
    if variant == "vector":
        assert plan["variant"] == "vector"
        assert plan["grid_blocks"] == 1 << 20 and plan["grid_blocks"] * plan["rows_per_block"] < T
    inp = wk.random_case(4242, 1, T, H, "bf16")
    gpu = G.run_gpu(inp, "bf16", 1e-6, 0.0, quant, plan=forced)
    stats = G.compare_rows_chunked(gpu, inp, "bf16", 1e-6, 0.0, quant, chunk=1 << 18,
                                   tag=f"T={T}")
    assert len(stats) == -(-T // (1 << 18))


# ------------------------------------------------------------------ shapes and edges

EDGE_CASES = [
    # (P, T, H, dtype, quant)
    (1, 1, 4, "bf16", "none"), (2, 3, 8, "bf16", "dynamic"), (3, 2, 12, "fp16", "static"),
    (8, 81, 2056, "bf16", "none"), (2, 17, 5120, "fp16", "dynamic"), (4, 3, 8192, "bf16", "static"),
    (5, 4, 8200, "bf16", "dynamic"), (2, 5, 16384, "fp16", "none"), (3, 2, 32768, "bf16", "dynamic"),
    (7, 9, 1000, "fp16", "none"), (6, 33, 4096, "bf16", "static"), (1, 4097, 64, "bf16", "dynamic"),
    (8, 2, 40960, "bf16", "none"), (2, 2, 40968, "fp16", "static"), (4, 300, 520, "bf16", "dynamic"),
    (8, 3, 3584, "fp16", "dynamic"), (2, 2, 65536, "bf16", "dynamic"),
    (2, 19, 5120, "bf16", "group"), (3, 5, 2056, "fp16", "group"), (1, 3, 12, "bf16", "group"),
    (8, 4, 40960, "bf16", "group"), (2, 2, 33000, "fp16", "group"),
    (2, 19, 5120, "bf16", "tensor"), (4, 7, 2056, "fp16", "tensor"), (1, 3, 12, "bf16", "tensor"),
    (8, 33, 4096, "bf16", "tensor"), (2, 2, 40968, "fp16", "tensor"),
]


@pytest.mark.parametrize("P,T,H,dtype,quant", EDGE_CASES)
def test_edge_shapes(P, T, H, dtype, quant):
    _say(f"[parity] edge P={P} T={T} H={H} {dtype} {quant} plan={B.far_plan(T, H, P, G.TORCH_DT[dtype])}")
    inp = wk.random_case(1000 + P * 7 + T + H, P, T, H, dtype)
    inp["scale"] = np.array([0.05], np.float32)
    eps, wb = 1e-6, (1.0 if dtype == "fp16" else 0.0)
    gpu = G.run_gpu(inp, dtype, eps, wb, quant)
    ref = G.run_oracle(inp, dtype, eps, wb, quant)
    G.compare(gpu, ref, dtype, quant, inp, tag=f"P{P} T{T} H{H}")


# Rows whose length is not a whole number of 16-byte packs (H % 8 != 0): the vector
# kernel's partial-last-pack form. The lengths put the partial pack (n = H % 8 = 1..7
# elements) in the first lane, mid-wave, at a wave boundary, in a deeper slot, and at
# the vector kernels' longest row (40959 = 5119 packs + 7 elements).
RAGGED_H = [1, 2, 3, 5, 7, 9, 12, 15, 61, 127, 129, 516, 1001, 1029, 4099, 5124, 8191, 40959]


@pytest.mark.parametrize("quant", ["none", "static", "dynamic", "group", "tensor"])
@pytest.mark.parametrize("H", RAGGED_H)
def test_partial_last_pack(H, quant):
    dtype = "bf16" if H % 2 else "fp16"
    P, T = 1 + H % 8, 7
    plan = B.far_plan(T, H, P, G.TORCH_DT[dtype], quant)
    _say(f"[parity] partial pack P={P} T={T} H={H} {dtype} {quant} plan={plan}")
    # the per-group mode holds at most four packs per lane: longer rows are generic
    max_n = 4 if quant == "group" else B.FAR_MAX_PACKS_PER_LANE
    assert plan["variant"] == ("vector" if -(-H // 8) <= 16 * 64 * max_n else "generic")
    inp = wk.random_case(500 + H, P, T, H, dtype)
    inp["scale"] = np.array([0.05], np.float32)
    wb = 1.0 if dtype == "fp16" else 0.0
    ref = G.run_oracle(inp, dtype, 1e-6, wb, quant)
    gpu = G.run_gpu(inp, dtype, 1e-6, wb, quant, want_norm=True)
    stats = G.compare(gpu, ref, dtype, quant, inp, tag=f"partial pack H={H} {quant}")
    assert stats["new_residual"]["cancellation_excused"] == 0
    if dtype == "fp16":  # the binary64 sum is exact: the oracle's codes
        assert stats["new_residual"]["max_ulp"] == 0
    if quant != "none":
        # the codes do not depend on whether norm_out is written
        gpu2 = G.run_gpu(inp, dtype, 1e-6, wb, quant, want_norm=False)
        assert np.array_equal(gpu2["quant_out"], gpu["quant_out"])


@pytest.mark.parametrize("quant", ["none", "dynamic", "group"])
@pytest.mark.parametrize("form", ["no_residual", "discard_residual", "in_place", "in_place_partial"])
def test_partial_last_pack_forms(form, quant):
    """The residual forms on rows ending in a partial pack (H = 1001: 125 packs and
    one element): no residual input, no new residual, and the new residual written
    over the residual or over a partial."""
    dtype, P, T, H = "bf16", 3, 11, 1001
    inp = wk.random_case(61, P, T, H, dtype)
    no_res = form == "no_residual"
    ref = G.run_oracle(inp, dtype, 1e-6, 0.0, quant, no_residual=no_res)
    if form in ("no_residual", "discard_residual"):
        gpu = G.run_gpu(inp, dtype, 1e-6, 0.0, quant, want_norm=True, no_residual=no_res,
                        discard_residual=form == "discard_residual")
        G.compare(gpu, ref, dtype, quant, inp, tag=f"{form} {quant}", no_residual=no_res)
        return
    partials = [G.to_dev(p, dtype) for p in inp["partials"]]
    residual = G.to_dev(inp["residual"], dtype)
    gamma = G.to_dev(inp["gamma"], dtype)
    target = residual if form == "in_place" else partials[1]
    outs = B.fused_add_rmsnorm(partials, residual, gamma, 1e-6, quant=quant, want_norm_out=True,
                               residual_out=target)
    torch.cuda.synchronize()
    assert outs[1].data_ptr() == target.data_ptr()
    gpu = {"new_residual": G.codes_of(target), "norm_out": G.codes_of(outs[-1] if quant != "none" else outs[0])}
    if quant != "none":
        gpu["quant_out"] = G.codes_of(outs[0])
        sc = G.codes_of(outs[2])
        gpu["scale_out"] = sc.reshape(T, -1) if quant == "group" else sc.reshape(-1)
    G.compare(gpu, ref, dtype, quant, inp, tag=f"{form} {quant}")


def test_c4_shape_with_partial_pack():
    """c4's parameters and input recipe at H = 5124 (640 whole packs and one of four
    elements), every row against the oracle: the partial-last-pack form at the
    prefill shape the benchmark times."""
    from residual_add_rmsnorm_fp32_amd.workloads import with_overrides
    wl = with_overrides(wk.WORKLOADS["c4"], H=5124)
    inp = wk.make_inputs(wl)
    plan = B.far_plan(wl.T, wl.H, wl.P, G.TORCH_DT[wl.dtype], wl.quant)
    _say(f"[parity] c4 at H=5124, plan {plan}")
    assert plan["variant"] == "vector"
    gpu = G.run_gpu(inp, wl.dtype, wl.eps, wl.weight_bias, wl.quant, want_norm=True)
    ref = G.run_oracle(inp, wl.dtype, wl.eps, wl.weight_bias, wl.quant)
    stats = G.compare(gpu, ref, wl.dtype, wl.quant, inp, tag="c4 H=5124")
    _say(f"[parity] c4 H=5124: {stats}")
    assert stats["new_residual"]["cancellation_excused"] == 0
    assert stats["new_residual"]["max_ulp"] == 0


def _valid_plans(T, H, quant="none"):
    packs = -(-H // 8)  # the last one partial when H % 8 != 0
    plans = [{"variant": "generic"}]
    max_n = 4 if quant == "group" else B.FAR_MAX_PACKS_PER_LANE
    for w in range(1, 17):
        for n in range(1, max_n + 1):
            if w * 64 * n < packs or (w - 1) * 64 * n >= packs:
                continue
            for r in (1, 2, 4):
                if r * w * 64 <= 1024:
                    plans.append({"variant": "vector", "waves_per_row": w, "packs_per_lane": n,
                                  "rows_per_block": r})
    return plans


@pytest.mark.parametrize("H", [1792, 1795])
@pytest.mark.parametrize("dtype,quant", [("bf16", "dynamic"), ("fp16", "none"), ("bf16", "static"),
                                         ("bf16", "group"), ("fp16", "tensor")])
def test_every_plan_same_input(dtype, quant, H):
    """Every launch shape of the library on one input, all within tolerance. 1792
    elements are 224 packs (ragged over most team sizes); 1795 add a partial pack of
    three elements, which lands in a different lane, wave and slot for each shape."""
    P, T = 3, 13
    inp = wk.random_case(77, P, T, H, dtype)
    inp["scale"] = np.array([0.5], np.float32)
    ref = G.run_oracle(inp, dtype, 1e-5, 0.0, quant)
    plans = _valid_plans(T, H, quant)
    _say(f"[parity] {len(plans)} plans, {dtype} {quant}")
    for plan in plans:
        gpu = G.run_gpu(inp, dtype, 1e-5, 0.0, quant, plan=plan)
        G.compare(gpu, ref, dtype, quant, inp, tag=str(plan))


@pytest.mark.parametrize("variant", ["auto", "generic"])
@pytest.mark.parametrize("quant", ["none", "static", "dynamic", "group", "tensor"])
@pytest.mark.parametrize("form", ["no_residual", "discard_residual", "neither"])
def test_optional_residual_forms(form, quant, variant):
    """No residual input (new residual = sum of partials) and no new residual written
    (only the normalised / quantised output), on both kernels."""
    dtype, P, T, H = "bf16", 3, 37, 2560
    inp = wk.random_case(31, P, T, H, dtype)
    inp["scale"] = np.array([0.25], np.float32)
    no_res = form in ("no_residual", "neither")
    discard = form in ("discard_residual", "neither")
    plan = {"variant": "generic"} if variant == "generic" else None
    gpu = G.run_gpu(inp, dtype, 1e-6, 0.0, quant, want_norm=(quant == "none"), plan=plan,
                    no_residual=no_res, discard_residual=discard)
    assert ("new_residual" in gpu) == (not discard)
    ref = G.run_oracle(inp, dtype, 1e-6, 0.0, quant, no_residual=no_res)
    G.compare(gpu, ref, dtype, quant, inp, tag=f"{form} {quant} {variant}", no_residual=no_res)


@pytest.mark.parametrize("where", ["residual", "partial0"])
def test_in_place_residual(where):
    dtype, P, T, H = "bf16", 3, 40, 2048
    inp = wk.random_case(5, P, T, H, dtype)
    ref = G.run_oracle(inp, dtype, 1e-6, 0.0, "none")
    partials = [G.to_dev(p, dtype) for p in inp["partials"]]
    residual = G.to_dev(inp["residual"], dtype)
    gamma = G.to_dev(inp["gamma"], dtype)
    target = residual if where == "residual" else partials[0]
    norm = torch.empty_like(residual)
    B.far_fused_add_rmsnorm(partials, residual, gamma, 1e-6, 0.0, None, None, norm, target, None, None)
    torch.cuda.synchronize()
    gpu = {"new_residual": G.codes_of(target), "norm_out": G.codes_of(norm)}
    G.compare(gpu, ref, dtype, "none", tag=f"in place {where}")
    # the other inputs are untouched
    for i, p in enumerate(partials):
        if p is not target:
            assert np.array_equal(G.codes_of(p), inp["partials"][i])
    if where != "residual":
        assert np.array_equal(G.codes_of(residual), inp["residual"])


@pytest.mark.parametrize("H", [1024, 1021])
@pytest.mark.parametrize("quant", ["none", "static", "dynamic", "group", "tensor"])
def test_element_aligned_views(quant, H):
    """Views starting one element (2 bytes) into larger buffers: not 16-byte aligned,
    still served by the vector kernels (16-byte accesses at any address), with whole
    rows of packs and with a partial last pack."""
    dtype, P, T = "fp16", 2, 7
    inp = wk.random_case(9, P, T, H, dtype)
    inp["scale"] = np.float32(0.05)
    ref = G.run_oracle(inp, dtype, 1e-6, 0.0, quant)
    assert B.far_plan(T, H, P, G.TORCH_DT[dtype], quant)["variant"] == "vector"

    def shifted(codes, dt=G.TORCH_DT[dtype]):
        buf = torch.empty(codes.size + 1, dtype=dt, device="cuda")
        v = buf[1:].view(codes.shape)
        v.copy_(G.to_dev(codes, dtype))
        return v

    def shifted_empty(shape, dt):
        n = int(np.prod(shape))
        return torch.empty(n + 1, dtype=dt, device="cuda")[1:].view(shape)

    partials = [shifted(p) for p in inp["partials"]]
    residual = shifted(inp["residual"])
    gamma = shifted(inp["gamma"])
    assert residual.data_ptr() % 16 != 0 and gamma.data_ptr() % 16 != 0
    kw = {"norm_out": shifted_empty((T, H), G.TORCH_DT[dtype]),
          "residual_out": shifted_empty((T, H), G.TORCH_DT[dtype])}
    scale = None
    if quant != "none":
        kw["quant_out"] = shifted_empty((T, H), torch.uint8)
        assert kw["quant_out"].data_ptr() % 2 == 1
    if quant == "static":
        scale = torch.tensor([0.05], dtype=torch.float32, device="cuda")
    outs = B.fused_add_rmsnorm(partials, residual, gamma, 1e-6, 0.0, quant=quant, scale=scale,
                               want_norm_out=True, **kw)
    torch.cuda.synchronize()
    gpu = {"new_residual": G.codes_of(outs[1]), "norm_out": G.codes_of(outs[-1] if quant != "none" else outs[0])}
    if quant != "none":
        gpu["quant_out"] = G.codes_of(outs[0])
    if quant in G.DYNAMIC:
        sc = G.codes_of(outs[2])
        gpu["scale_out"] = sc.reshape(T, -1) if quant == "group" else sc.reshape(-1)
    G.compare(gpu, ref, dtype, quant, inp, tag=f"element-aligned {quant}")


@pytest.mark.parametrize("quant", ["none", "dynamic", "group"])
def test_odd_address_tensors_take_generic_path(quant):
    """Tensors at odd byte addresses (possible through the C ABI only) take the generic
    kernel; the results are the same."""
    import ctypes
    dtype, P, T, H = "bf16", 3, 5, 264
    inp = wk.random_case(19, P, T, H, dtype)
    ref = G.run_oracle(inp, dtype, 1e-6, 0.0, quant)
    lib = B.load_library()

    def odd_bytes(codes=None, nbytes=None):
        raw = codes.view(np.uint8).reshape(-1) if codes is not None else None
        n = raw.size if raw is not None else nbytes
        buf = torch.zeros(n + 1, dtype=torch.uint8, device="cuda")
        if raw is not None:
            buf[1:].copy_(torch.from_numpy(raw.copy()).cuda())
        return buf

    bufs = {"p%d" % i: odd_bytes(np.ascontiguousarray(p)) for i, p in enumerate(inp["partials"])}
    bufs["res"] = odd_bytes(np.ascontiguousarray(inp["residual"]))
    bufs["gamma"] = odd_bytes(np.ascontiguousarray(inp["gamma"]))
    bufs["norm"] = odd_bytes(nbytes=T * H * 2)
    bufs["res_out"] = odd_bytes(nbytes=T * H * 2)
    groups = -(-H // 128)
    if quant != "none":
        bufs["q"] = odd_bytes(nbytes=T * H)
    n_sc = {"dynamic": T, "group": T * groups}.get(quant, 0)
    scale_out = torch.zeros(max(n_sc, 1), dtype=torch.float32, device="cuda")
    ptr = {k: v.data_ptr() + 1 for k, v in bufs.items()}
    arr = (ctypes.c_void_p * P)(*[ptr["p%d" % i] for i in range(P)])
    torch.cuda.synchronize()
    st = lib.far_fused_add_rmsnorm(arr, P, ptr["res"], ptr["gamma"], T, H, 0, 1e-6, 0.0,
                                   G.QUANT_ID[quant], None, ptr["norm"], ptr["res_out"],
                                   ptr.get("q"), scale_out.data_ptr() if n_sc else None,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.far_status_string(st)
    torch.cuda.synchronize()

    def codes16(k):
        return bufs[k][1:].cpu().numpy().copy().view(np.uint16).reshape(T, H)
    gpu = {"new_residual": codes16("res_out"), "norm_out": codes16("norm")}
    if quant != "none":
        gpu["quant_out"] = bufs["q"][1:].cpu().numpy().reshape(T, H)
        sc = scale_out.cpu().numpy()
        gpu["scale_out"] = sc.reshape(T, groups) if quant == "group" else sc.reshape(-1)
    G.compare(gpu, ref, dtype, quant, inp, tag=f"odd address {quant}")


def test_zero_rows_and_scale_one():
    dtype, P, T, H = "bf16", 2, 6, 256
    inp = wk.random_case(3, P, T, H, dtype)
    inp["partials"][:, 2] = 0
    inp["residual"][2] = 0
    inp["partials"][:, 4] = 0x8000  # -0
    inp["residual"][4] = 0
    inp["partials"][:, 5, 128:] = 0  # second group of row 5 is zero
    inp["residual"][5, 128:] = 0
    for quant in ("dynamic", "group"):
        for plan in (None, {"variant": "generic"}):
            gpu = G.run_gpu(inp, dtype, 1e-6, 0.0, quant, plan=plan)
            ref = G.run_oracle(inp, dtype, 1e-6, 0.0, quant)
            G.compare(gpu, ref, dtype, quant, tag=f"zero rows {quant} {plan}")
            assert np.all(gpu["scale_out"][2] == 1.0) and np.all(gpu["scale_out"][4] == 1.0)
            assert np.all(cmp.decode(gpu["quant_out"][2], "e4m3fn") == 0)
    gpu = G.run_gpu(inp, dtype, 1e-6, 0.0, "group")
    assert gpu["scale_out"][5, 1] == 1.0


def test_nan_and_inf_propagate_like_the_oracle():
    dtype, P, T, H = "fp16", 2, 4, 64
    inp = wk.random_case(4, P, T, H, dtype)
    inp["partials"][0, 1, 5] = 0x7E00      # NaN
    inp["partials"][1, 2, 7] = 0x7C00      # +inf
    inp["partials"][0, 3, 0] = 0x7BFF      # 65504 + 65504 -> overflow to inf
    inp["partials"][1, 3, 0] = 0x7BFF
    for quant in ("none", "dynamic", "group", "tensor"):
        for plan in (None, {"variant": "generic"}):
            gpu = G.run_gpu(inp, dtype, 1e-6, 0.0, quant, plan=plan)
            ref = G.run_oracle(inp, dtype, 1e-6, 0.0, quant)
            G.compare(gpu, ref, dtype, quant, tag=f"nan/inf {quant} {plan}")


def test_deterministic():
    wl = wk.WORKLOADS["c4"]
    inp = wk.make_inputs(wl, T=256)
    a = G.run_gpu(inp, wl.dtype, wl.eps, wl.weight_bias, wl.quant)
    b = G.run_gpu(inp, wl.dtype, wl.eps, wl.weight_bias, wl.quant)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_empty_batch():
    x = torch.empty(0, 4096, dtype=torch.bfloat16, device="cuda")
    g = torch.ones(4096, dtype=torch.bfloat16, device="cuda")
    n, r = B.fused_add_rmsnorm([x, x], x, g, 1e-6)
    assert n.shape == (0, 4096) and r.shape == (0, 4096)


@pytest.mark.parametrize("H", [4104, 4099, 4102])
def test_no_write_outside_outputs(H):
    """Outputs carved out of larger buffers filled with a sentinel: nothing outside the
    [T, H] (or [T]) window changes (rows of whole packs, and rows ending in a partial
    pack of three or six elements)."""
    dtype, P, T = "bf16", 2, 5
    inp = wk.random_case(8, P, T, H, dtype)
    pad = 4096
    def carve(n, dt, fill):
        buf = torch.full((n + 2 * pad,), fill, dtype=dt, device="cuda")
        return buf, buf[pad:pad + n]
    partials = [G.to_dev(p, dtype) for p in inp["partials"]]
    residual = G.to_dev(inp["residual"], dtype)
    gamma = G.to_dev(inp["gamma"], dtype)
    nb, norm = carve(T * H, torch.bfloat16, 7.0)
    rb, rout = carve(T * H, torch.bfloat16, 7.0)
    qb, qout = carve(T * H, torch.uint8, 0x5A)
    sb, sout = carve(T, torch.float32, 7.0)
    assert B.far_plan(T, H, P, torch.bfloat16, "dynamic")["variant"] == "vector"
    ref = G.run_oracle(inp, dtype, 1e-6, 0.0, "dynamic")
    for plan in (None, {"variant": "generic"}):
        B.far_fused_add_rmsnorm(partials, residual, gamma, 1e-6, 0.0, "dynamic", None,
                                norm.view(T, H), rout.view(T, H), qout.view(T, H), sout, plan=plan)
        torch.cuda.synchronize()
        for buf, fill in ((nb, 7.0), (rb, 7.0), (sb, 7.0)):
            assert torch.all(buf[:pad] == fill) and torch.all(buf[-pad:] == fill)
        assert torch.all(qb[:pad] == 0x5A) and torch.all(qb[-pad:] == 0x5A)
        gpu = {"new_residual": G.codes_of(rout.view(T, H)), "norm_out": G.codes_of(norm.view(T, H)),
               "quant_out": G.codes_of(qout.view(T, H)), "scale_out": G.codes_of(sout)}
        G.compare(gpu, ref, dtype, "dynamic", inp, tag=f"carved H={H} {plan}")


def test_graph_replay_matches_eager():
    """The call is capture-safe: a captured graph replayed several times, with eager
    work in between, reproduces the eager result every time."""
    wl = wk.WORKLOADS["c2"]
    inp = wk.make_inputs(wl)
    partials = [G.to_dev(p, wl.dtype) for p in inp["partials"]]
    residual = G.to_dev(inp["residual"], wl.dtype)
    gamma = G.to_dev(inp["gamma"], wl.dtype)
    norm_e, res_e = B.fused_add_rmsnorm(partials, residual, gamma, wl.eps)
    torch.cuda.synchronize()
    norm_g = torch.empty_like(norm_e)
    res_g = torch.empty_like(res_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up on the side stream before capture
        B.far_fused_add_rmsnorm(partials, residual, gamma, wl.eps, 0.0, None, None, norm_g, res_g, None, None)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.far_fused_add_rmsnorm(partials, residual, gamma, wl.eps, 0.0, None, None, norm_g, res_g, None, None)
    for i in range(4):
        norm_g.zero_()
        res_g.zero_()
        _ = (residual.float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(norm_g.view(torch.int16), norm_e.view(torch.int16)), f"replay {i}"
        assert torch.equal(res_g.view(torch.int16), res_e.view(torch.int16)), f"replay {i}"


def test_binding_shape_errors():
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    g = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        B.fused_add_rmsnorm([x[:, :32].contiguous()], x, g, 1e-6)
    with pytest.raises(ValueError):
        B.fused_add_rmsnorm([x], x, torch.ones(32, dtype=torch.bfloat16, device="cuda"), 1e-6)
    with pytest.raises(B.FarError) as e:
        B.far_fused_add_rmsnorm([x], x, g, 1e-6, 0.0, None, None, x, torch.empty_like(x), None, None)
    assert e.value.status == 6  # norm_out is an input


@pytest.mark.parametrize("quant", ["dynamic", "group", "tensor", "static"])
def test_3d_input_quantised_outputs(quant):
    """[B, S, H] inputs: every output keeps the leading dims (the scales drop H, or carry
    the group dim), and the values match the flattened oracle."""
    dtype, P, Bt, S, H = "bf16", 2, 3, 5, 384
    inp = wk.random_case(41, P, Bt * S, H, dtype)
    inp["scale"] = np.array([0.1], np.float32)
    partials = [G.to_dev(p, dtype).view(Bt, S, H) for p in inp["partials"]]
    residual = G.to_dev(inp["residual"], dtype).view(Bt, S, H)
    gamma = G.to_dev(inp["gamma"], dtype)
    scale = torch.tensor([0.1], dtype=torch.float32, device="cuda") if quant == "static" else None
    outs = B.fused_add_rmsnorm(partials, residual, gamma, 1e-6, quant=quant, scale=scale, want_norm_out=True)
    torch.cuda.synchronize()
    q, r = outs[0], outs[1]
    assert q.shape == (Bt, S, H) and r.shape == (Bt, S, H) and outs[-1].shape == (Bt, S, H)
    if quant == "dynamic":
        assert outs[2].shape == (Bt, S)
    if quant == "group":
        assert outs[2].shape == (Bt, S, H // 128)
    if quant == "tensor":
        assert outs[2].shape == (1,)
    gpu = {"quant_out": G.codes_of(q).reshape(-1, H), "new_residual": G.codes_of(r).reshape(-1, H),
           "norm_out": G.codes_of(outs[-1]).reshape(-1, H)}
    if quant in G.DYNAMIC:
        sc = G.codes_of(outs[2])
        gpu["scale_out"] = sc.reshape(-1, H // 128) if quant == "group" else sc.reshape(-1)
    ref = G.run_oracle(inp, dtype, 1e-6, 0.0, quant)
    G.compare(gpu, ref, dtype, quant, inp, tag=f"3-D {quant}")


@pytest.mark.parametrize("quant", ["dynamic", "group", "tensor"])
def test_graph_replay_quantised_modes(quant):
    """Capture of the quantised modes, the three-kernel per-tensor mode included:
    several replays, eager work in between, every replay equal to the eager result."""
    dtype, P, T, H = "bf16", 4, 48, 2048
    inp = wk.random_case(43, P, T, H, dtype)
    partials = [G.to_dev(p, dtype) for p in inp["partials"]]
    residual = G.to_dev(inp["residual"], dtype)
    gamma = G.to_dev(inp["gamma"], dtype)
    eager = B.fused_add_rmsnorm(partials, residual, gamma, 1e-6, quant=quant)
    torch.cuda.synchronize()
    q_g = torch.empty_like(eager[0])
    r_g = torch.empty_like(eager[1])
    s_g = torch.empty_like(eager[2])
    ws_bytes = B.far_workspace_bytes(T, H, quant)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def call():
        B.far_fused_add_rmsnorm(partials, residual, gamma, 1e-6, 0.0, quant, None, None, r_g, q_g, s_g,
                                workspace=ws if ws_bytes else None)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in range(4):
        q_g.view(torch.uint8).zero_()
        r_g.zero_()
        s_g.zero_()
        _ = (residual.float() * 3).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(q_g.view(torch.uint8), eager[0].view(torch.uint8)), f"{quant} replay {i} codes"
        assert torch.equal(r_g.view(torch.int16), eager[1].view(torch.int16)), f"{quant} replay {i} residual"
        assert torch.equal(s_g, eager[2]), f"{quant} replay {i} scales"


@pytest.mark.parametrize("H,variant", [(64, "auto"), (60, "auto"), (60, "generic")])
def test_tensor_scale_many_rows(H, variant):
    """Per-tensor mode over 16400 rows (the scale reduction loops over the row maxima):
    vector rows of whole packs (H = 64) and with a partial pack (H = 60; its codes come
    from the elementwise code pass), and the generic kernel."""
    dtype, P, T = "bf16", 2, 16400
    inp = wk.random_case(29, P, T, H, dtype)
    _say(f"[parity] per-tensor P={P} T={T} H={H} {variant}")
    plan = {"variant": "generic"} if variant == "generic" else None
    gpu = G.run_gpu(inp, dtype, 1e-6, 0.0, "tensor", want_norm=True, plan=plan)
    ref = G.run_oracle(inp, dtype, 1e-6, 0.0, "tensor")
    G.compare(gpu, ref, dtype, "tensor", inp, tag=f"tensor T={T} H={H}")


@pytest.mark.parametrize("dtype,sigma,gamma_mu", [("fp16", 2e-6, 1e-3), ("bf16", 1e-39, 1.0),
                                                  ("fp16", 1e-3, 1e-4)])
@pytest.mark.parametrize("quant", ["none", "dynamic", "static"])
def test_subnormal_storage_values(dtype, sigma, gamma_mu, quant):
    """Inputs, new residuals and normalised outputs in the subnormal range of the
    storage format (fp16 below 2^-14, bf16 below 2^-126), through the vector and the
    generic kernel."""
    P, T, H = 3, 9, 1032
    inp = wk.random_case(31, P, T, H, dtype, partial_sigma=sigma, residual_sigma=sigma,
                         gamma_mu=gamma_mu, gamma_sigma=gamma_mu / 10)
    inp["scale"] = np.float32(1e-6)
    _say(f"[parity] subnormal {dtype} sigma={sigma} gamma={gamma_mu} {quant}")
    ref = G.run_oracle(inp, dtype, 1e-6, 0.0, quant)
    for plan in (None, {"variant": "generic"}):
        gpu = G.run_gpu(inp, dtype, 1e-6, 0.0, quant, want_norm=True, plan=plan)
        stats = G.compare(gpu, ref, dtype, quant, inp, tag=f"subnormal {dtype} {quant} {plan}")
        _say(f"[parity]   {plan}: {stats}")


@pytest.mark.parametrize("H,quant", [(64, "dynamic"), (8, "none"), (8, "group"), (40, "static")])
def test_many_short_rows(H, quant):
    """Very many short rows (large grids; rows of one pack or less than a wave)."""
    dtype, P, T = "bf16", 2, 100_000
    inp = wk.random_case(37, P, T, H, dtype)
    inp["scale"] = np.float32(0.05)
    _say(f"[parity] many short rows P={P} T={T} H={H} {quant}, plan {B.far_plan(T, H, P, torch.bfloat16, quant)}")
    gpu = G.run_gpu(inp, dtype, 1e-6, 0.0, quant, want_norm=True)
    ref = G.run_oracle(inp, dtype, 1e-6, 0.0, quant)
    G.compare(gpu, ref, dtype, quant, inp, tag=f"short rows H={H} {quant}")


@pytest.mark.parametrize("variant", ["auto", "generic"])
def test_static_scale_rewritten_on_device_between_calls(variant):
    """The static scale is read at each launch: a scale that a GPU op rewrites in place,
    in stream order and with no synchronisation, is the one the next call uses (the
    vector kernel reads it through the scalar cache at kernel start)."""
    dtype, P, T, H = "bf16", 4, 24, 2048
    plan = None if variant == "auto" else {"variant": "generic"}
    _say(f"[parity] static scale rewritten between calls, {variant}")
    inp = wk.random_case(47, P, T, H, dtype)
    partials = [G.to_dev(p, dtype) for p in inp["partials"]]
    residual = G.to_dev(inp["residual"], dtype)
    gamma = G.to_dev(inp["gamma"], dtype)
    scale = torch.tensor([0.05], dtype=torch.float32, device="cuda")
    results = []
    for s_host in (0.05, 0.1, 0.0125):
        if s_host != 0.05:
            scale.mul_(s_host / float(results[-1][0]))  # on the device, in stream order
        q, r = B.fused_add_rmsnorm(partials, residual, gamma, 1e-6, quant="static", scale=scale,
                                   plan=plan)
        results.append((s_host, q, r))
    torch.cuda.synchronize()
    assert float(scale.cpu()[0]) == float(np.float32(0.0125))  # the doublings are exact
    for s_host, q, r in results:
        inp["scale"] = np.array([s_host], np.float32)
        ref = G.run_oracle(inp, dtype, 1e-6, 0.0, "static")
        gpu = {"quant_out": G.codes_of(q), "new_residual": G.codes_of(r)}
        G.compare(gpu, ref, dtype, "static", inp, tag=f"static S={s_host} {variant}")


@pytest.mark.parametrize("H", [5120, 5124])
def test_prefill_grids_deal_every_row_once(H):
    """Prefill-sized batches on grids that loop over the rows: a multiple of 8 (the
    kernel then deals the rows XCD by XCD), not a multiple of 8 (hardware order), down to
    8 workgroups, and one row per workgroup. Same team, so every output is bit-identical
    to the automatic plan's, and that plan matches the oracle."""
    dtype, P, T, quant = "bf16", 2, 2048, "dynamic"
    inp = wk.random_case(53, P, T, H, dtype)
    auto = B.far_plan(T, H, P, G.TORCH_DT[dtype], quant)
    _say(f"[parity] prefill grids H={H} auto={auto}")
    base = G.run_gpu(inp, dtype, 1e-6, 0.0, quant)
    rows = np.arange(0, T, 97)  # sampled rows, both trips of each XCD's block
    G.compare(base, G.run_oracle(inp, dtype, 1e-6, 0.0, quant, rows=rows), dtype, quant, inp,
              rows=rows, tag=f"auto H={H}")
    for grid in (8, 1000, 1024, 2048):
        plan = {"variant": "vector", "waves_per_row": auto["waves_per_row"],
                "packs_per_lane": auto["packs_per_lane"], "rows_per_block": 1, "grid_blocks": grid}
        gpu = G.run_gpu(inp, dtype, 1e-6, 0.0, quant, plan=plan)
        for k in base:
            assert np.array_equal(gpu[k], base[k]), (grid, k)
