"""far_fused_add_rmsnorm_noalloc (the entry point that allocates nothing) against
far_fused_add_rmsnorm_ex with a caller-provided workspace, through the C ABI (needs a
GPU). Two calls in a row share the library's scratch: the second, smaller one must not
see what the first left there."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import compare as cmp
import gpu_util as G
from residual_add_rmsnorm_fp32_amd import binding as B
from residual_add_rmsnorm_fp32_amd import workloads as wk

pytestmark = pytest.mark.gpu

QUANT = {"none": 0, "dynamic": 2, "tensor": 4}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _outputs(T, H, dtype, quant):
    dev = torch.device("cuda")
    tdt = G.TORCH_DT[dtype]
    # guard bands: one extra element after every output, filled with a marker
    out = {"residual_out": torch.full((T * H + 1,), 7.0, dtype=tdt, device=dev)}
    if quant == "none":
        out["norm_out"] = torch.full((T * H + 1,), 7.0, dtype=tdt, device=dev)
    else:
        out["quant_out"] = torch.full((T * H + 1,), 0x5A, dtype=torch.uint8, device=dev)
        n = T if quant == "dynamic" else 1
        out["scale_out"] = torch.full((n + 1,), 7.0, dtype=torch.float32, device=dev)
    return out


def _call(entry, inp, dtype, quant, eps, wb, out, workspace=None):
    """One call through the C ABI; returns the status."""
    lib = B.load_library()
    partials = [G.to_dev(p, dtype) for p in inp["partials"]]
    residual = G.to_dev(inp["residual"], dtype)
    gamma = G.to_dev(inp["gamma"], dtype)
    P, T, H = len(partials), inp["residual"].shape[0], inp["gamma"].shape[0]
    arr = (ctypes.c_void_p * P)(*[p.data_ptr() for p in partials])
    ptr = lambda k: out[k].data_ptr() if k in out else None
    stream = torch.cuda.current_stream().cuda_stream
    args = [arr, P, residual.data_ptr(), gamma.data_ptr(), T, H, 0 if dtype == "bf16" else 1,
            eps, wb, QUANT[quant], None, ptr("norm_out"), ptr("residual_out"), ptr("quant_out"),
            ptr("scale_out"), stream]
    if entry == "noalloc":
        st = lib.far_fused_add_rmsnorm_noalloc(*args)
    else:
        ws = workspace.data_ptr() if workspace is not None else None
        nbytes = workspace.numel() if workspace is not None else 0
        st = lib.far_fused_add_rmsnorm_ex(*args, None, ws, nbytes)
    torch.cuda.synchronize()
    # keep the inputs alive until the kernels are done
    del partials, residual, gamma
    return st


def _codes(out, T, H):
    """Codes of each output without its guard element, which must still hold its marker."""
    res = {}
    for k, v in out.items():
        marker = 0x5A if k == "quant_out" else 7.0
        assert v[-1].item() == marker, f"{k}: guard element overwritten"
        res[k] = G.codes_of(v[:-1])
    return res


def _case(seed, P, T, H, dtype, quant):
    _say(f"[no-alloc] seed={seed} P={P} T={T} H={H} {dtype} {quant}")
    inp = wk.random_case(seed, P, T, H, dtype)
    eps, wb = 1e-6, (1.0 if dtype == "fp16" else 0.0)
    out_n = _outputs(T, H, dtype, quant)
    assert _call("noalloc", inp, dtype, quant, eps, wb, out_n) == B.FAR_OK
    out_e = _outputs(T, H, dtype, quant)
    ws_bytes = B.far_workspace_bytes(T, H, quant)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes else None
    assert _call("ex", inp, dtype, quant, eps, wb, out_e, ws) == B.FAR_OK
    got, want = _codes(out_n, T, H), _codes(out_e, T, H)
    # the existing entry point's outputs as the reference, to the parity tolerances ...
    cmp.check_storage(got["residual_out"].reshape(T, H), want["residual_out"].reshape(T, H),
                      dtype, "residual_out")
    if quant == "none":
        cmp.check_storage(got["norm_out"].reshape(T, H), want["norm_out"].reshape(T, H), dtype,
                          "norm_out")
    else:
        cmp.check_fp8(got["quant_out"], want["quant_out"], "quant_out")
        cmp.check_scales(got["scale_out"], want["scale_out"], "scale_out")
    # ... and, as both run the same kernels, bit for bit
    for k in got:
        assert np.array_equal(got[k], want[k]), k
    # and the oracle agrees with both
    ref = G.run_oracle(inp, dtype, eps, wb, quant)
    if quant == "tensor":
        cmp.check_fp8(got["quant_out"].reshape(T, H), ref["quant_out"], "quant_out vs oracle")
        cmp.check_scales(got["scale_out"], ref["scale_out"], "scale_out vs oracle")
    cmp.check_storage(got["residual_out"].reshape(T, H), ref["new_residual"], dtype,
                      "residual_out vs oracle")


def test_noalloc_matches_workspace_entry_point_two_calls():
    # per-tensor mode (the one that uses the scratch): a large call, then a smaller one
    _case(11, 2, 3000, 5120, "bf16", "tensor")
    _case(12, 3, 77, 2056, "fp16", "tensor")
    # rows ending in a partial pack (H = 1001, elementwise code pass) with the scratch,
    # then rows of whole packs again
    _case(13, 2, 50, 1001, "bf16", "tensor")
    _case(14, 1, 5, 64, "bf16", "tensor")


def test_noalloc_at_the_scratch_limit_and_beyond():
    T = B.FAR_NOALLOC_SCRATCH_BYTES // 8  # 262144 rows: the whole scratch
    _case(15, 1, T, 16, "bf16", "tensor")
    inp = wk.random_case(16, 1, 4, 16, "bf16")
    # one row more than the scratch holds: an error, nothing launched (outputs untouched)
    big = {"partials": np.zeros((1, T + 1, 16), np.uint16), "residual": np.zeros((T + 1, 16), np.uint16),
           "gamma": inp["gamma"]}
    out = _outputs(T + 1, 16, "bf16", "tensor")
    assert _call("noalloc", big, "bf16", "tensor", 1e-6, 0.0, out) == 10  # FAR_ERR_SCRATCH_LIMIT
    assert int(G.codes_of(out["quant_out"]).max()) == 0x5A and int(G.codes_of(out["quant_out"]).min()) == 0x5A


def test_noalloc_other_modes_match():
    _case(17, 8, 80, 4096, "bf16", "none")
    _case(18, 2, 300, 5120, "bf16", "dynamic")
