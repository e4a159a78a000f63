"""Properties of the GPU outputs that hold at any size, checked on whole full-size
batches without the oracle: the fp8 codes dequantise to the normalised output within one
e4m3 step, every nonzero row of a dynamic per-token quantisation uses the code of
magnitude 448, and per-group scales make every nonzero group reach 448 too."""

import sys

import numpy as np
import pytest
import torch

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


def _e4m3_step(v: torch.Tensor) -> torch.Tensor:
    """Spacing of the OCP e4m3fn grid at |v| (normals: 2^(e - 3), subnormals: 2^-9)."""
    a = v.abs().clamp(min=2.0 ** -6)
    return torch.exp2(torch.floor(torch.log2(a)) - 3)


def _bf16_ulp(v: torch.Tensor) -> torch.Tensor:
    a = v.abs().clamp(min=2.0 ** -126)
    return torch.exp2(torch.floor(torch.log2(a)) - 7)


def _device_inputs(inp, dtype):
    return ([G.to_dev(p, dtype) for p in inp["partials"]], G.to_dev(inp["residual"], dtype),
            G.to_dev(inp["gamma"], dtype))


@pytest.mark.parametrize("quant", ["dynamic", "group"])
def test_dynamic_codes_dequantise_to_norm_out_c4(quant):
    wl = wk.WORKLOADS["c4"]
    _say(f"[self] c4 full size, {quant} scales")
    inp = wk.make_inputs(wl)
    parts, res, gamma = _device_inputs(inp, wl.dtype)
    q, new_res, scale, norm = B.fused_add_rmsnorm(parts, res, gamma, wl.eps, wl.weight_bias,
                                                  quant=quant, want_norm_out=True)
    torch.cuda.synchronize()
    code_val = q.float()                                   # e4m3 code values
    y = norm.float()                                       # norm_out, rounded to bf16
    if quant == "dynamic":
        sc = scale.view(-1, 1)
        groups = code_val.view(wl.T, 1, wl.H)
    else:
        sc = scale.view(wl.T, -1).repeat_interleave(B.FAR_FP8_GROUP, dim=1)[:, :wl.H]
        groups = code_val.view(wl.T, -1, B.FAR_FP8_GROUP)
    deq = code_val * sc
    # |dequant - y| <= 1.5 steps of the code grid (RNE half step, plus one step of slack
    # between the fused fp32 path and y) + the bf16 rounding of norm_out
    bound = 1.5 * _e4m3_step(code_val) * sc + _bf16_ulp(y)
    err = (deq - y).abs()
    assert torch.all(err <= bound), f"worst excess {(err - bound).max().item()}"
    # the largest |y| of every nonzero row / group lands on the code of magnitude 448
    amax_code = groups.abs().amax(-1)
    nonzero = y.view(groups.shape).abs().amax(-1) > 0
    assert torch.all(amax_code[nonzero] == 448.0)
    _say(f"[self] c4 {quant}: max err / bound {(err / bound).max().item():.3f}")


def test_static_codes_dequantise_to_norm_out_c3():
    wl = wk.WORKLOADS["c3"]
    _say("[self] c3 full size, static scale")
    inp = wk.make_inputs(wl)
    parts, res, gamma = _device_inputs(inp, wl.dtype)
    S = torch.tensor(inp["scale"], dtype=torch.float32, device="cuda").view(1)
    q, new_res, norm = B.fused_add_rmsnorm(parts, res, gamma, wl.eps, wl.weight_bias,
                                           quant="static", scale=S, want_norm_out=True)
    torch.cuda.synchronize()
    code_val = q.float()
    y = norm.float()
    deq = code_val * S
    inside = (y / S).abs() < 448.0
    bound = 1.5 * _e4m3_step(code_val) * S + _bf16_ulp(y)
    err = (deq - y).abs()
    assert torch.all(err[inside] <= bound[inside])
    # outside the range the code saturates at +-448 with the sign of y
    out = ~inside & (y.abs() > 0)
    assert torch.all(code_val[out].abs() == 448.0)
    assert torch.all(torch.sign(code_val[out]) == torch.sign(y[out]))
    _say(f"[self] c3: {int(out.sum())} saturated codes, max err / bound {(err[inside] / bound[inside]).max().item():.3f}")


def test_norm_out_is_rmsnorm_of_new_residual_c4():
    """The normalised output is RMSNorm of the rounded new residual the kernel returned
    (recomputed in float64 on the GPU), within one bf16 ulp."""
    wl = wk.WORKLOADS["c4"]
    inp = wk.make_inputs(wl)
    parts, res, gamma = _device_inputs(inp, wl.dtype)
    norm, new_res = B.fused_add_rmsnorm(parts, res, gamma, wl.eps, wl.weight_bias)
    torch.cuda.synchronize()
    x = new_res.double()
    r = torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + wl.eps)
    y = x * r * (wl.weight_bias + gamma.double())
    err = (norm.double() - y).abs()
    assert torch.all(err <= _bf16_ulp(y.float()).double()), float((err / _bf16_ulp(y.float()).double()).max())
