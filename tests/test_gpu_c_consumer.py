"""The library from plain C: run the example program (C ABI + HIP runtime only, no
Python, no torch) and compare what it prints with the CPU oracle on the same inputs."""

import json
import os
import subprocess

import numpy as np
import pytest

import compare as cmp
from oracle import far_oracle as orc

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "residual_add_rmsnorm_fp32_amd", "examples", "far_c_consumer")


def _bf16(v: np.ndarray) -> np.ndarray:
    # the example's values have at most 8 significant bits: truncation is exact
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_c_consumer_matches_oracle():
    if not os.path.exists(BIN):
        pytest.fail("far_c_consumer was not built (run __graft_entry__.build())")
    print("[c-consumer] running", BIN, flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    out = {}
    for line in res.stdout.splitlines():
        out.update(json.loads(line))
    P, T, H = out["P"], out["T"], out["H"]
    assert out["missing_scale_out_status"] == 5          # FAR_ERR_BAD_QUANT_ARGS
    t = np.arange(T)[:, None]
    h = np.arange(H)[None, :]
    partials = np.stack([_bf16(((7 * t + 3 * h + 5 * p) % 17 - 8) / 8.0) for p in range(P)])
    residual = _bf16(((11 * t + h) % 13 - 6) / 4.0)
    gamma = _bf16(1.0 + ((np.arange(H) % 9) - 4) / 16.0)
    ref = orc.fused_add_rmsnorm(partials, residual, gamma, "bf16", 1e-6, 0.0,
                                quant_mode=orc.QUANT_FP8_DYNAMIC_TOKEN)
    cmp.check_storage(np.array(out["new_residual"], np.uint16).reshape(T, H), ref["new_residual"],
                      "bf16", "C new_residual")
    cmp.check_fp8(np.array(out["quant_out"], np.uint8).reshape(T, H), ref["quant_out"], "C quant_out")
    cmp.check_scales(np.array(out["scale_out"], np.float32), ref["scale_out"], "C scale_out")
