"""The comparison helper's acceptance rules, on hand-made code arrays (no GPU)."""

import numpy as np
import pytest

import compare as cmp


def bf16(values):
    import torch
    t = torch.tensor(values, dtype=torch.float64).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_one_ulp_passes_two_fail():
    ref = bf16([1.0, -3.5, 0.0])
    gpu = ref.copy()
    gpu[0] += 1                                      # one ulp above 1.0
    st = cmp.check_storage(gpu, ref, "bf16", "x")
    assert st["max_ulp"] == 1
    gpu[1] += 2                                      # two ulps away from -3.5
    with pytest.raises(AssertionError, match="beyond 1 ulp"):
        cmp.check_storage(gpu, ref, "bf16", "x")


def test_zero_needs_zero():
    ref = bf16([0.0])
    gpu = ref.copy()
    gpu[0] = 1                                       # smallest subnormal, one ulp from 0
    with pytest.raises(AssertionError):
        cmp.check_storage(gpu, ref, "bf16", "x")
    gpu[0] = 0x8000                                  # -0 matches +0
    cmp.check_storage(gpu, ref, "bf16", "x")


def test_cancellation_allowance_follows_the_fp32_bound():
    # terms of magnitude ~2^10 cancel to a result near 2^-8: the fp32 sum of 9 terms may
    # be off by up to 8 * 2^-24 * sum|terms| = 8 * 2^-24 * 9 * 2^10 ~ 2^-8.8, several
    # bf16 ulps of the small result (ulp 2^-15 at 2^-8)
    ref = bf16([2.0 ** -8])
    abs_terms = np.array([9 * 2.0 ** 10])
    gpu = ref.copy()
    gpu[0] += 40                                     # 40 ulps = 40 * 2^-15 ~ 2^-9.7
    st = cmp.check_storage(gpu, ref, "bf16", "x", abs_terms, n_adds=8)
    assert st["cancellation_excused"] == 1
    # with one addition the bound is 2^-24 * sum|terms| + ulp ~ 2^-11.8: 40 ulps fail
    with pytest.raises(AssertionError):
        cmp.check_storage(gpu, ref, "bf16", "x", abs_terms, n_adds=1)
    # without the terms there is no allowance at all
    with pytest.raises(AssertionError):
        cmp.check_storage(gpu, ref, "bf16", "x")


def test_ulp_of_formats():
    assert cmp.ulp_of(np.array([1.0]), "bf16")[0] == 2.0 ** -7
    assert cmp.ulp_of(np.array([1.0]), "fp16")[0] == 2.0 ** -10
    assert cmp.ulp_of(np.array([0.0]), "fp16")[0] == 2.0 ** -24    # subnormal spacing
    assert cmp.ulp_of(np.array([-6.0e4]), "fp16")[0] == 32.0


def test_fp8_steps():
    ref = np.array([0x38, 0xB8, 0x00, 0x7F], np.uint8)   # 1.0, -1.0, 0, NaN
    gpu = np.array([0x39, 0xB7, 0x80, 0xFF], np.uint8)   # +1 step, -1 step, -0, NaN
    assert cmp.check_fp8(gpu, ref, "q")["max_step"] == 1
    gpu[0] = 0x3A
    with pytest.raises(AssertionError):
        cmp.check_fp8(gpu, ref, "q")
