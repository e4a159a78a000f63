"""Element-by-element comparison of the HIP outputs with the oracle's (test helper).

Acceptance (the tolerances the method is held to):
* new_residual and norm_out: within 1 ulp of the oracle's rounded value (distance
  between codes on the ordered integer line, +0 and -0 both at 0), and max |rel err|
  <= 8e-3 over non-zero oracle values; an oracle zero needs a GPU zero (either sign); NaN where the oracle has NaN, inf where it has
  the same inf.
* fp32 cancellation in new_residual: the method sums the P + 1 terms of an element in
  fp32 (one rounding per addition), the oracle exactly. Recursive summation of
  n terms in binary32 is off by at most (n - 1) * 2^-24 * sum |terms| (to first order),
  and rounding that sum to the storage type adds at most one ulp of the result. Where
  the terms cancel, that error can exceed one ulp of the small result: such an element
  passes if |err| <= n_adds * 2^-24 * sum |terms| + ulp(oracle value), and is counted
  (``cancellation_excused``). The parity tests of the named workloads require that
  count to be zero.
* fp8 codes: within +-1 e4m3 step on the ordered integer line (+0 = -0; 448 and
  -448 are the ends); NaN codes where the oracle has NaN.
* per-token scales: relative error <= 1e-6.
"""

from __future__ import annotations

import numpy as np
import torch

REL_TOL = 8e-3
SCALE_REL_TOL = 1e-6

_SPEC = {"bf16": (16, 0x7F80, 0x007F), "fp16": (16, 0x7C00, 0x03FF), "e4m3fn": (8, 0x78, 0x07)}


def ordered(codes: np.ndarray, fmt: str) -> np.ndarray:
    bits = _SPEC[fmt][0]
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> (bits - 1)) & 1
    mag = c & ((1 << (bits - 1)) - 1)
    return np.where(sign == 1, -mag, mag)


def is_nan(codes: np.ndarray, fmt: str) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    bits = _SPEC[fmt][0]
    mag = c & ((1 << (bits - 1)) - 1)
    if fmt == "e4m3fn":
        return mag == 0x7F
    emask, mmask = _SPEC[fmt][1], _SPEC[fmt][2]
    return ((mag & emask) == emask) & ((mag & mmask) != 0)


def decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    c = np.asarray(codes)
    if fmt == "fp16":
        return c.astype(np.uint16).view(np.float16).astype(np.float64)
    if fmt == "bf16":
        return torch.from_numpy(c.astype(np.uint16).view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    if fmt == "e4m3fn":
        return torch.from_numpy(c.astype(np.uint8).copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    raise ValueError(fmt)


def ulp_of(values: np.ndarray, fmt: str) -> np.ndarray:
    """Spacing of the storage format at each (finite) value: 2^(e - mbits), with e held
    at the smallest normal exponent for subnormals."""
    mbits, emin = {"bf16": (7, -126), "fp16": (10, -14)}[fmt]
    a = np.where(np.isfinite(values), np.abs(values), 1.0)
    _, k = np.frexp(a)
    e = np.where(a == 0.0, emin, np.maximum(k - 1, emin))
    return np.ldexp(1.0, (e - mbits).astype(np.int32))


def check_storage(gpu: np.ndarray, ref: np.ndarray, fmt: str, what: str,
                  abs_terms: np.ndarray | None = None, n_adds: int = 0) -> dict:
    """Assert the storage-dtype tolerance; returns statistics. ``abs_terms`` (sum of
    |terms| per element) and ``n_adds`` (fp32 additions per element) enable the fp32
    cancellation allowance for new_residual."""
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    gn, rn = is_nan(gpu, fmt), is_nan(ref, fmt)
    bad_nan = gn != rn
    assert not bad_nan.any(), f"{what}: NaN pattern differs at {np.argwhere(bad_nan)[:5].tolist()}"
    ok = ~rn
    d = np.abs(ordered(gpu, fmt) - ordered(ref, fmt))
    gv, rv = decode(gpu, fmt), decode(ref, fmt)
    finite = np.isfinite(rv) & ok
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(finite & (rv != 0), np.abs(gv - rv) / np.abs(rv), 0.0)
    fail = ok & (d > 1)
    # an oracle value of zero must be matched by a zero (either sign), not by the
    # smallest subnormal one ulp away
    fail |= finite & (rv == 0) & (gv != 0)
    inf_mismatch = ok & ~np.isfinite(rv) & (gv != rv)
    fail |= inf_mismatch
    fail |= finite & (rel > REL_TOL)
    cancel_ok = 0
    if abs_terms is not None and fail.any():
        err = np.abs(gv - rv)
        bound = n_adds * 2.0 ** -24 * np.asarray(abs_terms) + ulp_of(rv, fmt)
        excused = fail & finite & (err <= bound)
        cancel_ok = int(excused.sum())
        fail &= ~excused
    n_fail = int(fail.sum())
    if n_fail:
        idx = np.argwhere(fail)[:5]
        samples = [(tuple(i), int(gpu[tuple(i)]), int(ref[tuple(i)]), float(gv[tuple(i)]), float(rv[tuple(i)]))
                   for i in idx]
        raise AssertionError(f"{what}: {n_fail} elements beyond 1 ulp / rel {REL_TOL}; "
                             f"(index, gpu code, oracle code, gpu value, oracle value): {samples}")
    return {"max_ulp": int(d[ok].max()) if ok.any() else 0,
            "ulp1_frac": float((d[ok] == 1).mean()) if ok.any() else 0.0,
            "max_rel": float(rel.max()) if rel.size else 0.0,
            "cancellation_excused": cancel_ok}


def check_fp8(gpu: np.ndarray, ref: np.ndarray, what: str) -> dict:
    gpu = np.asarray(gpu).astype(np.uint8)
    ref = np.asarray(ref).astype(np.uint8)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    gn, rn = is_nan(gpu, "e4m3fn"), is_nan(ref, "e4m3fn")
    assert not (gn != rn).any(), f"{what}: NaN pattern differs"
    d = np.abs(ordered(gpu, "e4m3fn") - ordered(ref, "e4m3fn"))
    d = np.where(rn, 0, d)
    n_fail = int((d > 1).sum())
    if n_fail:
        idx = np.argwhere(d > 1)[:5]
        raise AssertionError(f"{what}: {n_fail} codes beyond +-1 step, e.g. "
                             f"{[(tuple(i), int(gpu[tuple(i)]), int(ref[tuple(i)])) for i in idx]}")
    return {"max_step": int(d.max()) if d.size else 0, "step1_frac": float((d == 1).mean()) if d.size else 0.0}


def check_scales(gpu: np.ndarray, ref: np.ndarray, what: str) -> dict:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape
    nan_r = np.isnan(ref)
    assert np.array_equal(np.isnan(gpu), nan_r), f"{what}: NaN pattern differs"
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(nan_r, 0.0, np.abs(gpu - ref) / np.abs(ref))
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= SCALE_REL_TOL, f"{what}: scale rel err {worst:.3e} > {SCALE_REL_TOL}"
    return {"max_rel": worst}
