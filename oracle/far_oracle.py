"""CPU oracle for the fused "sum of partials + residual add + RMSNorm (+ fp8 quant)" epilogue.

TEST INFRASTRUCTURE. Only the tests, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path (the HIP
library under ``residual_add_rmsnorm_fp32_amd/`` and its Python binding) never does, and
this module imports nothing from it.

The oracle is the plain definition, evaluated in binary64 (numpy float64) with every
input decoded to its exact value. It shares no code with the HIP path.

What is computed, per token row t (sources are the pages' titles and sections):

* Page "vllm.models.common.ops.fused_allreduce_rms_norm", function
  ``fused_allreduce_rms_norm``: the fused op returns ``(normed_output, new_residual)``
  and equals ``norm(all_reduce(hidden_states), residual)`` where ``hidden_states`` is
  one rank's partial output of a row-parallel linear layer. On one GPU the all-reduce
  becomes the sum of P partial tensors held locally. The same source passes
  ``fp32_acc=True`` (the sum is accumulated wide, rounded once), ``rms_eps`` from the
  norm's ``variance_epsilon`` and a ``weight_bias`` argument (0 for a plain RMSNorm, 1
  for Gemma-style norms), so the
  effective weight is ``weight_bias + gamma``.
* Page "vllm.compilation.fusion", ``kFp8StaticTensorSym`` / ``kFp8DynamicTokenSym`` and
  the patterns ``FusedAddRMSNormStaticQuantPattern`` / ``FusedAddRMSNormDynamicQuantPattern``:
  the optional epilogue quantises the normalised row to fp8, symmetric, either with one
  static fp32 scale per tensor or with one dynamic scale per token that is also
  returned.

Readings taken where the pages are silent (each is listed in the design notes):

* RMSNorm is ``x / sqrt(mean_h(x^2) + eps) * w`` with the mean over H elements and eps
  added to the mean square (``variance_epsilon``, the norm being the ordinary
  RMSNorm).
* ``new_residual`` is rounded once to the storage dtype; the rounded tensor is what is
  normalised (it is the tensor the op returns and feeds to ``norm``). The other reading
  is available with ``normalize="unrounded"``.
* The static scale S is a dequantisation multiplier: ``q = E4M3(y / S)``.
* The dynamic per-token scale is ``RNE_f32(max_h |y| / 448)``; an all-zero row gets
  scale 1.0. Codes are ``E4M3(y / scale)`` with the stored fp32 scale.
* Per-group scales (page "vllm.distributed.device_communicators.aiter_custom_all_reduce",
  build_supports_per_group_quant, names a per-group AR + RMSNorm + quant kernel but not
  its group shape): groups of 128 consecutive elements along H (the last group of a row
  may be shorter), one scale per (token, group), computed like the per-token scale over
  the group. Per-tensor dynamic scale (page "vllm.compilation.fusion",
  kFp8DynamicTensorSym): the same over the whole [T, H] tensor.
* fp8 is OCP e4m3fn (largest finite 448, no infinities). Values are clamped to
  [-448, 448] before rounding; NaN maps to code 0x7F with the sign kept.
* All roundings are IEEE round-to-nearest-even, subnormals included; bf16/fp16
  overflow goes to +-inf.

Parity is pinned (not self-referentially) by the ``-m "not gpu"`` tests: exhaustive
format checks against numpy/torch conversions, exact brute force on tiny inputs,
closed forms (unit RMS, single-nonzero rows), hand-derived fixtures and invariants.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

QUANT_NONE = 0
QUANT_FP8_STATIC_TENSOR = 1
QUANT_FP8_DYNAMIC_TOKEN = 2
QUANT_FP8_DYNAMIC_GROUP = 3
QUANT_FP8_DYNAMIC_TENSOR = 4

FP8_GROUP = 128  # elements per group along H for the per-group scales

E4M3_MAX = 448.0


@dataclass(frozen=True)
class Format:
    """A binary floating-point storage format: sign, ``ebits`` exponent bits with
    bias ``bias``, ``mbits`` stored mantissa bits."""

    name: str
    ebits: int
    mbits: int
    bias: int
    ieee_specials: bool  # top exponent field = inf/NaN (IEEE style)
    nan_code: int        # canonical NaN magnitude bits
    storage: type        # numpy integer type of one code

    @property
    def sign_bit(self) -> int:
        return 1 << (self.ebits + self.mbits)

    @property
    def emin(self) -> int:
        """Exponent of the smallest normal value."""
        return 1 - self.bias

    @property
    def max_finite(self) -> float:
        top = (1 << self.ebits) - 1
        if self.ieee_specials:
            # top exponent field reserved: largest normal has field top-1, all-ones mantissa
            return float(np.ldexp(2.0 - 2.0 ** -self.mbits, top - 1 - self.bias))
        # OCP e4m3fn: field top is normal except the all-ones mantissa (NaN)
        return float(np.ldexp(2.0 - 2.0 ** (1 - self.mbits), top - self.bias))


BF16 = Format("bf16", 8, 7, 127, True, 0x7FC0, np.uint16)
FP16 = Format("fp16", 5, 10, 15, True, 0x7E00, np.uint16)
E4M3FN = Format("e4m3fn", 4, 3, 7, False, 0x7F, np.uint8)

FORMATS = {"bf16": BF16, "fp16": FP16, "e4m3fn": E4M3FN}


def decode(codes, fmt: Format) -> np.ndarray:
    """Exact value of every code of ``fmt`` as float64 (binary64 holds them all)."""
    b = np.asarray(codes).astype(np.int64)
    sign = (b >> (fmt.ebits + fmt.mbits)) & 1
    e = (b >> fmt.mbits) & ((1 << fmt.ebits) - 1)
    m = b & ((1 << fmt.mbits) - 1)
    mf = m.astype(np.float64)
    normal = np.ldexp(mf + float(1 << fmt.mbits), (e - fmt.bias - fmt.mbits).astype(np.int32))
    subnormal = np.ldexp(mf, np.int32(fmt.emin - fmt.mbits))
    val = np.where(e == 0, subnormal, normal)
    top = (1 << fmt.ebits) - 1
    if fmt.ieee_specials:
        val = np.where((e == top) & (m == 0), np.inf, val)
        val = np.where((e == top) & (m != 0), np.nan, val)
    else:
        val = np.where((e == top) & (m == (1 << fmt.mbits) - 1), np.nan, val)
    return np.where(sign == 1, -val, val)


def round_to(x, fmt: Format, saturate: bool = False) -> np.ndarray:
    """Round float64 values to the nearest code of ``fmt``, ties to even.

    ``saturate`` clamps to the largest finite magnitude first (used for e4m3fn);
    otherwise magnitudes that round beyond it become infinity (IEEE formats).
    """
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    sign = np.signbit(x)
    a = np.abs(np.where(nan, 0.0, x))
    if saturate:
        a = np.minimum(a, fmt.max_finite)
    finite = np.isfinite(a)
    a_f = np.where(finite, a, 0.0)

    # Exponent of the leading bit, held at emin for the subnormal range; the grid
    # spacing there is 2**(e - mbits). Dividing by a power of two is exact, and rint
    # is round-half-even, so n * quantum is the correctly rounded magnitude.
    _, k = np.frexp(a_f)
    e = np.maximum(k - 1, fmt.emin)
    quantum = np.ldexp(1.0, (e - fmt.mbits).astype(np.int32))
    n = np.rint(a_f / quantum)
    mag = n * quantum
    overflow = ~finite | (mag > fmt.max_finite)

    # Encode the (finite, representable) magnitude.
    is_sub = mag < 2.0 ** fmt.emin
    _, k2 = np.frexp(np.where(is_sub, 1.0, mag))
    E = k2 - 1
    m_norm = mag / np.ldexp(1.0, (E - fmt.mbits).astype(np.int32)) - float(1 << fmt.mbits)
    m_sub = mag / 2.0 ** (fmt.emin - fmt.mbits)
    field_e = np.where(is_sub, 0, E + fmt.bias).astype(np.int64)
    field_m = np.where(is_sub, m_sub, m_norm).astype(np.int64)
    code = (field_e << fmt.mbits) | field_m

    top = (1 << fmt.ebits) - 1
    if fmt.ieee_specials:
        code = np.where(overflow, top << fmt.mbits, code)
    code = np.where(nan, fmt.nan_code, code)
    code = np.where(sign, code | fmt.sign_bit, code)
    return code.astype(fmt.storage)


def round_f32(x) -> np.ndarray:
    """Round float64 to the nearest binary32 value (numpy's cast is IEEE RNE)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def quantize_e4m3(v) -> np.ndarray:
    """OCP e4m3fn code of v: NaN -> 0x7F (sign kept), clamp to +-448, RNE."""
    return round_to(v, E4M3FN, saturate=True)


def sum_partials(partials, residual, fmt: Format) -> np.ndarray:
    """Sum of the P partial rows plus the residual, in binary64.

    Page "vllm.models.common.ops.fused_allreduce_rms_norm": the new residual is
    ``all_reduce(hidden_states) + residual``; on one GPU the all-reduce is the sum of the
    P partial tensors. ``residual=None`` is the form without a residual input.
    """
    s = np.zeros(np.shape(partials[0]), dtype=np.float64)
    for p in range(len(partials)):
        s = s + decode(partials[p], fmt)
    if residual is not None:
        s = s + decode(residual, fmt)
    return s


def rms_norm(x, gamma, eps, weight_bias) -> np.ndarray:
    """Unrounded RMSNorm of each row of x (float64), weight = weight_bias + gamma.

    ``eps`` and ``weight_bias`` are the fp32 values the caller passes, widened exactly.
    """
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1]
    mean_sq = np.sum(x * x, axis=-1, keepdims=True) / h
    r = 1.0 / np.sqrt(mean_sq + float(np.float32(eps)))
    w = float(np.float32(weight_bias)) + np.asarray(gamma, dtype=np.float64)
    return x * r * w


def scale_from_amax(amax) -> np.ndarray:
    """fp32 scale ``amax / 448`` (1.0 where amax is 0), as float64; NaN stays NaN."""
    amax = np.asarray(amax, dtype=np.float64)
    scale = round_f32(amax / E4M3_MAX)
    scale = np.where(amax == 0.0, 1.0, scale)
    return np.where(np.isnan(amax), np.nan, scale)


def dynamic_token_scale(y) -> np.ndarray:
    """Per-row fp32 scale ``max|y| / 448`` (1.0 for an all-zero row), as float64."""
    return scale_from_amax(np.max(np.abs(y), axis=-1))


def dynamic_group_scale(y, group: int = FP8_GROUP) -> np.ndarray:
    """[T, ceil(H / group)] fp32 scales, each over ``group`` consecutive elements of a
    row (the last group may be shorter), as float64."""
    H = y.shape[-1]
    starts = np.arange(0, H, group)
    amax = np.stack([np.max(np.abs(y[..., g:g + group]), axis=-1) for g in starts], axis=-1)
    return scale_from_amax(amax)


def fused_add_rmsnorm(partials, residual, gamma, dtype: str, eps: float,
                      weight_bias: float = 0.0, quant_mode: int = QUANT_NONE,
                      scale=None, normalize: str = "rounded") -> dict:
    """The whole epilogue on host arrays of raw storage codes.

    partials: sequence of P arrays (or one [P, T, H] array) of uint16 codes;
    residual: [T, H] uint16 codes, or None for the form without a residual;
    gamma: [H] uint16 codes; dtype: "bf16" or "fp16"; scale: the static fp32 scale.

    Returns a dict of numpy arrays: ``new_residual`` and ``norm_out`` (codes of dtype),
    ``y`` (the unrounded normalised rows, float64), and with quantisation ``quant_out``
    (uint8 e4m3fn codes) plus, for the dynamic mode, ``scale_out`` (float32).
    """
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        return _fused_add_rmsnorm(partials, residual, gamma, dtype, eps, weight_bias,
                                  quant_mode, scale, normalize)


def _fused_add_rmsnorm(partials, residual, gamma, dtype, eps, weight_bias, quant_mode,
                       scale, normalize):
    # IEEE semantics throughout: an overflowed residual gives inf, 0 * inf gives NaN.
    fmt = FORMATS[dtype]
    s = sum_partials(partials, residual, fmt)
    new_residual = round_to(s, fmt)
    if normalize == "rounded":
        x = decode(new_residual, fmt)
    elif normalize == "unrounded":
        x = s
    else:
        raise ValueError(normalize)
    y = rms_norm(x, decode(gamma, fmt), eps, weight_bias)
    out = {"new_residual": new_residual, "y": y, "norm_out": round_to(y, fmt)}
    if quant_mode == QUANT_FP8_STATIC_TENSOR:
        s_val = float(np.float32(np.asarray(scale).reshape(-1)[0]))
        out["quant_out"] = quantize_e4m3(y / s_val)
    elif quant_mode == QUANT_FP8_DYNAMIC_TOKEN:
        tok_scale = dynamic_token_scale(y)
        out["quant_out"] = quantize_e4m3(y / tok_scale[..., None])
        out["scale_out"] = tok_scale.astype(np.float32)
    elif quant_mode == QUANT_FP8_DYNAMIC_GROUP:
        grp_scale = dynamic_group_scale(y)
        per_elem = np.repeat(grp_scale, FP8_GROUP, axis=-1)[..., :y.shape[-1]]
        out["quant_out"] = quantize_e4m3(y / per_elem)
        out["scale_out"] = grp_scale.astype(np.float32)
    elif quant_mode == QUANT_FP8_DYNAMIC_TENSOR:
        ten_scale = scale_from_amax(np.max(np.abs(y)) if y.size else 0.0)
        out["quant_out"] = quantize_e4m3(y / ten_scale)
        out["scale_out"] = np.asarray(ten_scale, dtype=np.float32).reshape(1)
    elif quant_mode != QUANT_NONE:
        raise ValueError(f"unknown quant mode {quant_mode}")
    return out
