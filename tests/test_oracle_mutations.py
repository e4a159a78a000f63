"""Plant a mistake in a copy of the oracle and require the pins to catch it.

Each mutation is a textual edit of oracle/far_oracle.py, applied to an in-memory copy
(the file on disk is never touched). A pin suite that lets a plausible mistake through
is not pinning the oracle. CPU only.
"""

import os
import sys
import types

import pytest

import pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "far_oracle.py")

# (name, text in the oracle, replacement)
MUTATIONS = [
    ("residual dropped", "        s = s + decode(residual, fmt)", "        s = s"),
    ("last partial skipped", "for p in range(len(partials)):", "for p in range(len(partials) - 1):"),
    ("mean over H-1", "axis=-1, keepdims=True) / h", "axis=-1, keepdims=True) / (h - 1)"),
    ("eps outside the root", "r = 1.0 / np.sqrt(mean_sq + float(np.float32(eps)))",
     "r = 1.0 / (np.sqrt(mean_sq) + float(np.float32(eps)))"),
    ("no square root", "r = 1.0 / np.sqrt(mean_sq + float(np.float32(eps)))",
     "r = 1.0 / (mean_sq + float(np.float32(eps)))"),
    ("abs instead of square", "np.sum(x * x, axis=-1", "np.sum(np.abs(x), axis=-1"),
    ("weight_bias ignored", "w = float(np.float32(weight_bias)) + np.asarray(gamma",
     "w = 0.0 + np.asarray(gamma"),
    ("gamma reversed", "np.asarray(gamma, dtype=np.float64)", "np.asarray(gamma, dtype=np.float64)[::-1]"),
    ("unrounded residual normalised", "        x = decode(new_residual, fmt)\n", "        x = s\n"),
    ("static scale multiplies", "quantize_e4m3(y / s_val)", "quantize_e4m3(y * s_val)"),
    ("amax without abs", "scale_from_amax(np.max(np.abs(y), axis=-1))", "scale_from_amax(np.max(y, axis=-1))"),
    ("zero row not special", "scale = np.where(amax == 0.0, 1.0, scale)", "scale = scale"),
    ("fp8 max 240 (fnuz)", "E4M3_MAX = 448.0", "E4M3_MAX = 240.0"),
    ("scale not rounded to fp32", "scale = round_f32(amax / E4M3_MAX)", "scale = amax / E4M3_MAX"),
    ("ties away from zero", "n = np.rint(a_f / quantum)", "n = np.floor(a_f / quantum + 0.5)"),
    ("truncation", "n = np.rint(a_f / quantum)", "n = np.floor(a_f / quantum)"),
    ("no subnormal clamp", "e = np.maximum(k - 1, fmt.emin)", "e = k - 1"),
    ("no fp8 clamp", "        a = np.minimum(a, fmt.max_finite)\n", "        a = a\n"),
    ("exponent bias off by one", "(e - fmt.bias - fmt.mbits).astype(np.int32)",
     "(e - fmt.bias - fmt.mbits + 1).astype(np.int32)"),
    ("sign dropped in decode", "return np.where(sign == 1, -val, val)", "return val"),
    ("sign dropped in rounding", "code = np.where(sign, code | fmt.sign_bit, code)", "code = code"),
    ("no overflow to inf", "code = np.where(overflow, top << fmt.mbits, code)", "code = code"),
    ("eps rounded away", "float(np.float32(eps))", "0.0"),
    ("group of 64", "FP8_GROUP = 128", "FP8_GROUP = 64"),
    ("ragged last group dropped", "starts = np.arange(0, H, group)", "starts = np.arange(0, H - group + 1, group)"),
    ("group max without abs", "np.max(np.abs(y[..., g:g + group]), axis=-1)", "np.max(y[..., g:g + group], axis=-1)"),
    ("tensor max without abs", "scale_from_amax(np.max(np.abs(y)) if y.size else 0.0)",
     "scale_from_amax(np.max(y) if y.size else 0.0)"),
    ("tensor scale per row", "scale_from_amax(np.max(np.abs(y)) if y.size else 0.0)",
     "scale_from_amax(np.max(np.abs(y), axis=-1, keepdims=True))"),
]

_ORDER = [pins.check_goldens, pins.check_format_facts, pins.check_round_trip,
          pins.check_overflow_and_saturation, pins.check_single_nonzero, pins.check_unit_rms,
          pins.check_invariants, pins.check_quant_invariants, pins.check_torch_rmsnorm,
          pins.check_p1_is_plain_fused_add_rmsnorm, pins.check_decode_all_codes,
          pins.check_midpoints, pins.check_against_library_rounding, pins.check_bruteforce_tiny,
          pins.check_dynamic_scale_ties, pins.check_bruteforce_group_and_tensor,
          pins.check_group_and_tensor_invariants]


def _mutant(old, new):
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    name = "far_oracle_mutant"
    mod = types.ModuleType(name)
    mod.__dict__["__file__"] = ORACLE_SRC
    sys.modules[name] = mod          # dataclasses look their module up here
    try:
        exec(compile(src.replace(old, new), name, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


def _first_failure(mod):
    for check in _ORDER:
        try:
            check(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            return f"{check.__name__}: {type(e).__name__}: {str(e)[:80]}"
    return None


def test_order_covers_all_checks():
    assert set(_ORDER) == set(pins.ALL_CHECKS)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    caught = _first_failure(_mutant(old, new))
    assert caught is not None, f"planted mistake '{name}' passes every pin"
