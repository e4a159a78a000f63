"""Exact brute-force evaluation of the epilogue on tiny inputs (test helper).

Independent of the oracle: formats are decoded with exact rationals straight from
their bit-field definitions, sums are exact (``fractions.Fraction``), the square root
is taken with ``decimal`` at 60 significant digits, and every rounding is a search of
the complete table of finite codes for the nearest value (ties to the even code).
Overflow of IEEE formats follows IEEE 754's rule for round-to-nearest: a magnitude at
least ``max_finite + ulp(max_finite)/2`` becomes infinity.
"""

from __future__ import annotations

import bisect
from decimal import Decimal, localcontext
from fractions import Fraction
from functools import lru_cache

SPECS = {
    # name: (exponent bits, mantissa bits, bias, IEEE specials)
    "bf16": (8, 7, 127, True),
    "fp16": (5, 10, 15, True),
    "e4m3fn": (4, 3, 7, False),
    "f32": (8, 23, 127, True),
}


def exact_value(code: int, name: str):
    """Exact value of a code: a Fraction, or the strings 'inf', '-inf', 'nan'."""
    eb, mb, bias, ieee = SPECS[name]
    sign = (code >> (eb + mb)) & 1
    e = (code >> mb) & ((1 << eb) - 1)
    m = code & ((1 << mb) - 1)
    top = (1 << eb) - 1
    if ieee and e == top:
        if m:
            return "nan"
        return "-inf" if sign else "inf"
    if not ieee and e == top and m == (1 << mb) - 1:
        return "nan"
    if e == 0:
        v = Fraction(m) * Fraction(2) ** (1 - bias - mb)
    else:
        v = Fraction((1 << mb) + m) * Fraction(2) ** (e - bias - mb)
    return -v if sign else v


@lru_cache(maxsize=None)
def _positive_table(name: str):
    """Sorted (value, code) of every finite non-negative code."""
    eb, mb, bias, ieee = SPECS[name]
    out = []
    for code in range(1 << (eb + mb)):
        v = exact_value(code, name)
        if isinstance(v, Fraction):
            out.append((v, code))
    out.sort()
    return [v for v, _ in out], [c for _, c in out]


def nearest_code(value, name: str, negative_zero: bool = False, saturate: bool = False) -> int:
    """Code of the value of ``name`` nearest to ``value`` (a Fraction), ties to the
    even code. ``saturate`` clamps to the largest finite magnitude first."""
    eb, mb, bias, ieee = SPECS[name]
    sign_bit = 1 << (eb + mb)
    neg = value < 0 or (value == 0 and negative_zero)
    mag = abs(value)
    vals, codes = _positive_table(name)
    vmax = vals[-1]
    if saturate and mag > vmax:
        mag = vmax
    if ieee:
        ulp_at_max = vals[-1] - vals[-2]
        if mag >= vmax + ulp_at_max / 2:
            inf_code = ((1 << eb) - 1) << mb
            return inf_code | (sign_bit if neg else 0)
    i = bisect.bisect_left(vals, mag)
    if i < len(vals) and vals[i] == mag:
        c = codes[i]
    else:
        lo_v, lo_c = vals[i - 1], codes[i - 1]
        hi_v, hi_c = vals[i], codes[i]
        d_lo, d_hi = mag - lo_v, hi_v - mag
        if d_lo < d_hi:
            c = lo_c
        elif d_hi < d_lo:
            c = hi_c
        else:
            c = lo_c if lo_c % 2 == 0 else hi_c
    return c | (sign_bit if neg else 0)


def nearest_f32(value: Fraction) -> Fraction:
    """Nearest binary32 value (finite inputs well inside the range), ties to even,
    by binary search over the ordered positive bit patterns."""
    neg = value < 0
    mag = abs(value)
    lo, hi = 0, 0x7F7FFFFF
    while hi - lo > 1:  # invariant: value(lo) <= mag < value(hi) or mag beyond
        mid = (lo + hi) // 2
        if exact_value(mid, "f32") <= mag:
            lo = mid
        else:
            hi = mid
    v_lo, v_hi = exact_value(lo, "f32"), exact_value(hi, "f32")
    if mag - v_lo < v_hi - mag:
        r = v_lo
    elif v_hi - mag < mag - v_lo:
        r = v_hi
    else:
        r = v_lo if lo % 2 == 0 else v_hi
    return -r if neg else r


def _frac(d: Decimal) -> Fraction:
    return Fraction(d)


def _scale_of(amax):
    return nearest_f32(amax / 448) if amax > 0 else Fraction(1)


def fused_add_rmsnorm(partials, residual, gamma, dtype, eps, weight_bias, quant, scale=None,
                      group=128):
    """Brute-force epilogue on nested lists of codes. Rows must be finite.

    Returns dict with lists: new_residual, norm_out (codes), y (Fractions, 60-digit
    accurate), and quant_out / scale_out (Fractions) when ``quant`` is set
    ("static", "dynamic" per token, "group" per ``group`` elements of a row, "tensor").
    """
    P = len(partials)
    T = len(residual) if residual is not None else len(partials[0])
    H = len(gamma)
    eps_v = exact_value(_f32_code(eps), "f32")
    wb_v = exact_value(_f32_code(weight_bias), "f32")
    g = [exact_value(int(c), dtype) for c in gamma]
    out = {"new_residual": [], "norm_out": [], "y": [], "quant_out": [], "scale_out": []}
    for t in range(T):
        s = []
        for h in range(H):
            acc = Fraction(0)
            for p in range(P):
                acc += exact_value(int(partials[p][t][h]), dtype)
            if residual is not None:
                acc += exact_value(int(residual[t][h]), dtype)
            s.append(acc)
        nr = [nearest_code(v, dtype) for v in s]
        x = [exact_value(c, dtype) for c in nr]
        ms = sum(v * v for v in x) / H
        with localcontext() as ctx:
            ctx.prec = 60
            denom = (Decimal(ms.numerator) / Decimal(ms.denominator)
                     + Decimal(eps_v.numerator) / Decimal(eps_v.denominator)).sqrt()
            r = _frac(Decimal(1) / denom)
        y = [x[h] * r * (wb_v + g[h]) for h in range(H)]
        out["new_residual"].append(nr)
        out["y"].append(y)
        out["norm_out"].append([nearest_code(v, dtype) for v in y])
        if quant == "static":
            S = exact_value(_f32_code(scale), "f32")
            out["quant_out"].append([nearest_code(v / S, "e4m3fn", saturate=True) for v in y])
        elif quant == "dynamic":
            sc = _scale_of(max(abs(v) for v in y))
            out["scale_out"].append(sc)
            out["quant_out"].append([nearest_code(v / sc, "e4m3fn", saturate=True) for v in y])
        elif quant == "group":
            scs = [_scale_of(max(abs(v) for v in y[g:g + group])) for g in range(0, H, group)]
            out["scale_out"].append(scs)
            out["quant_out"].append([nearest_code(y[h] / scs[h // group], "e4m3fn", saturate=True)
                                     for h in range(H)])
    if quant == "tensor":
        sc = _scale_of(max(abs(v) for row in out["y"] for v in row))
        out["scale_out"] = [sc]
        out["quant_out"] = [[nearest_code(v / sc, "e4m3fn", saturate=True) for v in row]
                            for row in out["y"]]
    return out


def _f32_code(x: float) -> int:
    import struct
    return struct.unpack("<I", struct.pack("<f", x))[0]
