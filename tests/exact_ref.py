"""Exact-rational restatement of the quantizer, used to pin the oracle.

It shares nothing with the oracle: values are exact ``Fraction``s, rounding to
binary32 and to integers is done with integer arithmetic written here, and the
E4M3 / BF16 decodes come from torch's own dtype conversions.  A mistake in the
oracle's float code path (a reciprocal instead of a divide, an FMA, flushed
subnormals, a wrong tie rule, a wrong clamp) shows up as a disagreement.
"""
from fractions import Fraction

import numpy as np
import torch

F32_MIN_EXP = -126      # smallest normal exponent
F32_MANT = 23           # stored mantissa bits


def f32_round(x: Fraction) -> Fraction:
    """Nearest binary32 value to x (ties to even, subnormals kept, no overflow allowed)."""
    if x == 0:
        return Fraction(0)
    neg = x < 0
    num, den = abs(x.numerator), x.denominator
    e = num.bit_length() - den.bit_length()          # 2^e <= |x| < 2^(e+1) after the fix-up
    if (num << max(0, -e)) < (den << max(0, e)):
        e -= 1
    qe = max(e, F32_MIN_EXP) - F32_MANT              # exponent of the unit in the last place
    if qe >= 0:
        n_, d_ = num, den << qe
    else:
        n_, d_ = num << (-qe), den
    q, r = divmod(n_, d_)
    if 2 * r > d_ or (2 * r == d_ and (q & 1)):
        q += 1
    out = Fraction(q) * (Fraction(2) ** qe)
    if out >= Fraction(2) ** 128:
        raise OverflowError("binary32 overflow")
    return -out if neg else out


def rne_int(x: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even."""
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and (fl & 1)):
        fl += 1
    return fl


def quantize_block(values):
    """values: exact rationals of one 32-element block -> (scale, [q])."""
    amax = max(abs(v) for v in values)
    s = f32_round(amax / 127)
    if s == 0:
        return Fraction(0), [0] * len(values)
    qs = []
    for v in values:
        q = rne_int(f32_round(v / s))
        qs.append(max(-127, min(127, q)))
    return s, qs


def bf16_values(bits):
    """Exact values of raw BF16 bit patterns, via torch's BF16 -> FP32 conversion."""
    t = torch.from_numpy(np.asarray(bits, dtype=np.uint16).astype(np.int16).copy()).view(torch.bfloat16)
    return [Fraction(float(x)) for x in t.float().numpy().ravel()]


def e4m3_values(codes):
    """Exact values of E4M3 codes via torch.float8_e4m3fn (NaN codes give nan floats)."""
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy()).view(torch.float8_e4m3fn)
    return [float(x) for x in t.float().numpy().ravel()]


def f32_bits(x: Fraction) -> int:
    return int(np.array([float(x)], dtype=np.float32).view(np.uint32)[0])
