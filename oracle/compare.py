"""Pass/fail rule for BF16 outputs against the FP64 oracle -- TEST INFRASTRUCTURE ONLY.

An output passes when either

  (i)  |out - y| <= max(4e-3 * |y|, ulp(y))          relative error 4e-3 or one
       BF16 ulp of the FP64 evaluation over the same quantized values; or
  (ii) |out - y| <= B + ulp(|y| + B),  B = (K/32 + 2) * 2^-24 * T,

where T = sum over blocks of |a_s * w_s * P| and ulp(x) = 2^(floor(log2|x|) - 7)
(BF16 keeps 8 significant bits; below 2^-126 the spacing stays 2^-133).
Clause (ii) is the first-order worst-case error of an FP32 sum of K/32 rescaled
block terms taken in any order (one rounding for the scale product, one for the
product with P, K/32 - 1 for the additions), plus the final BF16 rounding.  It
only matters under cancellation, where |y| is far below T.

The W4A16 decode GEMV (T = sum of |x * w| over k) takes `terms` from
w4a16_terms(K): its two kernels sum differently.
"""
from dataclasses import dataclass

import numpy as np


def bf16_bits_to_f64(bits):
    b = np.ascontiguousarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_ulp(x):
    """Spacing of BF16 numbers at |x| (0 where x == 0)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(ax > 0, np.ldexp(1.0, (e - 7).astype(np.int64)), 0.0)


@dataclass
class CheckResult:
    count: int
    failures: int
    needed_ii: int
    max_rel_err: float
    max_ulp_err: float
    first_failure: tuple

    @property
    def ok(self) -> bool:
        return self.failures == 0

    def __str__(self):
        return (f"{self.count} outputs, {self.failures} failures, {self.needed_ii} passed only by the "
                f"FP32 sum bound, max rel err {self.max_rel_err:.3e}, max ulp err {self.max_ulp_err:.2f}"
                + (f", first failure at {self.first_failure}" if self.failures else ""))


def w4a16_terms(k):
    """FP32 sum terms of the W4A16 GEMV's first-order error bound.

    K a multiple of 256 (streamed kernel): per 16-element scale block the 16
    exact products x * e2m1 are summed in FP32 in one matrix-core operation
    (at most 15 roundings, each bounded by the block's magnitude sum), the block
    sum is scaled by its E4M3 scale and added to the wave's accumulator (one
    rounding per block: K/16 over the row), up to 16 wave partials are added
    (15) and scale_2 multiplies once (1): K/16 + 31.
    Other K (register-decode kernel): the exact products x * (e2m1 * s16) are
    accumulated in FP32 inside the matrix-core operations over the whole K
    range of a wave, then the wave partials and scale_2: K + 16."""
    return k / 16 + 31 if k % 256 == 0 else k + 16


def check_bf16(out_bits, y64, t, k, terms=None) -> CheckResult:
    """Apply the pass rule element-wise; out_bits are raw BF16 uint16 values.
    `terms` is the number of FP32 sum terms of the bound (default K/32)."""
    out = bf16_bits_to_f64(out_bits).reshape(np.shape(y64))
    y = np.asarray(y64, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    finite = np.isfinite(out)
    err = np.abs(np.where(finite, out, 0.0) - y)
    ay = np.abs(y)
    ulp_y = bf16_ulp(ay)
    ok_i = finite & (err <= np.maximum(4e-3 * ay, ulp_y))
    bound = ((k / 32 if terms is None else terms) + 2) * 2.0 ** -24 * t
    ok_ii = finite & (err <= bound + bf16_ulp(ay + bound))
    ok = ok_i | ok_ii
    nz = ok_i & (ay > 0)
    max_rel = float(np.max(err[nz] / ay[nz])) if nz.any() else 0.0
    with np.errstate(divide="ignore", invalid="ignore"):
        ulps = np.where(ulp_y > 0, err / np.where(ulp_y > 0, ulp_y, 1.0), 0.0)
    max_ulp = float(np.max(ulps[ok_i])) if ok_i.any() else 0.0
    bad = np.argwhere(~ok)
    first = tuple(int(i) for i in bad[0]) if bad.size else ()
    return CheckResult(int(ok.size), int((~ok).sum()), int((ok_ii & ~ok_i).sum()), max_rel, max_ulp, first)
