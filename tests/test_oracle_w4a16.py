"""Pins of the oracle's W4A16 decode GEMV reference (CPU only).

* a second formulation: the NVFP4 weight dequantized to float64 through the
  OCP E2M1 table (tests/golden/e2m1_ocp.txt) and torch's float8_e4m3fn decode,
  activations through torch's bfloat16 decode, then a float64 matmul -- agrees
  to rounding-order level;
* exact special case: small integer activations, power-of-two E4M3 scales and a
  power-of-two scale_2 make every partial sum an exact binary64 value, so the
  reference must equal integer arithmetic exactly;
* t >= |y|, and y flips sign with the activations (linearity).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_requant_amd import inputs
from golden_io import e2m1_table


def _dequant64(packed, e4m3, scale2):
    tab = e2m1_table()
    table = np.array([tab[c] for c in range(16)], np.float64)
    n, half = packed.shape
    k = 2 * half
    codes = np.empty((n, k), np.int64)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    s16 = torch.from_numpy(e4m3.copy()).view(torch.float8_e4m3fn).double().numpy()
    return table[codes] * np.repeat(s16, 16, axis=1) * float(np.float32(scale2))


def _bf16_to_f64(bits):
    return torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("m,n,k", [(1, 64, 512), (3, 50, 160), (8, 33, 1024)])
def test_matches_float64_matmul_of_dequantized_weight(m, n, k):
    rng = np.random.default_rng(m * 100 + n + k)
    x = inputs.bf16_normal(rng, m, k)
    wp, we = inputs.nvfp4_weight(rng, n, k, -4, 2)
    we[:, ::3] = rng.integers(0x01, 0x7F, size=we[:, ::3].shape)     # general codes, not only powers of two
    y, t = oracle.w4a16_ref(x, wp, we, inputs.SCALE2_1_448)
    ref = _bf16_to_f64(x) @ _dequant64(wp, we, inputs.SCALE2_1_448).T
    assert np.all(np.abs(y - ref) <= 1e-13 * t + 1e-300)
    assert np.all(t >= np.abs(y))


def test_exact_integer_case():
    rng = np.random.default_rng(5)
    m, n, k = 4, 20, 256
    x = inputs.f32_to_bf16_bits(rng.integers(-20, 21, size=(m, k)).astype(np.float32))
    wp = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    e = rng.integers(-3, 3, size=(n, k // 16))
    we = ((e + 7) << 3).astype(np.uint8)
    scale2 = np.float32(2.0 ** -6)
    y, _ = oracle.w4a16_ref(x, wp, we, scale2)
    # integer arithmetic: 2 * e2m1 and 8 * s16 are integers (s16 >= 2^-3), so
    # y = scale2 * sum(x * (2 * e2m1) * (8 * s16)) / 16
    table_half = [0, 1, 2, 3, 4, 6, 8, 12]                         # e2m1 magnitude * 2
    xi = _bf16_to_f64(x).astype(np.int64)
    for i in range(m):
        for j in range(n):
            acc = 0
            for c in range(k):
                byte = int(wp[j, c // 2])
                code = (byte >> 4) if c & 1 else (byte & 15)
                mag = table_half[code & 7] * (-1 if code & 8 else 1)
                acc += int(xi[i, c]) * mag * (2 ** (int(e[j, c // 16]) + 3))
            assert y[i, j] == float(Fraction(acc, 16) * Fraction(1, 2 ** 6))


def test_linearity_in_activations():
    rng = np.random.default_rng(8)
    x = inputs.bf16_normal(rng, 2, 128)
    wp, we = inputs.nvfp4_weight(rng, 9, 128, -4, 2)
    y1, t1 = oracle.w4a16_ref(x, wp, we, inputs.SCALE2_1_448)
    y2, t2 = oracle.w4a16_ref(x ^ np.uint16(0x8000), wp, we, inputs.SCALE2_1_448)
    assert np.array_equal(y1, -y2) and np.array_equal(t1, t2)


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.w4a16_ref(np.zeros((1, 48), np.uint16), np.zeros((1, 24), np.uint8),
                         np.zeros((1, 3), np.uint8), 1.0)
