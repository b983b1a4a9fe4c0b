"""Pins of the oracle's number-format decoders and nibble order (CPU only).

E2M1 against the OCP MX table, E4M3 against torch.float8_e4m3fn for all 256
codes plus the spec's anchors, the low-nibble-first packing on hand-built bytes.
"""
import math
from fractions import Fraction

import numpy as np
import torch

import oracle
from exact_ref import e4m3_values, quantize_block
from golden_io import e2m1_table, e4m3_anchors


def test_e2m1_all_codes_match_ocp_table():
    table = e2m1_table()
    assert sorted(table) == list(range(16))
    for code, val in table.items():
        got = oracle.e2m1_value(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def test_e4m3_all_codes_match_torch_float8_e4m3fn():
    ref = e4m3_values(np.arange(256))
    for code in range(256):
        got = oracle.e4m3_value(code)
        if math.isnan(ref[code]):
            assert math.isnan(got), code
        else:
            assert got == ref[code] and math.copysign(1, got) == math.copysign(1, ref[code]), code


def test_e4m3_anchors():
    for code, val in e4m3_anchors().items():
        got = oracle.e4m3_value(code)
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val, hex(code)
    for e in range(-6, 5):
        assert oracle.e4m3_value((e + 7) << 3) == 2.0 ** e


def test_nibble_order_low_first():
    # One 32-element row where only element 0 (low nibble of byte 0) is 6.0 and
    # element 1 (high nibble) is 0.5: amax = 6 -> element 0 must quantize to 127.
    packed = np.zeros((1, 16), np.uint8)
    packed[0, 0] = 0x17          # low nibble code 7 (6.0), high nibble code 1 (0.5)
    e4m3 = np.full((1, 2), 0x38, np.uint8)
    q, s = oracle.requant_w(packed, e4m3, np.float32(1.0))
    assert q[0, 0] == 127 and q[0, 1] == 11
    assert np.all(q[0, 2:] == 0)


def test_e4m3_scale_index_per_16():
    # Elements 0..15 use scale code 0, elements 16..31 scale code 1.
    packed = np.full((1, 16), 0x22, np.uint8)   # every element code 2 (1.0)
    e4m3 = np.array([[0x38, 0x40]], np.uint8)   # 1.0 and 2.0
    q, s = oracle.requant_w(packed, e4m3, np.float32(1.0))
    vals = [Fraction(1)] * 16 + [Fraction(2)] * 16
    s_ref, q_ref = quantize_block(vals)
    assert list(q[0]) == q_ref
    assert np.all(q[0, 16:] == 127)
    assert s[0, 0] == np.float32(float(s_ref))


def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 16, size=(4, 32), dtype=np.uint16)
    exp = (bits >> 7) & 0xFF
    bits[exp == 0xFF] &= 0x7F7F                  # drop inf/NaN (outside the contract)
    q, s = oracle.requant_a(bits)
    vals = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).float().numpy()
    amax = np.abs(vals).max(axis=1)
    assert np.array_equal(s[:, 0], (amax / np.float32(127.0)).astype(np.float32))
