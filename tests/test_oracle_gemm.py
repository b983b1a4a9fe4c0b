"""Pins of the oracle's block partials and FP64 reference output (CPU only).

References: numpy integer einsum for the block partials, a float64 matmul over
dequantized operands (a second formulation of the same sum), exact integer
arithmetic for power-of-two scales, and the hand-worked two-block example A6.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from block_scaled_precision_requant_amd import inputs
from exact_ref import bf16_values
from golden_io import quant_blocks


def _rand_q(rng, shape):
    return rng.integers(-127, 128, size=shape, dtype=np.int64).astype(np.int8)


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (5, 7, 96), (33, 17, 256)])
def test_block_partials_match_numpy_einsum(m, n, k):
    rng = np.random.default_rng(m * 1000 + n)
    a = _rand_q(rng, (m, k))
    w = _rand_q(rng, (n, k))
    p = oracle.block_partials(a, w)
    ref = np.einsum("mbj,nbj->mnb", a.astype(np.int64).reshape(m, k // 32, 32),
                    w.astype(np.int64).reshape(n, k // 32, 32))
    assert np.array_equal(p, ref)


def test_block_partial_extremes():
    a = np.full((1, 64), 127, np.int8)
    w = np.full((1, 64), -127, np.int8)
    assert np.all(oracle.block_partials(a, w) == -32 * 127 * 127)


@pytest.mark.parametrize("m,n,k", [(3, 4, 64), (5, 3, 96), (16, 9, 512)])
def test_gemm_ref_matches_dequantized_matmul(m, n, k):
    rng = np.random.default_rng(k + m)
    a = _rand_q(rng, (m, k))
    w = _rand_q(rng, (n, k))
    a_s = rng.uniform(1e-3, 1e-1, size=(m, k // 32)).astype(np.float32)
    w_s = rng.uniform(1e-4, 1e-2, size=(n, k // 32)).astype(np.float32)
    y, t = oracle.gemm_ref(a, w, a_s, w_s)
    ad = a.astype(np.float64) * np.repeat(a_s.astype(np.float64), 32, axis=1)
    wd = w.astype(np.float64) * np.repeat(w_s.astype(np.float64), 32, axis=1)
    ref = ad @ wd.T
    mag = np.abs(ad) @ np.abs(wd).T
    assert np.all(np.abs(y - ref) <= 1e-13 * mag + 1e-300)
    assert np.all(t <= mag * (1 + 1e-13)) and np.all(t >= np.abs(y) * (1 - 1e-13))


def test_gemm_ref_exact_power_of_two_case():
    rng = np.random.default_rng(3)
    m, n, k = 4, 6, 128
    a = rng.integers(-15, 16, size=(m, k)).astype(np.int8)
    w = rng.integers(-15, 16, size=(n, k)).astype(np.int8)
    a_e = rng.integers(-8, 3, size=(m, k // 32))
    w_e = rng.integers(-8, 3, size=(n, k // 32))
    a_s = np.ldexp(1.0, a_e).astype(np.float32)
    w_s = np.ldexp(1.0, w_e).astype(np.float32)
    y, _ = oracle.gemm_ref(a, w, a_s, w_s)
    for i in range(m):
        for j in range(n):
            exact = Fraction(0)
            for b in range(k // 32):
                p = sum(int(a[i, 32 * b + u]) * int(w[j, 32 * b + u]) for u in range(32))
                exact += Fraction(2) ** int(a_e[i, b] + w_e[j, b]) * p
            assert Fraction(y[i, j]) == exact


def test_gemm_ref_transpose_symmetry_and_row_subset():
    rng = np.random.default_rng(5)
    a = _rand_q(rng, (7, 96))
    w = _rand_q(rng, (5, 96))
    a_s = rng.uniform(0.01, 1, size=(7, 3)).astype(np.float32)
    w_s = rng.uniform(0.01, 1, size=(5, 3)).astype(np.float32)
    y, t = oracle.gemm_ref(a, w, a_s, w_s)
    yt, tt = oracle.gemm_ref(w, a, w_s, a_s)
    assert np.array_equal(y, yt.T) and np.array_equal(t, tt.T)
    ys, ts = oracle.gemm_ref(a, w, a_s, w_s, rows=np.array([6, 0, 3]))
    assert np.array_equal(ys, y[[6, 0, 3]]) and np.array_equal(ts, t[[6, 0, 3]])


def test_zero_scale_blocks_contribute_nothing():
    rng = np.random.default_rng(9)
    a = _rand_q(rng, (3, 96))
    w = _rand_q(rng, (4, 96))
    a_s = rng.uniform(0.01, 1, size=(3, 3)).astype(np.float32)
    w_s = rng.uniform(0.01, 1, size=(4, 3)).astype(np.float32)
    a_s[:, 1] = 0.0
    y, _ = oracle.gemm_ref(a, w, a_s, w_s)
    keep = np.r_[0:32, 64:96]
    y2, _ = oracle.gemm_ref(a[:, keep], w[:, keep], a_s[:, [0, 2]], w_s[:, [0, 2]])
    assert np.array_equal(y, y2)


def _a6_inputs():
    g = quant_blocks()
    a = np.zeros(64, np.float32)
    a1 = [float(x) for x in g["A1"]["values"]]
    a2 = [float(x) for x in g["A2"]["values"]]
    a[: len(a1)] = a1
    a[32: 32 + len(a2)] = a2
    a_bits = inputs.f32_to_bf16_bits(a)[None, :]
    packed = np.array([[int(x, 16) for x in g["W1"]["packed_hex"]] +
                       [int(x, 16) for x in g["W2"]["packed_hex"]]], np.uint8)
    e4m3 = np.array([[int(x, 16) for x in g["W1"]["e4m3_hex"]] +
                     [int(x, 16) for x in g["W2"]["e4m3_hex"]]], np.uint8)
    return a_bits, packed, e4m3, g


def test_golden_a6_two_block_gemm():
    a_bits, packed, e4m3, g = _a6_inputs()
    # W1 and W2 as one row need one scale2: W1 was worked with scale2 = 1, W2 with
    # fl32(1/448).  Requantize each half with its own scale2 and join them.
    q1, s1 = oracle.requant_w(packed[:, :16], e4m3[:, :2], np.float32(1.0))
    s2v = np.array([int(g["W2"]["scale2_bits"][0], 16)], np.uint32).view(np.float32)[0]
    q2, s2 = oracle.requant_w(packed[:, 16:], e4m3[:, 2:], s2v)
    assert list(q2[0, :16]) == [int(x) for x in g["W2"]["q_first_half"]]
    w_i8 = np.concatenate([q1, q2], axis=1)
    w_s = np.concatenate([s1, s2], axis=1)
    a_i8, a_s = oracle.requant_a(a_bits)
    exp_q = g["A2"]["q_except_ties"]
    for i, tok in enumerate(exp_q):
        if tok != "*":
            assert a_i8[0, 32 + i] == int(tok)
    p = oracle.block_partials(a_i8, w_i8)
    assert list(p[0, 0]) == [int(x) for x in g["A6"]["P"]]
    y, t = oracle.gemm_ref(a_i8, w_i8, a_s, w_s)
    exact = sum(Fraction(float(a_s[0, b])) * Fraction(float(w_s[0, b])) * int(p[0, 0, b]) for b in range(2))
    assert abs(Fraction(y[0, 0]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)
    from oracle.compare import check_bf16
    good = np.array([[int(g["A6"]["out_bf16"][0], 16)]], np.uint16)
    assert check_bf16(good, y, t, 64).ok
    assert check_bf16(good - 1, y, t, 64).ok          # -740 is one BF16 ulp (4) away: allowed
    assert not check_bf16(good - 2, y, t, 64).ok      # -736 is 6.9 away: beyond 1 ulp and 4e-3


def test_gemm_ref_on_tiny_workload_matches_dequantized_matmul():
    proj = inputs.workload("tiny").projections[0]
    wp, we = proj.weight()
    a = proj.activations()
    w_i8, w_s = oracle.requant_w(wp, we, proj.scale2)
    a_i8, a_s = oracle.requant_a(a)
    y, t = oracle.gemm_ref(a_i8, w_i8, a_s, w_s)
    ad = a_i8.astype(np.float64) * np.repeat(a_s.astype(np.float64), 32, axis=1)
    wd = w_i8.astype(np.float64) * np.repeat(w_s.astype(np.float64), 32, axis=1)
    assert np.all(np.abs(y - ad @ wd.T) <= 1e-13 * (np.abs(ad) @ np.abs(wd).T))
    # and the quantized product approximates the unquantized one (a sanity bound only)
    af = np.asarray(bf16_values(a.ravel()), dtype=np.float64).reshape(a.shape)
    assert np.corrcoef((af @ wd.T).ravel(), y.ravel())[0, 1] > 0.999
