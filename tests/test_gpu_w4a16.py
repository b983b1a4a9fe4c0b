"""GPU parity of the W4A16 decode GEMV (BF16 x NVFP4, no int8 requant) against
the oracle's FP64 reference, under the pass rule with each kernel's FP32 bound
(w4a16_terms: K/16 + 31 terms for the streamed kernel, K + 16 otherwise),
plus an exact power-of-two case that must be bit-equal."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_requant_amd import bsr, inputs
from gpu_util import DEV, gpu_w4a16, host, say, to_dev
from oracle.compare import check_bf16, w4a16_terms

pytestmark = pytest.mark.gpu


def _check(name, out, y, t, k):
    res = check_bf16(out, y, t, k, terms=w4a16_terms(k))
    say(f"{name}: {res}")
    assert res.ok, f"{name}: {res}"


def _weight(rng, n, k, general=True):
    wp, we = inputs.nvfp4_weight(rng, n, k, -4, 2)
    if general:                                      # any finite E4M3 code, negatives and zeros too
        codes = rng.integers(0, 0x7F, size=we.shape).astype(np.uint8)
        codes |= (rng.random(we.shape) < 0.2).astype(np.uint8) << 7
        mask = rng.random(we.shape) < 0.5
        we = np.where(mask, codes, we).astype(np.uint8)
    return wp, we


# K % 256 == 0 -> the streamed kernel (the last three cases: wide grids, the
# last column tile ragged); other K -> the register-decode kernel, per-step
# 2-byte scale loads, and K % 128 != 0 leaves a partial last super-step.
@pytest.mark.parametrize("m,n,k", [(1, 333, 256), (2, 70, 2048), (8, 129, 4096), (3, 333, 1056),
                                   (5, 40, 96), (7, 16, 4128), (4, 1, 512), (8, 300, 14336),
                                   (16, 600, 4096), (12, 300, 14336), (9, 70, 1056),
                                   (4, 8193, 256), (8, 8200, 512), (16, 8200, 1024)])
def test_random_shapes(m, n, k):
    rng = np.random.default_rng(m * 7919 + n * 31 + k)
    x = inputs.bf16_normal(rng, m, k)
    wp, we = _weight(rng, n, k)
    y, t = oracle.w4a16_ref(x, wp, we, inputs.SCALE2_1_448)
    out = host(gpu_w4a16(x, wp, we, inputs.SCALE2_1_448))
    _check(f"w4a16 {m}x{n}x{k}", out, y, t, k)


# Register-decode shapes whose largest fitting staging pass is odd (3, 5, 7
# super-steps): the launch plan rounds it down to an instantiated length
# inside the 160 KB LDS (rounding up once asked for 165-200 KB and failed).
@pytest.mark.parametrize("m,n,k", [(12, 4096, 6016), (7, 4096, 9856), (5, 4096, 13696)])
def test_register_decode_odd_pass_shapes(m, n, k):
    say(f"w4a16 odd-pass plan m={m} n={n} k={k}")
    rng = np.random.default_rng(m * 131 + k)
    x = inputs.bf16_normal(rng, m, k)
    wp, we = _weight(rng, n, k)
    y, t = oracle.w4a16_ref(x, wp, we, inputs.SCALE2_1_448)
    out = host(gpu_w4a16(x, wp, we, inputs.SCALE2_1_448))
    _check(f"w4a16 {m}x{n}x{k}", out, y, t, k)


@pytest.mark.parametrize("proj", inputs.workload("decode").projections, ids=lambda p: p.name)
def test_decode_workload_full(proj):
    wp, we = proj.weight()
    x = proj.activations()
    y, t = oracle.w4a16_ref(x, wp, we, proj.scale2)
    out = host(gpu_w4a16(x, wp, we, proj.scale2))
    _check(proj.name, out, y, t, proj.k)


def test_exact_power_of_two_bit_equal():
    # small integer activations, power-of-two scales: every FP32 partial sum is exact
    rng = np.random.default_rng(12)
    m, n, k = 6, 200, 1024
    x = inputs.f32_to_bf16_bits(rng.integers(-20, 21, size=(m, k)).astype(np.float32))
    wp = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    we = ((rng.integers(-3, 3, size=(n, k // 16)) + 7) << 3).astype(np.uint8)
    scale2 = np.float32(2.0 ** -6)
    y, _ = oracle.w4a16_ref(x, wp, we, scale2)
    exp_bits = inputs.f32_to_bf16_bits(y.astype(np.float32))
    out = host(gpu_w4a16(x, wp, we, scale2))
    assert np.array_equal(out, exp_bits), f"{np.sum(out != exp_bits)} mismatches"


# Every finite E4M3 scale code -- signs, zeros, subnormals, non-powers of two
# up to 448 -- with every E2M1 code, through both kernels (K = 2048 streamed,
# decoding the scale with the hardware conversion; K = 1056 register decode).
@pytest.mark.parametrize("k", [2048, 1056])
def test_all_finite_scale_codes(k):
    rng = np.random.default_rng(k)
    m, n = 5, 200
    x = inputs.bf16_normal(rng, m, k)
    wp = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    we = finite[rng.integers(0, finite.size, size=(n, k // 16))]
    we.flat[:finite.size] = finite  # each code at least once
    y, t = oracle.w4a16_ref(x, wp, we, inputs.SCALE2_1_448)
    out = host(gpu_w4a16(x, wp, we, inputs.SCALE2_1_448))
    _check(f"w4a16 all scale codes k={k}", out, y, t, k)


def test_rows_independent_of_m():
    rng = np.random.default_rng(4)
    k, n = 2048, 97
    x = inputs.bf16_normal(rng, 8, k)
    wp, we = _weight(rng, n, k)
    full = host(gpu_w4a16(x, wp, we, inputs.SCALE2_1_448))
    for m in (1, 3, 5):
        part = host(gpu_w4a16(x[:m].copy(), wp, we, inputs.SCALE2_1_448))
        assert np.array_equal(part, full[:m])


def test_errors_launch_nothing():
    L = bsr.lib()
    x = torch.zeros((9, 256), dtype=torch.int16, device=DEV)
    wp = torch.zeros((4, 128), dtype=torch.uint8, device=DEV)
    we = torch.zeros((4, 16), dtype=torch.uint8, device=DEV)
    out = torch.full((9, 4), 3, dtype=torch.int16, device=DEV)
    args = lambda m, k, e=we.data_ptr(): (x.data_ptr(), wp.data_ptr(), e, 1.0, out.data_ptr(), m, 4, k, None)
    assert L.w4a16_gemv(*args(17, 256)) == bsr.BSR_EINVAL         # m > 16
    assert L.w4a16_gemv(*args(1, 48)) == bsr.BSR_EINVAL           # k
    assert L.w4a16_gemv(*args(1, 256, we.data_ptr() + 2)) == bsr.BSR_EALIGN
    assert L.w4a16_gemv(x.data_ptr(), wp.data_ptr(), we.data_ptr(), float("inf"), out.data_ptr(), 1, 4, 256,
                        None) == bsr.BSR_EINVAL
    assert L.w4a16_gemv(*args(0, 256)) == bsr.BSR_OK
    torch.cuda.synchronize()
    assert bool((out == 3).all())
