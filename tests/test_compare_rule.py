"""Pins of the BF16 pass rule (CPU only): accepts correctly rounded FP32 sums in
any block order, rejects planted errors, handles zeros and cancellation."""
import numpy as np

import oracle
from oracle.compare import bf16_ulp, check_bf16
from block_scaled_precision_requant_amd import inputs


def _to_bf16_bits(x):
    return inputs.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_ulp_definition():
    assert bf16_ulp(1.0) == 2.0 ** -7
    assert bf16_ulp(1.99) == 2.0 ** -7
    assert bf16_ulp(-3.0) == 2.0 ** -6
    assert bf16_ulp(2.0 ** -130) == 2.0 ** -133
    assert bf16_ulp(0.0) == 0.0


def _fp32_block_sums(a_i8, w_i8, a_s, w_s, order):
    p = oracle.block_partials(a_i8, w_i8).astype(np.float32)
    sprod = (a_s[:, None, :] * w_s[None, :, :]).astype(np.float32)
    acc = np.zeros(p.shape[:2], np.float32)
    for b in order:
        acc = (acc + (sprod[:, :, b] * p[:, :, b]).astype(np.float32)).astype(np.float32)
    return acc


def test_fp32_accumulation_in_any_order_passes():
    proj = inputs.workload("tiny").projections[0]
    wp, we = proj.weight()
    w_i8, w_s = oracle.requant_w(wp, we, proj.scale2)
    a_i8, a_s = oracle.requant_a(proj.activations())
    y, t = oracle.gemm_ref(a_i8, w_i8, a_s, w_s)
    nb = proj.k // 32
    rng = np.random.default_rng(0)
    for order in (range(nb), range(nb - 1, -1, -1), rng.permutation(nb)):
        out = _to_bf16_bits(_fp32_block_sums(a_i8, w_i8, a_s, w_s, order))
        res = check_bf16(out, y, t, proj.k)
        assert res.ok, str(res)


def test_planted_errors_fail():
    y = np.array([[1.0, -3.5, 100.0, 1e-3]])
    t = np.abs(y)
    out = _to_bf16_bits(y)
    assert check_bf16(out, y, t, 32).ok
    bad = out.copy()
    bad[0, 2] += 2                     # two BF16 steps at 100 (0.8%)
    res = check_bf16(bad, y, t, 32)
    assert not res.ok and res.first_failure == (0, 2)
    nan = out.copy()
    nan[0, 0] = 0x7FC0
    assert not check_bf16(nan, y, t, 32).ok


def test_zero_reference():
    y = np.zeros((1, 2))
    t = np.zeros((1, 2))
    assert check_bf16(np.array([[0x0000, 0x8000]], np.uint16), y, t, 64).ok
    assert not check_bf16(np.array([[0x0001, 0x0000]], np.uint16), y, t, 64).ok
    # with cancellation (t > 0) a tiny nonzero output is within the FP32 sum bound
    t2 = np.full((1, 2), 1.0)
    res = check_bf16(np.array([[0x3380, 0x0000]], np.uint16), y, t2, 64)   # 2^-24 * ~1
    assert res.ok and res.needed_ii == 1


def test_cancellation_uses_sum_bound():
    # y is tiny next to T: a 1% miss on y is inside (K/32 + 2) * 2^-24 * T.
    y = np.array([[1e-6]])
    t = np.array([[10.0]])
    out = _to_bf16_bits(y * 1.01)
    res = check_bf16(out, y, t, 4096)
    assert res.ok and res.needed_ii == 1
    assert not check_bf16(_to_bf16_bits(y * 1.5), np.array([[1e-6]]), np.array([[1e-5]]), 4096).ok


def test_w4a16_bound_per_kernel():
    """The streamed W4A16 kernel (K % 256 == 0) gets the bound of K/16 block terms plus
    the in-block, wave and scale_2 roundings; the register-decode kernel keeps K + 16."""
    from oracle.compare import w4a16_terms
    assert w4a16_terms(14336) == 14336 / 16 + 31
    assert w4a16_terms(4096) == 4096 / 16 + 31
    assert w4a16_terms(4128) == 4128 + 16
    assert w4a16_terms(96) == 96 + 16
    # an error of half the streamed bound passes, twice it fails (no cancellation help:
    # y = 0, T large)
    import numpy as np
    from oracle.compare import check_bf16
    k, t = 4096, np.array([[2.0 ** 20]])
    b = (w4a16_terms(k) + 2) * 2.0 ** -24 * t[0, 0]
    f32 = lambda v: np.array([[v]], np.float32).view(np.uint32) >> 16
    ok = check_bf16(f32(0.5 * b).astype(np.uint16), np.zeros((1, 1)), t, k, terms=w4a16_terms(k))
    bad = check_bf16(f32(2.0 * b).astype(np.uint16), np.zeros((1, 1)), t, k, terms=w4a16_terms(k))
    assert ok.ok and not bad.ok
