"""Pins of the oracle's other activation layouts (CPU only): int8 with one scale
per 128 or per row, E4M3 with one scale per 32, 128 or per row, and the GEMM
reference with grouped activation scales.

* E4M3 encoding agrees with torch's float32 -> float8_e4m3fn conversion (round
  to nearest even) on random values, every binade boundary and every tie, and
  decodes back through the pinned E4M3 decoder within half a step;
* int8 groups: the exact-rational quantizer of exact_ref on every group;
* E4M3 groups: scale = fl32(amax / 448), the amax element encodes to +-448,
  codes monotone in v, |decode(q) * s - v| within half an E4M3 step of v/s;
* per-32 grouping reproduces the activation requant bit for bit;
* the grouped GEMM reference equals the per-32 reference after expanding the
  activation scales to every 32-block.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_requant_amd import inputs
from exact_ref import bf16_values, f32_bits, quantize_block


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch():
    rng = np.random.default_rng(1)
    grid = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    grid = grid[np.isfinite(grid)]
    mids = (np.sort(np.unique(np.abs(grid)))[:-1] + np.sort(np.unique(np.abs(grid)))[1:]) / 2
    x = np.concatenate([grid, mids, -mids, rng.uniform(-448, 448, 4000), rng.standard_normal(4000) * 0.01,
                        (2.0 ** rng.uniform(-12, 8.8, 4000)).astype(np.float32)]).astype(np.float32)
    ours = np.array([oracle.e4m3_encode(float(v)) for v in x], np.uint8)
    ref = _torch_e4m3(x)
    # -0 and +0 differ only in sign; torch keeps the sign too
    assert np.array_equal(ours, ref), x[ours != ref][:8]


@pytest.mark.parametrize("group", [32, 128, 512])
def test_int8_groups_against_exact(group):
    rng = np.random.default_rng(group)
    m, k = 3, 512
    a = inputs.bf16_normal(rng, m, k)
    a[1, : group] = 0
    q, s = oracle.quant_act(a, group)
    vals = bf16_values(a.ravel())
    for gi in range(m * k // group):
        s_ref, q_ref = quantize_block(vals[gi * group:(gi + 1) * group])
        assert f32_bits(s_ref) == int(s.ravel()[gi:gi + 1].view(np.uint32)[0])
        assert list(q.ravel()[gi * group:(gi + 1) * group].view(np.int8)) == q_ref


def test_per32_int8_equals_requant_a():
    a = inputs.workload("attn_proj").projections[0].activations(m=4)
    q, s = oracle.quant_act(a, 32)
    q2, s2 = oracle.requant_a(a)
    assert np.array_equal(q.view(np.int8), q2) and np.array_equal(s, s2)


@pytest.mark.parametrize("group", [32, 128, 1024])
def test_e4m3_groups_invariants(group):
    rng = np.random.default_rng(7 + group)
    m, k = 4, 1024
    a = inputs.bf16_student_t(rng, m, k)
    a[2, :group] = 0
    q, s = oracle.quant_act(a, group, e4m3=True)
    v = np.array([float(x) for x in bf16_values(a.ravel())]).reshape(-1, group)
    codes = q.reshape(-1, group)
    sc = s.reshape(-1).astype(np.float64)
    amax = np.abs(v).max(axis=1)
    assert np.array_equal(s.reshape(-1), amax.astype(np.float32) / np.float32(448.0))
    dec = np.array([oracle.e4m3_value(int(c)) for c in codes.ravel()]).reshape(codes.shape)
    zero = sc == 0
    assert np.all(codes[zero] == 0)
    nz = ~zero
    at = np.abs(v) == amax[:, None]
    assert np.all(np.abs(dec[nz][at[nz]]) == 448.0)
    # nearest E4M3 value of fl32(v / s): the error is at most half the local step
    r = (v / np.where(zero, 1.0, sc)[:, None]).astype(np.float32).astype(np.float64)
    step = np.where(np.abs(r) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 3), 2.0 ** -9)
    assert np.all((np.abs(dec - r) <= step / 2 + 1e-12)[nz])
    order = np.argsort(v, axis=1, kind="stable")
    ds = np.take_along_axis(dec, order, axis=1)
    assert np.all(np.diff(ds, axis=1)[nz] >= 0)


@pytest.mark.parametrize("group", [128, 512])
def test_grouped_gemm_reference_matches_expanded_scales(group):
    rng = np.random.default_rng(3)
    m, n, k = 5, 7, 512
    a = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    w = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    a_s = (rng.uniform(0.5, 2, size=(m, k // group)) * 2.0 ** -8).astype(np.float32)
    w_s = (rng.uniform(0.5, 2, size=(n, k // 32)) * 2.0 ** -9).astype(np.float32)
    y, t = oracle.gemm_ref_agroup(a, w, a_s, w_s, group)
    y2, t2 = oracle.gemm_ref(a, w, np.repeat(a_s, group // 32, axis=1), w_s)
    assert np.array_equal(y, y2) and np.array_equal(t, t2)
