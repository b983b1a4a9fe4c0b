"""Path and batch invariance on the GPU: with BSR_PATH_INVARIANT a row's BF16
bits do not depend on m or on which kernel ran.  For m <= 16 that path runs the
chain GEMV, for m > 16 the GEMM without its K split, both accumulating every
output over the K blocks in increasing order, so the same row must give the
same bits run alone, in a small batch (GEMV) or padded past 16 rows (GEMM) --
and stay within the oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_requant_amd import bsr, inputs
from gpu_util import DEV, gpu_gemm, gpu_gemm_agroup, gpu_quant_act, gpu_requant_a, gpu_requant_w, host, say, \
    to_dev
from oracle.compare import check_bf16

pytestmark = pytest.mark.gpu

PAD = 17  # rows that lift an m <= 16 input onto the GEMM (m > 16)


def _padded(t, rows=PAD):
    """t with `rows` extra rows of its last row appended (same dtype, on the GPU)."""
    return torch.cat([t, t[-1:].expand(rows, *t.shape[1:])]).contiguous()


def _gemm_rows(a_i8, w_i8, a_s, w_s):
    """The invariant path's GEMM on these rows (padded past 16 rows), first m rows."""
    m = a_i8.shape[0]
    return host(gpu_gemm(_padded(a_i8), w_i8, _padded(a_s), w_s, path=bsr.PATH_INVARIANT))[:m]


def _operands(seed, m, n, k):
    rng = np.random.default_rng(seed)
    a = inputs.bf16_student_t(rng, m, k)
    packed, e4m3 = inputs.nvfp4_weight(rng, n, k, -4, 2)
    return a, packed, e4m3


@pytest.mark.parametrize("k", [32, 96, 256, 1056, 1152, 2304, 4096, 14336])  # 1152: a partial last chunk
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 9, 16])
def test_invariant_gemv_equals_gemm(m, k):
    n = 200
    say(f"invariant gemv m={m} n={n} k={k}")
    a, packed, e4m3 = _operands(m * 1000 + k, m, n, k)
    w_i8, w_s = gpu_requant_w(packed, e4m3, inputs.SCALE2_1_448)
    a_i8, a_s = gpu_requant_a(a)
    inv = host(gpu_gemm(a_i8, w_i8, a_s, w_s, path=bsr.PATH_INVARIANT))
    ref = _gemm_rows(a_i8, w_i8, a_s, w_s)
    assert np.array_equal(inv, ref), np.argwhere(inv != ref)[:5]
    oa, osa = oracle.requant_a(a)
    ow, osw = oracle.requant_w(packed, e4m3, inputs.SCALE2_1_448)
    y, t = oracle.gemm_ref(oa, ow, osa, osw)
    res = check_bf16(inv, y, t, k)
    assert res.ok, res


def test_invariant_rows_independent_of_m():
    """Rows of a 300-row GEMM equal the same rows run alone or in groups of up to 16."""
    m, n, k = 300, 333, 2048
    a, packed, e4m3 = _operands(5, m, n, k)
    w_i8, w_s = gpu_requant_w(packed, e4m3, inputs.SCALE2_1_448)
    a_i8, a_s = gpu_requant_a(a)
    full = host(gpu_gemm(a_i8, w_i8, a_s, w_s, path=bsr.PATH_INVARIANT))
    for lo, hi in [(0, 1), (7, 15), (100, 103), (299, 300), (42, 48), (150, 159), (10, 140), (20, 36),
                   (283, 295)]:
        part = host(gpu_gemm(a_i8[lo:hi].contiguous(), w_i8, a_s[lo:hi].contiguous(), w_s,
                             path=bsr.PATH_INVARIANT))
        assert np.array_equal(part, full[lo:hi]), (lo, hi)


@pytest.mark.parametrize("name", ["decode_m1_n14336_k4096", "decode_m8_n14336_k4096",
                                  "decode_m1_n4096_k14336", "decode_m8_n4096_k14336"])
def test_invariant_decode_workloads(name):
    p = [q for q in inputs.workload("decode").projections if q.name == name][0]
    packed, e4m3 = p.weight()
    w_i8, w_s = gpu_requant_w(packed, e4m3, p.scale2)
    a_i8, a_s = gpu_requant_a(p.activations())
    inv = host(gpu_gemm(a_i8, w_i8, a_s, w_s, path=bsr.PATH_INVARIANT))
    ref = _gemm_rows(a_i8, w_i8, a_s, w_s)
    say(f"{name}: {int((inv != ref).sum())} differing outputs")
    assert np.array_equal(inv, ref)


@pytest.mark.parametrize("group", [128, 0])
@pytest.mark.parametrize("m", [1, 8, 16])
def test_invariant_grouped_scales(m, group):
    n, k = 130, 4096
    a, packed, e4m3 = _operands(77 + m, m, n, k)
    w_i8, w_s = gpu_requant_w(packed, e4m3, inputs.SCALE2_1_448)
    q, s = gpu_quant_act(a, group)
    inv = host(gpu_gemm_agroup(q.view(torch.int8), w_i8, s, group, w_s, path=bsr.PATH_INVARIANT))
    ref = host(gpu_gemm_agroup(_padded(q.view(torch.int8)), w_i8, _padded(s), group, w_s,
                               path=bsr.PATH_INVARIANT))[:m]
    assert np.array_equal(inv, ref)


# Grids of more than one 16-column workgroup per CU (n = 4112: 257 of them,
# the last one ragged) with K a multiple of 256 take the streamed kernel as
# one wave per workgroup; its outputs must equal the GEMM's chain bit for bit.
@pytest.mark.parametrize("group", [32, 128, 0])
@pytest.mark.parametrize("m,k", [(1, 256), (3, 2048), (9, 512), (16, 4096)])
def test_invariant_wide_grid(m, k, group):
    n = 4112
    say(f"invariant wide grid m={m} n={n} k={k} group={group}")
    a, packed, e4m3 = _operands(31 * m + k + group, m, n, k)
    w_i8, w_s = gpu_requant_w(packed, e4m3, inputs.SCALE2_1_448)
    q, s = gpu_quant_act(a, group)
    inv = host(gpu_gemm_agroup(q.view(torch.int8), w_i8, s, group, w_s, path=bsr.PATH_INVARIANT))
    ref = host(gpu_gemm_agroup(_padded(q.view(torch.int8)), w_i8, _padded(s), group, w_s,
                               path=bsr.PATH_INVARIANT))[:m]
    assert np.array_equal(inv, ref), np.argwhere(inv != ref)[:5]


def test_invariant_tiny_scale_products():
    """Scale products in the binary32 subnormal range and the largest finite
    products: the GEMM's matrix-core product and the GEMV's vector product of
    a_s * w_s must round alike."""
    rng = np.random.default_rng(9)
    m, n, k = 4, 96, 1024
    a_i8 = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    w_i8 = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    a_s = (rng.uniform(1, 2, (m, k // 32)) * 2.0 ** rng.integers(-80, -60, (m, k // 32))).astype(np.float32)
    w_s = (rng.uniform(1, 2, (n, k // 32)) * 2.0 ** rng.integers(-80, -60, (n, k // 32))).astype(np.float32)
    a_s[:, ::5] *= np.float32(2.0 ** 100)
    w_s[:, ::7] *= np.float32(2.0 ** 100)
    da, dw, das, dws = to_dev(a_i8), to_dev(w_i8), to_dev(a_s), to_dev(w_s)
    inv = host(gpu_gemm(da, dw, das, dws, path=bsr.PATH_INVARIANT))
    ref = _gemm_rows(da, dw, das, dws)
    y, t = oracle.gemm_ref(a_i8, w_i8, a_s, w_s)
    say(f"tiny scales: {int((inv != ref).sum())} differing outputs; "
        f"gemm {check_bf16(ref, y, t, k)}; chain {check_bf16(inv, y, t, k)}")
    # the default GEMM path (which may split K) stays within the oracle's rule
    res = check_bf16(host(gpu_gemm(da, dw, das, dws, path=bsr.PATH_GEMM)), y, t, k)
    assert res.ok, res
    assert np.array_equal(inv, ref)


def test_invariant_path_errors():
    a = torch.zeros((4, 64), dtype=torch.int8, device=DEV)
    w = torch.zeros((8, 64), dtype=torch.int8, device=DEV)
    s_a = torch.zeros((4, 2), dtype=torch.float32, device=DEV)
    s_w = torch.zeros((8, 2), dtype=torch.float32, device=DEV)
    out = torch.empty((4, 8), dtype=torch.int16, device=DEV)
    with pytest.raises(bsr.BsrError):
        bsr.int8_gemm_blockscaled_ex(a, w, s_a, s_w, out, path=4)
    bsr.int8_gemm_blockscaled_ex(a, w, s_a, s_w, out, path=bsr.PATH_INVARIANT)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


@pytest.mark.parametrize("k", [512, 544])
def test_rows_equal_across_gemm_tile_shapes(k):
    """A 2048-row GEMM at N = 4096 runs 256x128 tiles; the same rows inside a
    2112-row GEMM run 128x128 tiles (a 256-row tiling would pad 2112); 100 of
    them alone run 64x64 tiles, and 16 of them the chain GEMV: the same bits
    every time.  The big tiles stage scales 8 blocks at a time: K = 544 (17
    blocks, 5 stages) ends in a scale stage with one live block."""
    m, n = 2048, 4096
    a, packed, e4m3 = _operands(11, m, n, k)
    w_i8, w_s = gpu_requant_w(packed, e4m3, inputs.SCALE2_1_448)
    a_i8, a_s = gpu_requant_a(a)
    full = host(gpu_gemm(a_i8, w_i8, a_s, w_s, path=bsr.PATH_INVARIANT))
    wider = host(gpu_gemm(torch.cat([a_i8, a_i8[:64]]).contiguous(), w_i8, torch.cat([a_s, a_s[:64]]).contiguous(),
                          w_s, path=bsr.PATH_INVARIANT))
    assert np.array_equal(wider[:m], full)
    for lo, hi in [(5, 105), (1000, 1016), (1900, 2048)]:
        part = host(gpu_gemm(a_i8[lo:hi].contiguous(), w_i8, a_s[lo:hi].contiguous(), w_s,
                             path=bsr.PATH_INVARIANT))
        assert np.array_equal(part, full[lo:hi]), (lo, hi)
