"""The kernels at their size limits, where 32-bit index arithmetic would wrap:
the GEMM at the largest K it accepts (k = 2^25 - 32, a 64-row tile's A rows then
span 2 GiB), the int8 GEMV at k = 2^27 and the W4A16 GEMV at k = 2^28 (weight rows
starting past 4 GiB), and the quantizers on more than 2^32
elements (offsets past 4 GiB of codes, 8 GiB of BF16 input).  Inputs this large
are drawn on the device with a seeded torch generator (synthetic, as everywhere
else); the oracle then checks the rows or 32-element blocks it can afford,
copied back from those same input tensors -- the first and last of every row,
the ones straddling the 2^31 and 2^32 element marks, and random ones."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_requant_amd import bsr, inputs
from gpu_util import DEV, canary_out, f32_bits, host, say
from oracle.compare import check_bf16, w4a16_terms

pytestmark = pytest.mark.gpu

K_MAX_GEMM = (1 << 25) - 32


@pytest.fixture(autouse=True)
def _release_memory():
    """These tests hold up to ~35 GB of device memory; hand it back to the
    device after each, so later tests see the usual free memory."""
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _i8(gen, rows, cols):
    return torch.randint(-127, 128, (rows, cols), dtype=torch.int8, device=DEV, generator=gen)


def _scales(gen, rows, cols, lo, hi):
    """Positive binary32 scales, uniform in [0.5, 2) times 2^e, e in [lo, hi)."""
    mant = torch.rand((rows, cols), device=DEV, generator=gen) * 1.5 + 0.5
    e = torch.randint(lo, hi, (rows, cols), device=DEV, generator=gen).to(torch.float32)
    return (mant * torch.exp2(e)).contiguous()


def _bf16(gen, rows, cols):
    return torch.randn((rows, cols), device=DEV, generator=gen, dtype=torch.bfloat16).view(torch.int16)


def _sample_blocks(rows, k, rng, extra=48):
    """(row, block) pairs: each row's first and last block, the blocks holding
    elements 2^31 and 2^32 (row-major over [rows, k]) and random ones."""
    nb = k // 32
    picks = set()
    for r in range(rows):
        picks.update({(r, 0), (r, nb - 1)})
    for e in (1 << 31, (1 << 32) - 32, 1 << 32):
        if e < rows * k:
            picks.add((e // k, (e % k) // 32))
    for _ in range(extra):
        picks.add((int(rng.integers(0, rows)), int(rng.integers(0, nb))))
    return sorted(picks)


def _block(t, r, b):
    """Elements [32 b, 32 b + 32) of row r of a device tensor, on the host."""
    return host(t[r, 32 * b:32 * b + 32].contiguous())[None, :]


def test_gemm_at_max_k():
    m, n, k = 129, 40, K_MAX_GEMM
    say(f"gemm at max k: m={m} n={n} k={k}")
    gen = _gen(101)
    a, w = _i8(gen, m, k), _i8(gen, n, k)
    a_s, w_s = _scales(gen, m, k // 32, -12, -2), _scales(gen, n, k // 32, -14, -4)
    rows = np.array([0, 31, 32, 63, 64, 127, 128])
    sel = torch.as_tensor(rows, device=DEV)
    y, t = oracle.gemm_ref(host(a[sel]), host(w), host(a_s[sel]), host(w_s))
    need = bsr.int8_gemm_blockscaled_ws_bytes(m, n, k)
    assert need > 0, "a split plan at this shape"
    ws = torch.empty(need // 4, dtype=torch.float32, device=DEV)
    for name in ("auto", "invariant", "workspace"):
        say(f"  {name}")
        out = canary_out(m, n)
        if name == "auto":            # 32 x 32 tiles, K split over 8 wave groups
            bsr.int8_gemm_blockscaled(a, w, a_s, w_s, out)
        elif name == "invariant":     # 64 x 64 tiles, no K split
            bsr.int8_gemm_blockscaled_ex(a, w, a_s, w_s, out, path=bsr.PATH_INVARIANT)
        else:                         # K slices across workgroups
            bsr.int8_gemm_blockscaled_ws(a, w, a_s, w_s, out, ws)
        got = host(out)
        assert not np.any(got == 0x7FA5), "every output written"
        res = check_bf16(got[rows], y, t, k)
        say(f"  {res}")
        assert res.ok, (name, res)


def test_gemv_and_w4a16_at_long_k():
    m, n, k = 5, 40, 1 << 27
    say(f"gemv at long k: m={m} n={n} k={k}")
    gen = _gen(102)
    a, w = _i8(gen, m, k), _i8(gen, n, k)
    a_s, w_s = _scales(gen, m, k // 32, -12, -2), _scales(gen, n, k // 32, -14, -4)
    y, t = oracle.gemm_ref(host(a), host(w), host(a_s), host(w_s))
    for path in (bsr.PATH_GEMV, bsr.PATH_INVARIANT):
        out = canary_out(m, n)
        bsr.int8_gemm_blockscaled_ex(a, w, a_s, w_s, out, path=path)
        res = check_bf16(host(out), y, t, k)
        say(f"  path {path}: {res}")
        assert res.ok, (path, res)
    del a, w, a_s, w_s
    # W4A16 at k = 2^28: a packed weight row is 128 MiB, so rows from 32 on
    # start past 4 GiB; the oracle checks output columns 0, 32 and 39 (weight
    # rows are independent) and the canary every output
    k = 1 << 28
    say(f"w4a16 at long k: m={m} n={n} k={k}")
    x = _bf16(gen, m, k)
    wp = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device=DEV, generator=gen)
    we = ((torch.randint(0x20, 0x48, (n, k // 16), device=DEV, generator=gen)) |
          (torch.randint(0, 2, (n, k // 16), device=DEV, generator=gen) << 7)).to(torch.uint8)
    out = canary_out(m, n)
    bsr.w4a16_gemv(x, wp, we, inputs.SCALE2_1_448, out)
    got = host(out)
    assert not np.any(got == 0x7FA5), "every output written"
    cols = torch.as_tensor([0, 32, 39], device=DEV)
    y, t = oracle.w4a16_ref(host(x), host(wp[cols]), host(we[cols]), inputs.SCALE2_1_448)
    res = check_bf16(got[:, [0, 32, 39]], y, t, k, terms=w4a16_terms(k))
    say(f"  {res}")
    assert res.ok, res


def test_quantizers_past_2_32_elements():
    rows, k = 3, 1 << 31
    rng = np.random.default_rng(103)
    gen = _gen(103)
    picks = _sample_blocks(rows, k, rng)
    say(f"requant_a on {rows}x{k} ({len(picks)} blocks checked)")
    a = _bf16(gen, rows, k)
    q = torch.empty((rows, k), dtype=torch.int8, device=DEV)
    s = torch.empty((rows, k // 32), dtype=torch.float32, device=DEV)
    bsr.requant_a_int8(a, q, s)
    for r, b in picks:
        q_ref, s_ref = oracle.requant_a(_block(a, r, b))
        assert np.array_equal(_block(q, r, b), q_ref), (r, b)
        assert f32_bits(host(s[r, b:b + 1]))[0] == f32_bits(s_ref)[0, 0], (r, b)

    say(f"silu_mul_requant on {rows}x{k}")
    up = _bf16(gen, rows, k)
    bsr.silu_mul_requant_int8(a, up, q, s)
    for r, b in picks:
        q_ref, s_ref = oracle.silu_mul_requant(_block(a, r, b), _block(up, r, b))
        assert np.array_equal(_block(q, r, b), q_ref), (r, b)
        assert f32_bits(host(s[r, b:b + 1]))[0] == f32_bits(s_ref)[0, 0], (r, b)
    del a, up

    say(f"requant_w on {rows}x{k}")
    wp = torch.randint(0, 256, (rows, k // 2), dtype=torch.uint8, device=DEV, generator=gen)
    we = torch.randint(0, 0x7F, (rows, k // 16), dtype=torch.uint8, device=DEV, generator=gen)
    bsr.requant_w_nvfp4_int8(wp, we, inputs.SCALE2_1_448, q, s)
    for r, b in picks:
        q_ref, s_ref = oracle.requant_w(host(wp[r, 16 * b:16 * b + 16].contiguous())[None, :],
                                        host(we[r, 2 * b:2 * b + 2].contiguous())[None, :], inputs.SCALE2_1_448)
        assert np.array_equal(_block(q, r, b), q_ref), (r, b)
        assert f32_bits(host(s[r, b:b + 1]))[0] == f32_bits(s_ref)[0, 0], (r, b)


@pytest.mark.parametrize("group,fmt,e4m3", [(32, bsr.FMT_E4M3, True), (128, bsr.FMT_INT8, False),
                                            (0, bsr.FMT_E4M3, True)])
def test_quantize_act_past_2_32_elements(group, fmt, e4m3):
    rows, k = 3, 1 << 31
    rng = np.random.default_rng(104)
    say(f"quantize_act on {rows}x{k}, group {group}, e4m3 {e4m3}")
    a = _bf16(_gen(104), rows, k)
    q = torch.empty((rows, k), dtype=torch.uint8, device=DEV)
    s = torch.empty((rows, 1 if group == 0 else k // group), dtype=torch.float32, device=DEV)
    bsr.quantize_act(a, q, s, group=group, fmt=fmt)
    if group == 0:
        # One scale per row.  A block's codes depend only on its values and the
        # row's scale, so the oracle quantizes each sampled block beside a block
        # that holds only the row's largest-magnitude element (found with a
        # torch argmax): that 64-element row has the same scale.
        for r in range(rows):
            i = int(a[r].view(torch.bfloat16).float().abs().argmax())
            peak = np.zeros((1, 32), dtype=np.uint16)
            peak[0, 0] = host(a[r, i:i + 1])[0]
            for rr, b in _sample_blocks(rows, k, rng):
                if rr != r:
                    continue
                q_ref, s_ref = oracle.quant_act(np.concatenate([_block(a, r, b), peak], axis=1), 64, e4m3=e4m3)
                assert f32_bits(host(s[r]))[0] == f32_bits(s_ref)[0, 0], (r, b)
                assert np.array_equal(host(q[r, 32 * b:32 * b + 32].contiguous()), q_ref[0, :32]), (r, b)
    else:
        for r, b in _sample_blocks(rows, k, rng):
            g0 = (32 * b) // group * group            # the block's scale group
            src = host(a[r, g0:g0 + group].contiguous())[None, :]
            q_ref, s_ref = oracle.quant_act(src, group, e4m3=e4m3)
            assert np.array_equal(host(q[r, g0:g0 + group].contiguous()), q_ref[0]), (r, b)
            assert f32_bits(host(s[r, g0 // group:g0 // group + 1]))[0] == f32_bits(s_ref)[0, 0], (r, b)
