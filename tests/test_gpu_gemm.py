"""GPU parity of the block-scaled GEMM and GEMV against the CPU oracle's FP64
reference (pass rule in oracle/compare.py), plus the bit-exact special cases,
invariants and guard bands."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_requant_amd import bsr, inputs
from gpu_util import CANARY, DEV, canary_out, gpu_gemm, gpu_requant_a, gpu_requant_w, host, say, to_dev
from oracle.compare import bf16_ulp, bf16_bits_to_f64, check_bf16

pytestmark = pytest.mark.gpu


def _rand_operands(seed, m, n, k, zero_frac=0.0):
    rng = np.random.default_rng(seed)
    a = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    w = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    a_s = (rng.uniform(0.5, 2.0, size=(m, k // 32)) * 2.0 ** rng.integers(-12, -2, size=(m, k // 32))
           ).astype(np.float32)
    w_s = (rng.uniform(0.5, 2.0, size=(n, k // 32)) * 2.0 ** rng.integers(-14, -4, size=(n, k // 32))
           ).astype(np.float32)
    if zero_frac:
        a_s[rng.random(a_s.shape) < zero_frac] = 0.0
    return a, w, a_s, w_s


def _check(name, out_bits, y, t, k):
    res = check_bf16(out_bits, y, t, k)
    say(f"{name}: {res}")
    assert res.ok, f"{name}: {res}"
    return res


# Small grids split K over 8, 4 or 2 groups inside a workgroup (32x32 tiles
# for at most one or two tiles per CU, else 64x64): uneven group ranges (544:
# 5 stages; 4128: 33 stages with a partial last one), empty groups, and K too
# short to split (96, 32) are all here; (20, 14336, 4096) and (100, 3000,
# 2048) take the 4-group 32x32 tiles, (128, 4200, 1024) and (37, 1000, 160)
# the 2-group 64x64 tiles, (64, 4096, 4096) the 8-group 32x32 tiles; (600, 2000,
# 1056) and (129, 257, 96) the 64x64 tiles with a 4-deep ring (320 and 15
# tiles; 9 stages, the last scale stage holding one live block; one stage).
@pytest.mark.parametrize("m,n,k", [(16, 256, 512), (200, 300, 544), (129, 257, 96), (9, 33, 32), (600, 2000, 1056),
                                   (1000, 130, 1024), (256, 128, 4096), (37, 1000, 160),
                                   (48, 1000, 14336), (17, 512, 4128), (100, 200, 1056), (300, 700, 2080),
                                   (20, 14336, 4096), (100, 3000, 2048), (128, 4200, 1024), (64, 4096, 4096)])
def test_gemm_parity_random(m, n, k):
    say(f"gemm random m={m} n={n} k={k}")
    a, w, a_s, w_s = _rand_operands(m * 7 + n * 13 + k, m, n, k, zero_frac=0.05)
    y, t = oracle.gemm_ref(a, w, a_s, w_s)
    out = gpu_gemm(to_dev(a), to_dev(w), to_dev(a_s), to_dev(w_s), path=bsr.PATH_GEMM)
    _check(f"gemm {m}x{n}x{k}", host(out), y, t, k)


# m > 128 with at least 512 tiles of 128 x 128 takes the big tiles: 256 x 128 at
# m = 1200 (m % 256 = 176, last tile row 1024..1199), 128 x 128 at m = 1100 (a
# 256-row tiling would pad it; last tile row 1024..1099).  The last tile column
# (7296..7399) and the last K stage (33 blocks: 8 stages of 4 and one of 1) are
# partial too.  Rows are independent, so sampled rows (both sides of each tile
# edge) are checked whole against the oracle, and guard bands around the output
# catch stores past its end.
@pytest.mark.parametrize("m", [1100, 1200])
def test_gemm_big_tiles_ragged(m):
    n, k = 7400, 1056
    assert m > 128 and -(-m // 128) * -(-n // 128) >= 512
    a, w, a_s, w_s = _rand_operands(4242, m, n, k, zero_frac=0.02)
    pad = 4096
    buf = torch.full((pad + m * n + pad,), 0x7B7B, dtype=torch.int16, device=DEV)
    out = buf[pad:pad + m * n].view(m, n)
    bsr.int8_gemm_blockscaled_ex(to_dev(a), to_dev(w), to_dev(a_s), to_dev(w_s), out, path=bsr.PATH_GEMM)
    hb = host(buf)
    assert np.all(hb[:pad] == 0x7B7B) and np.all(hb[pad + m * n:] == 0x7B7B)
    # ... and every element inside was written (0x7B7B, ~2^119, is far above any result here)
    assert not np.any(hb[pad:pad + m * n] == 0x7B7B)
    rows = np.array([0, 1, 127, 128, 255, 256, 555, 1023, 1024, 1050, m - 2, m - 1])
    y, t = oracle.gemm_ref(a[rows], w, a_s[rows], w_s)
    _check(f"gemm big tiles {m}x{n}x{k}, rows {rows.tolist()}",
           hb[pad:pad + m * n].reshape(m, n)[rows], y, t, k)


# K = 1056 (33 blocks) and 2400 (75): direct kernel with per-element scale
# loads; 2176 (68 blocks, scale rows padded to 128 in LDS) and 4096: staged
# kernel; m = 8 at K = 16384 needs 180 KB of LDS, so the direct kernel with
# vector scale loads runs, while m = 1 at that K is staged.
@pytest.mark.parametrize("m,k", [(1, 1056), (2, 1056), (3, 1056), (4, 1056), (5, 1056), (6, 1056),
                                 (7, 1056), (8, 1056), (2, 2400), (1, 2176), (3, 2176), (8, 2176),
                                 (5, 4096), (8, 4096), (1, 16384), (8, 16384), (9, 1056), (12, 2176),
                                 (13, 2400), (16, 4096), (16, 16384), (11, 14336)])
def test_gemv_parity_random_and_against_gemm(m, k):
    n = 333
    say(f"gemv m={m} n={n} k={k}")
    a, w, a_s, w_s = _rand_operands(100 + m, m, n, k, zero_frac=0.05)
    y, t = oracle.gemm_ref(a, w, a_s, w_s)
    da, dw, das, dws = to_dev(a), to_dev(w), to_dev(a_s), to_dev(w_s)
    out_v = host(gpu_gemm(da, dw, das, dws, path=bsr.PATH_AUTO))     # m <= 16 -> GEMV
    out_g = host(gpu_gemm(da, dw, das, dws, path=bsr.PATH_GEMM))
    _check(f"gemv m={m}", out_v, y, t, k)
    _check(f"gemm m={m}", out_g, y, t, k)
    dv, dg = bf16_bits_to_f64(out_v), bf16_bits_to_f64(out_g)
    assert np.all(np.abs(dv - dg) <= np.maximum(bf16_ulp(dv), bf16_ulp(dg)))


# The streamed GEMV over two to four 16-row tiles (K a multiple of 256): every
# tile count, ragged last tiles and columns, one chunk per wave (K = 256) and
# long K; the automatic path takes the GEMV for m <= 48 on these narrow grids
# and the GEMM for (64, 257, 4096).
@pytest.mark.parametrize("m,n,k", [(17, 333, 256), (24, 300, 2048), (32, 4096, 4096), (33, 200, 14336),
                                   (48, 1000, 1024), (49, 130, 512), (64, 257, 4096)])
def test_gemv_multi_tile_parity(m, n, k):
    say(f"gemv multi-tile m={m} n={n} k={k}")
    a, w, a_s, w_s = _rand_operands(500 + m, m, n, k, zero_frac=0.05)
    y, t = oracle.gemm_ref(a, w, a_s, w_s)
    da, dw, das, dws = to_dev(a), to_dev(w), to_dev(a_s), to_dev(w_s)
    _check(f"gemv {m}x{n}x{k}", host(gpu_gemm(da, dw, das, dws, path=bsr.PATH_GEMV)), y, t, k)
    _check(f"auto {m}x{n}x{k}", host(gpu_gemm(da, dw, das, dws, path=bsr.PATH_AUTO)), y, t, k)


def test_gemm_exact_power_of_two_bit_equal():
    # Power-of-two scales and small codes: every FP32 step is exact, so the output
    # must be the BF16 rounding of the exact integer result, bit for bit.
    rng = np.random.default_rng(77)
    for (m, n, k, path) in [(300, 200, 1024, bsr.PATH_GEMM), (5, 200, 1024, bsr.PATH_GEMV)]:
        a = rng.integers(-15, 16, size=(m, k)).astype(np.int8)
        w = rng.integers(-15, 16, size=(n, k)).astype(np.int8)
        a_s = np.ldexp(1.0, rng.integers(-6, 2, size=(m, k // 32))).astype(np.float32)
        w_s = np.ldexp(1.0, rng.integers(-6, 2, size=(n, k // 32))).astype(np.float32)
        y, _ = oracle.gemm_ref(a, w, a_s, w_s)     # exact here (integers times 2^-12 .. 2^2)
        exp_bits = inputs.f32_to_bf16_bits(y.astype(np.float32))
        out = host(gpu_gemm(to_dev(a), to_dev(w), to_dev(a_s), to_dev(w_s), path=path))
        assert np.array_equal(out, exp_bits), f"path {path}: {np.sum(out != exp_bits)} mismatches"


def test_gemm_extreme_codes_long_k():
    m, n, k = 130, 96, 8192
    a = np.full((m, k), 127, np.int8)
    a[1::2] = -127
    w = np.full((n, k), 127, np.int8)
    a_s = np.full((m, k // 32), 1.0, np.float32)
    w_s = np.full((n, k // 32), 2.0 ** -20, np.float32)
    y, t = oracle.gemm_ref(a, w, a_s, w_s)
    out = host(gpu_gemm(to_dev(a), to_dev(w), to_dev(a_s), to_dev(w_s), path=bsr.PATH_GEMM))
    _check("extremes", out, y, t, k)
    exp_bits = inputs.f32_to_bf16_bits(y.astype(np.float32))
    assert np.array_equal(out, exp_bits)


def test_a6_worked_example_on_gpu():
    from golden_io import quant_blocks
    g = quant_blocks()
    a = np.zeros((1, 64), np.float32)
    a1 = [float(x) for x in g["A1"]["values"]]
    a2 = [float(x) for x in g["A2"]["values"]]
    a[0, :len(a1)] = a1
    a[0, 32:32 + len(a2)] = a2
    a_bits = inputs.f32_to_bf16_bits(a)
    p1 = np.array([[int(x, 16) for x in g["W1"]["packed_hex"]]], np.uint8)
    e1 = np.array([[int(x, 16) for x in g["W1"]["e4m3_hex"]]], np.uint8)
    p2 = np.array([[int(x, 16) for x in g["W2"]["packed_hex"]]], np.uint8)
    e2 = np.array([[int(x, 16) for x in g["W2"]["e4m3_hex"]]], np.uint8)
    s2 = np.array([int(g["W2"]["scale2_bits"][0], 16)], np.uint32).view(np.float32)[0]
    q1, s1 = gpu_requant_w(p1, e1, np.float32(1.0))
    q2, s2d = gpu_requant_w(p2, e2, s2)
    w_i8 = torch.cat([q1, q2], dim=1).contiguous()
    w_s = torch.cat([s1, s2d], dim=1).contiguous()
    a_i8, a_s = gpu_requant_a(a_bits)
    expect = int(g["A6"]["out_bf16"][0], 16)
    for path in (bsr.PATH_GEMV, bsr.PATH_GEMM):
        out = host(gpu_gemm(a_i8, w_i8, a_s, w_s, path=path))
        assert int(out[0, 0]) == expect


def _tile_rows(m, per_tile, seed, tile=128):
    """`per_tile` distinct seeded rows inside every `tile`-row band of the output
    (offsets differ from band to band), plus the first and the last row."""
    rng = np.random.default_rng(seed)
    rows = {0, m - 1}
    for t0 in range(0, m, tile):
        h = min(tile, m - t0)
        for off in rng.choice(h, size=min(per_tile, h), replace=False):
            rows.add(t0 + int(off))
    return np.array(sorted(rows), dtype=np.int64)


def test_tile_rows_cover_every_band():
    rows = _tile_rows(8192, 2, 4)
    bands = np.unique(rows // 128)
    assert len(bands) == 64 and len(rows) >= 128
    offsets = rows % 128
    assert len(np.unique(offsets)) > 32          # the offset varies from band to band


def _prefill_projections():
    out = [inputs.workload("tiny").projections[0], inputs.workload("attn_proj").projections[0]]
    out += inputs.workload("dense_ffn").projections
    out += inputs.workload("large").projections
    return out


# Workloads the oracle evaluates in full (the tiny and attention-projection
# ones: 2048 x 4096 x 4096 takes about a second on the host); the others on
# seeded rows in every 128-row tile band: 4 per band for the dense FFN's two
# projections (M = 4096: 128 rows + the ends), 3 for the large one (M = 8192:
# 192 rows + the ends).
FULL_ORACLE = {"tiny", "attn_proj"}


@pytest.mark.parametrize("proj", _prefill_projections(), ids=lambda p: p.name)
def test_prefill_workload(proj):
    """Full-size requant + GEMM on the GPU in the benchmark's launch configuration,
    the output pre-filled with a canary: every element must be overwritten, and the
    oracle recomputes every row (small workloads) or seeded rows in every tile band
    from the same seeded inputs."""
    say(f"prefill {proj.name} m={proj.m} n={proj.n} k={proj.k}")
    packed, e4m3 = proj.weight()
    a = proj.activations()
    w_i8, w_s = gpu_requant_w(packed, e4m3, proj.scale2)
    a_i8, a_s = gpu_requant_a(a)
    out = canary_out(proj.m, proj.n)
    bsr.int8_gemm_blockscaled(a_i8, w_i8, a_s, w_s, out)
    out_h = host(out)
    del out, w_i8, w_s, a_i8, a_s
    torch.cuda.empty_cache()
    unwritten = int(np.count_nonzero(out_h == CANARY))
    assert unwritten == 0, f"{unwritten} output elements never written"
    if proj.name in FULL_ORACLE:
        rows = np.arange(proj.m)
    else:
        rows = _tile_rows(proj.m, 4 if proj.m <= 4096 else 3, proj.seed)
    ow, osw = oracle.requant_w(packed, e4m3, proj.scale2)
    oa, osa = oracle.requant_a(a[rows])
    y, t = oracle.gemm_ref(oa, ow, osa, osw)
    _check(f"prefill {proj.name} rows {len(rows)} of {proj.m}", out_h[rows], y, t, proj.k)


@pytest.mark.parametrize("proj", inputs.workload("decode").projections, ids=lambda p: p.name)
def test_decode_workload_full(proj):
    say(f"decode {proj.name}")
    packed, e4m3 = proj.weight()
    a = proj.activations()
    w_i8, w_s = gpu_requant_w(packed, e4m3, proj.scale2)
    a_i8, a_s = gpu_requant_a(a)
    out = host(gpu_gemm(a_i8, w_i8, a_s, w_s))
    ow, osw = oracle.requant_w(packed, e4m3, proj.scale2)
    oa, osa = oracle.requant_a(a)
    y, t = oracle.gemm_ref(oa, ow, osa, osw)
    _check(f"decode {proj.name}", out, y, t, proj.k)


def test_guard_bands_at_edge_shapes():
    k = 96
    for m in [1, 2, 3, 5, 7, 8, 9, 16, 127, 129]:
        for n in [1, 31, 130]:
            a, w, a_s, w_s = _rand_operands(m * 1000 + n, m, n, k)
            pad = 4096
            buf = torch.full((pad + m * n + pad,), 0x7B7B, dtype=torch.int16, device=DEV)
            out = buf[pad:pad + m * n].view(m, n)
            bsr.int8_gemm_blockscaled(to_dev(a), to_dev(w), to_dev(a_s), to_dev(w_s), out)
            hb = host(buf)
            assert np.all(hb[:pad] == 0x7B7B) and np.all(hb[pad + m * n:] == 0x7B7B), (m, n)
            y, t = oracle.gemm_ref(a, w, a_s, w_s)
            assert check_bf16(hb[pad:pad + m * n].reshape(m, n), y, t, k).ok, (m, n)


def test_requant_guard_bands():
    rng = np.random.default_rng(5)
    m, k = 3, 96
    a = inputs.bf16_normal(rng, m, k)
    pad = 256
    qbuf = torch.full((pad + m * k + pad,), 0x5A, dtype=torch.int8, device=DEV)
    sbuf = torch.full((pad + m * k // 32 + pad,), 7.0, dtype=torch.float32, device=DEV)
    bsr.requant_a_int8(to_dev(a.view(np.int16)), qbuf[pad:pad + m * k].view(m, k),
                       sbuf[pad:pad + m * k // 32].view(m, k // 32))
    hq, hs = host(qbuf), host(sbuf)
    assert np.all(hq[:pad] == 0x5A) and np.all(hq[pad + m * k:] == 0x5A)
    assert np.all(hs[:pad] == 7.0) and np.all(hs[pad + m * k // 32:] == 7.0)


def test_stream_ordering_without_sync():
    proj = inputs.workload("tiny").projections[0]
    packed, e4m3 = proj.weight()
    a = proj.activations()
    w_i8, w_s = gpu_requant_w(packed, e4m3, proj.scale2)
    a_i8_ref, a_s_ref = gpu_requant_a(a)
    ref = host(gpu_gemm(a_i8_ref, w_i8, a_s_ref, w_s))
    side = torch.cuda.Stream()
    a_dev = to_dev(a.view(np.int16))
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        a_i8 = torch.empty((proj.m, proj.k), dtype=torch.int8, device=DEV)
        a_s = torch.empty((proj.m, proj.k // 32), dtype=torch.float32, device=DEV)
        out = torch.empty((proj.m, proj.n), dtype=torch.int16, device=DEV)
        for _ in range(3):
            a_i8.fill_(0)
            bsr.prefill(a_dev, w_i8, w_s, a_i8, a_s, out, stream=side)
    side.synchronize()
    assert np.array_equal(host(out), ref)


def test_segments_bit_equal_to_stacked():
    # Requantizing and multiplying the two halves of a stacked weight separately
    # writes the same bits as the stacked launch.
    rng = np.random.default_rng(21)
    n_half, k, m = 192, 512, 144
    packed = rng.integers(0, 256, size=(2 * n_half, k // 2), dtype=np.uint8)
    e4m3 = ((rng.integers(-4, 3, size=(2 * n_half, k // 16)) + 7) << 3).astype(np.uint8)
    a = inputs.bf16_normal(rng, m, k)
    a_i8, a_s = gpu_requant_a(a)
    w_all, s_all = gpu_requant_w(packed, e4m3, inputs.SCALE2_1_448)
    out_all = host(gpu_gemm(a_i8, w_all, a_s, s_all))
    for h in range(2):
        rows = slice(h * n_half, (h + 1) * n_half)
        w_h, s_h = gpu_requant_w(packed[rows], e4m3[rows], inputs.SCALE2_1_448)
        assert torch.equal(w_h, w_all[rows]) and torch.equal(s_h, s_all[rows])
        out_h = host(gpu_gemm(a_i8, w_h, a_s, s_h))
        assert np.array_equal(out_h, out_all[:, rows])


def test_rows_independent_of_m():
    rng = np.random.default_rng(22)
    m, n, k = 300, 160, 512
    a = inputs.bf16_normal(rng, m, k)
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    e4m3 = ((rng.integers(-4, 3, size=(n, k // 16)) + 7) << 3).astype(np.uint8)
    w_i8, w_s = gpu_requant_w(packed, e4m3, inputs.SCALE2_1_448)
    a_i8, a_s = gpu_requant_a(a)
    full = host(gpu_gemm(a_i8, w_i8, a_s, w_s))
    sub_i8, sub_s = gpu_requant_a(a[37:200])
    assert torch.equal(sub_i8, a_i8[37:200]) and torch.equal(sub_s, a_s[37:200])
    sub = host(gpu_gemm(sub_i8, w_i8, sub_s, w_s))
    assert np.array_equal(sub, full[37:200])


def test_error_status_leaves_output_untouched():
    m, n, k = 16, 64, 64
    a_i8 = torch.zeros((m, k), dtype=torch.int8, device=DEV)
    w_i8 = torch.zeros((n, k), dtype=torch.int8, device=DEV)
    a_s = torch.ones((m, k // 32), dtype=torch.float32, device=DEV)
    w_s = torch.ones((n, k // 32), dtype=torch.float32, device=DEV)
    raw = torch.full((m * n + 8,), 0x1234, dtype=torch.int16, device=DEV)
    L = bsr.lib()
    vp = lambda t, off=0: __import__("ctypes").c_void_p(t.data_ptr() + off)
    st = L.int8_gemm_blockscaled(vp(a_i8, 1), vp(w_i8), vp(a_s), vp(w_s), vp(raw), m, n, k, None)
    assert st == bsr.BSR_EALIGN
    st = L.int8_gemm_blockscaled(vp(a_i8), vp(w_i8), vp(a_s), vp(w_s), vp(raw), m, n, 48, None)
    assert st == bsr.BSR_EINVAL
    torch.cuda.synchronize()
    assert torch.all(raw == 0x1234)
    st = L.int8_gemm_blockscaled(vp(a_i8), vp(w_i8), vp(a_s), vp(w_s), vp(raw), m, n, k, None)
    assert st == bsr.BSR_OK
    torch.cuda.synchronize()
    assert torch.all(raw[:m * n] == 0) and torch.all(raw[m * n:] == 0x1234)


@pytest.mark.parametrize("m,k,path", [(300, 1024, bsr.PATH_GEMM), (4, 4096, bsr.PATH_GEMV),
                                      (8, 16384, bsr.PATH_GEMV), (3, 1056, bsr.PATH_GEMV),
                                      (5, 4096, bsr.PATH_INVARIANT), (2, 1056, bsr.PATH_INVARIANT)])
def test_scales_at_4_byte_alignment(m, k, path):
    """The ABI asks only 4-byte alignment of the F32 scales: scale tensors that
    start one float into their allocation give the same bits."""
    n = 96
    say(f"4-byte-aligned scales m={m} k={k} path={path}")
    a, w, a_s, w_s = _rand_operands(7 + m + k, m, n, k)
    da, dw = to_dev(a), to_dev(w)
    ref = host(gpu_gemm(da, dw, to_dev(a_s), to_dev(w_s), path=path))
    big_a = torch.zeros(a_s.size + 4, dtype=torch.float32, device=DEV)
    big_w = torch.zeros(w_s.size + 4, dtype=torch.float32, device=DEV)
    sa = big_a[1:1 + a_s.size].view(a_s.shape)
    sw = big_w[1:1 + w_s.size].view(w_s.shape)
    sa.copy_(to_dev(a_s))
    sw.copy_(to_dev(w_s))
    assert sa.data_ptr() % 16 == 4 and sw.data_ptr() % 16 == 4
    out = host(gpu_gemm(da, dw, sa, sw, path=path))
    assert np.array_equal(out, ref)


# Grids of fewer 64 x 64 tiles than CUs split K across workgroups when given a
# workspace (m > 32, K >= 8192): m = 33..192 at n = 4096 and 14336, ragged m,
# n and K (65 x 130 x 8992: 71 stages, the last one a single block, in 15
# slices of 5 -- the last slice one partial stage), two slices (48 x 14336,
# 192 x 4096) and sixteen (129 x 300).
@pytest.mark.parametrize("m,n,k", [(33, 4096, 14336), (64, 4096, 14336), (65, 130, 8992), (100, 200, 8192),
                                   (48, 14336, 8192), (129, 300, 8192), (192, 4096, 14336)])
def test_gemm_split_k_parity(m, n, k):
    say(f"split-K gemm m={m} n={n} k={k}")
    need = bsr.int8_gemm_blockscaled_ws_bytes(m, n, k)
    assert 0 < need <= 8 << 20
    a, w, a_s, w_s = _rand_operands(900 + m + n, m, n, k, zero_frac=0.03)
    y, t = oracle.gemm_ref(a, w, a_s, w_s)
    da, dw, das, dws = to_dev(a), to_dev(w), to_dev(a_s), to_dev(w_s)
    # the workspace's contents on entry do not matter: NaN-filled, then reused as left
    ws = torch.full((need // 4 + 64,), float("nan"), dtype=torch.float32, device=DEV)
    outs = []
    for _ in range(2):
        out = canary_out(m, n)
        bsr.int8_gemm_blockscaled_ws(da, dw, das, dws, out, ws[:need // 4])
        outs.append(host(out))
    assert torch.isnan(ws[need // 4:]).all(), "stores past the workspace size"
    _check(f"split-K {m}x{n}x{k}", outs[0], y, t, k)
    assert np.array_equal(outs[0], outs[1]), "the split is deterministic"


def test_gemm_split_k_errors_and_no_split():
    m, n, k = 64, 4096, 8192
    need = bsr.int8_gemm_blockscaled_ws_bytes(m, n, k)
    assert need > 0
    a, w, a_s, w_s = _rand_operands(31, m, n, k)
    da, dw, das, dws = to_dev(a), to_dev(w), to_dev(a_s), to_dev(w_s)
    out = canary_out(m, n)
    small = torch.zeros(need // 4 - 4, dtype=torch.float32, device=DEV)
    with pytest.raises(bsr.BsrError) as e:
        bsr.int8_gemm_blockscaled_ws(da, dw, das, dws, out, small)
    assert e.value.status == bsr.BSR_EINVAL
    with pytest.raises(bsr.BsrError) as e:
        bsr.int8_gemm_blockscaled_ws(da, dw, das, dws, out, None)
    assert e.value.status == bsr.BSR_ENULL
    torch.cuda.synchronize()
    assert np.all(host(out) == CANARY), "an error launches nothing"
    # a problem with no split ignores the workspace and equals int8_gemm_blockscaled bit for bit
    m2, n2, k2 = 1024, 2048, 1024
    assert bsr.int8_gemm_blockscaled_ws_bytes(m2, n2, k2) == 0
    a, w, a_s, w_s = _rand_operands(32, m2, n2, k2)
    da, dw, das, dws = to_dev(a), to_dev(w), to_dev(a_s), to_dev(w_s)
    ref = canary_out(m2, n2)
    bsr.int8_gemm_blockscaled(da, dw, das, dws, ref)
    got = canary_out(m2, n2)
    bsr.int8_gemm_blockscaled_ws(da, dw, das, dws, got, None)
    assert np.array_equal(host(got), host(ref))


def _padded(arr, fill, pad_bytes=512):
    """A device copy of `arr` followed, in the same allocation, by pad_bytes of
    `fill`: reads past the tensor's end stay inside memory the test owns."""
    flat = torch.from_numpy(np.ascontiguousarray(arr).ravel())
    extra = pad_bytes // flat.element_size()
    buf = torch.full((flat.numel() + extra,), fill, dtype=flat.dtype, device=DEV)
    buf[:flat.numel()] = flat.to(DEV)
    return buf[:flat.numel()].view(arr.shape)


# Inputs followed by poison (NaN scales, 0x7F codes) with K tails in a later
# stage: the K tail of a tile's last row reads past the row's end, which the
# buffer range check turns into zeros; anything else would bring NaN into the
# FP32 sums (a zeroed activation-scale product times a NaN weight scale).  The
# big-tile shape stages scales 8 blocks at a time, so 13 blocks leave 3 past
# the end of its second scale stage (1 block: one stage; 7 blocks: two stages
# in one scale stage); the small-grid and GEMV shapes run too.
@pytest.mark.parametrize("m,n,k,path", [(1100, 7400, 416, bsr.PATH_GEMM), (1100, 7400, 32, bsr.PATH_GEMM),
                                        (1100, 7400, 224, bsr.PATH_GEMM), (1200, 7400, 416, bsr.PATH_GEMM),
                                        (1200, 7400, 32, bsr.PATH_GEMM), (1200, 7400, 224, bsr.PATH_GEMM),
                                        (300, 260, 160, bsr.PATH_GEMM),
                                        (40, 70, 160, bsr.PATH_AUTO), (8, 70, 416, bsr.PATH_AUTO),
                                        (8, 70, 160, bsr.PATH_INVARIANT), (20, 300, 224, bsr.PATH_INVARIANT)])
def test_tail_reads_ignore_bytes_past_buffers(m, n, k, path):
    say(f"poisoned tails m={m} n={n} k={k} path={path}")
    a, w, a_s, w_s = _rand_operands(m + n + k, m, n, k)
    out = canary_out(m, n)
    bsr.int8_gemm_blockscaled_ex(_padded(a, 0x7F), _padded(w, 0x7F), _padded(a_s, float("nan")),
                                 _padded(w_s, float("nan")), out, path=path)
    y, t = oracle.gemm_ref(a, w, a_s, w_s)
    _check(f"poisoned tails {m}x{n}x{k}", host(out), y, t, k)


@pytest.mark.parametrize("m", [1100, 1200])
def test_tail_reads_ignore_bytes_past_buffers_agroup(m):
    """The same with activation scales per 128 elements and per row on the big
    tiles (128 x 128 at m = 1100, 256 x 128 at m = 1200): K = 1152 is 36
    blocks, 9 stages, so the last 8-block scale stage holds 4 blocks past the
    end (one 128-element group past each row)."""
    n, k = 7400, 1152
    a, w, _, w_s = _rand_operands(77, m, n, k)
    rng = np.random.default_rng(78)
    rows = np.array([0, 127, 128, 255, 256, 1023, 1024, m - 1])
    for group in (128, 0):
        ng = 1 if group == 0 else k // group
        a_s = (rng.uniform(0.5, 2.0, size=(m, ng)) * 2.0 ** -8).astype(np.float32)
        say(f"poisoned tails, activation scale group {group}")
        out = canary_out(m, n)
        bsr.int8_gemm_blockscaled_agroup(_padded(a, 0x7F), _padded(w, 0x7F), _padded(a_s, float("nan")), group,
                                         _padded(w_s, float("nan")), out, path=bsr.PATH_GEMM)
        y, t = oracle.gemm_ref_agroup(a, w, a_s, w_s, group if group else k, rows=rows)
        _check(f"poisoned tails agroup {group}", host(out)[rows], y, t, k)
