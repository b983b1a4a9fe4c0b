"""GPU parity of the fused SiLU·mul -> int8 per-32 requant against the CPU
oracle: bit-exact codes and scales (the quantizer is exact; the SiLU uses the
binary32 rounding of a binary64 exp on both sides, pinned on the CPU)."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_requant_amd import bsr, inputs
from gpu_util import DEV, gpu_requant_a, gpu_silu_requant, host, say, to_dev

pytestmark = pytest.mark.gpu


def _same(name, q, s, q_ref, s_ref):
    bad_q = int(np.sum(q != q_ref))
    bad_s = int(np.sum(s.view(np.uint32) != s_ref.view(np.uint32)))
    say(f"{name}: {q.size} codes, {bad_q} differ; {s.size} scales, {bad_s} differ")
    assert bad_q == 0 and bad_s == 0


# 128 x 512 runs the per-element kernel.  The LDS-table kernel takes inputs with
# at least 256 x 4096 chunks of 8 elements: 2048 x 4096 is exactly that (256
# persistent workgroups, 8 whole passes), 2049 x 4160 (1 065 480 chunks, 261
# workgroups) ends in a ragged pass; both hit the closed-form ranges and every
# table entry.
@pytest.mark.parametrize("m,k", [(128, 512), (2048, 4096), (2049, 4160)])
def test_every_finite_bf16_gate(m, k):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]
    rng = np.random.default_rng(1)
    fill = rng.choice(bits, size=m * k - bits.size)
    gate = rng.permutation(np.concatenate([bits, fill])).reshape(m, k)
    assert np.unique(gate).size == bits.size
    # |up| <= 1/2 keeps silu(g) * up finite in BF16 for the largest gates
    up = inputs.f32_to_bf16_bits(np.random.default_rng(2).uniform(-0.5, 0.5, (m, k)).astype(np.float32))
    q_ref, s_ref = oracle.silu_mul_requant(gate, up)
    q, s = gpu_silu_requant(gate, up)
    _same(f"all BF16 gates {m}x{k}", host(q), host(s), q_ref, s_ref)


@pytest.mark.parametrize("m,k", [(1, 32), (3, 96), (7, 2080), (129, 1024)])
def test_random_shapes(m, k):
    rng = np.random.default_rng(m * 1000 + k)
    gate = inputs.bf16_normal(rng, m, k, scale=3.0)
    up = inputs.bf16_normal(rng, m, k)
    q_ref, s_ref = oracle.silu_mul_requant(gate, up)
    q, s = gpu_silu_requant(gate, up)
    _same(f"{m}x{k}", host(q), host(s), q_ref, s_ref)


def test_workload_full():
    src = inputs.silu_mul_input()
    say(f"silu workload {src.m}x{src.k}")
    gate, up = src.gate(), src.up()
    q_ref, s_ref = oracle.silu_mul_requant(gate, up)
    q, s = gpu_silu_requant(gate, up)
    _same("ffn_down_input", host(q), host(s), q_ref, s_ref)


@pytest.mark.parametrize("m,k", [(37, 640), (512, 8192), (1100, 8192)])   # the last on the table kernel
def test_halves_of_one_buffer(m, k):
    # gate and up as the two halves of one [m, 2k] gate+up output (row pitch 2k)
    rng = np.random.default_rng(9)
    both = inputs.bf16_normal(rng, m, 2 * k, scale=2.0)
    q_ref, s_ref = oracle.silu_mul_requant(both[:, :k].copy(), both[:, k:].copy())
    d = to_dev(both.view(np.int16))
    q = torch.empty((m, k), dtype=torch.int8, device=DEV)
    s = torch.empty((m, k // 32), dtype=torch.float32, device=DEV)
    bsr.silu_mul_requant_int8(d[:, :k], d[:, k:], q, s)
    _same("halves", host(q), host(s), q_ref, s_ref)


def test_equals_requant_of_the_bf16_product():
    # the fused step is the activation requant of h = bf16(silu(g) * u)
    rng = np.random.default_rng(21)
    m, k = 8, 1024
    gate = inputs.bf16_normal(rng, m, k, scale=2.0)
    up = inputs.bf16_normal(rng, m, k)
    gf = (gate.astype(np.uint32) << 16).view(np.float32)
    uf = (up.astype(np.uint32) << 16).view(np.float32)
    h = np.array([[oracle.silu_mul(float(a), float(b)) for a, b in zip(ra, rb)] for ra, rb in zip(gf, uf)],
                 np.float32)
    h_bits = (h.view(np.uint32) >> 16).astype(np.uint16)
    q1, s1 = gpu_silu_requant(gate, up)
    q2, s2 = gpu_requant_a(h_bits)
    _same("fused vs chain", host(q1), host(s1), host(q2), host(s2))


def test_errors_launch_nothing():
    g = torch.zeros((4, 64), dtype=torch.int16, device=DEV)
    q = torch.full((4, 64), 5, dtype=torch.int8, device=DEV)
    s = torch.full((4, 2), 7.0, dtype=torch.float32, device=DEV)
    L = bsr.lib()
    st = L.silu_mul_requant_int8(g.data_ptr(), g.data_ptr(), 32, q.data_ptr(), s.data_ptr(), 4, 64, None)
    assert st == bsr.BSR_EINVAL                              # ld < k
    st = L.silu_mul_requant_int8(g.data_ptr(), g.data_ptr(), 68, q.data_ptr(), s.data_ptr(), 4, 64, None)
    assert st == bsr.BSR_EINVAL                              # ld not a multiple of 8
    st = L.silu_mul_requant_int8(g.data_ptr(), g.data_ptr(), 64, q.data_ptr(), s.data_ptr(), 4, 48, None)
    assert st == bsr.BSR_EINVAL                              # k
    st = L.silu_mul_requant_int8(g.data_ptr() + 2, g.data_ptr(), 64, q.data_ptr(), s.data_ptr(), 4, 64, None)
    assert st == bsr.BSR_EALIGN
    assert L.silu_mul_requant_int8(g.data_ptr(), g.data_ptr(), 64, q.data_ptr(), s.data_ptr(), 0, 64, None) == 0
    torch.cuda.synchronize()
    assert bool((q == 5).all()) and bool((s == 7.0).all())
