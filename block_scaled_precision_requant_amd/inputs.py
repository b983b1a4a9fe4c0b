"""Seeded synthetic inputs for the block-scaled int8 projection.

This module holds no step of the method: it only draws random bits in the
formats the method reads (BF16 activations, packed E2M1 nibbles, E4M3 block
scale codes, a binary32 ``scale2``).  Both the GPU path and the CPU oracle take
their inputs from here, so the two always see identical bytes.

Every tensor comes from ``numpy.random.default_rng([seed, tensor_id])`` (PCG64),
so each can be regenerated on its own.  Recipes:

* BF16 activations: a float32 draw rounded to BF16 (round-to-nearest-even,
  torch's conversion), returned as raw uint16 bits.
* NVFP4 weight: packed bytes uniform on 0..255 (both nibbles uniform on 0..15,
  codes 8 = -0 included; element 2j is the low nibble of byte j), E4M3 block
  scale codes ``(e + 7) << 3`` (the value 2^e) with e uniform on a stated range,
  and a binary32 per-tensor ``scale2``.
"""
from dataclasses import dataclass, field

import numpy as np
import torch

SCALE2_1_64 = np.float32(1.0 / 64.0)
SCALE2_1_448 = np.float32(1.0) / np.float32(448.0)


def rng_for(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tensor_id)])


def f32_to_bf16_bits(x) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_normal(rng, m, k, scale=1.0):
    return f32_to_bf16_bits(scale * rng.standard_normal((m, k), dtype=np.float32))


def bf16_student_t(rng, m, k, nu=4.0, scale=0.5):
    return f32_to_bf16_bits((scale * rng.standard_t(nu, size=(m, k))).astype(np.float32))


def bf16_normal_outlier_columns(rng, m, k, fraction=0.001, factor=100.0):
    """N(0,1) with round(fraction*K) fixed random columns scaled by `factor` in FP32."""
    x = rng.standard_normal((m, k), dtype=np.float32)
    ncols = int(round(fraction * k))
    cols = np.sort(rng.choice(k, size=ncols, replace=False))
    x[:, cols] *= np.float32(factor)
    return f32_to_bf16_bits(x), cols


def nvfp4_weight(rng, n, k, e_lo, e_hi):
    """(w_packed [n, k/2] uint8, w_e4m3 [n, k/16] uint8) with scales 2^U{e_lo..e_hi}."""
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    e = rng.integers(e_lo, e_hi + 1, size=(n, k // 16))
    codes = ((e + 7) << 3).astype(np.uint8)
    return packed, codes


@dataclass
class Projection:
    """One projection Y[M,N] = A[M,K] W[N,K]^T of a workload."""
    name: str
    m: int
    n: int
    k: int
    seed: int
    a_kind: str            # "normal", "student_t", "outlier_cols"
    e_range: tuple         # E4M3 block-scale exponent range of W
    scale2: np.float32
    tensor_base: int = 0   # keeps tensor ids of the projections of one workload apart

    def weight(self):
        return nvfp4_weight(rng_for(self.seed, self.tensor_base + 1), self.n, self.k, *self.e_range)

    def activations(self, m=None):
        m = self.m if m is None else m
        rng = rng_for(self.seed, self.tensor_base + 2)
        if self.a_kind == "normal":
            return bf16_normal(rng, m, self.k)
        if self.a_kind == "student_t":
            return bf16_student_t(rng, m, self.k)
        if self.a_kind == "outlier_cols":
            return bf16_normal_outlier_columns(rng, m, self.k)[0]
        raise ValueError(self.a_kind)


@dataclass
class Workload:
    name: str
    description: str
    projections: list = field(default_factory=list)


def workloads():
    """The five synthetic workloads, smallest first."""
    w = []
    w.append(Workload("tiny", "M=16 N=256 K=512, A ~ N(0,1), W scales 2^U{-4..2}, scale2 = 1/64",
                      [Projection("tiny", 16, 256, 512, 0, "normal", (-4, 2), SCALE2_1_64)]))
    w.append(Workload("attn_proj", "prefill attention projection M=2048 N=4096 K=4096, A ~ N(0,1), "
                      "W scales 2^U{-4..2}, scale2 = fl32(1/448)",
                      [Projection("attn_proj", 2048, 4096, 4096, 1, "normal", (-4, 2), SCALE2_1_448)]))
    w.append(Workload("dense_ffn", "prefill dense FFN M=4096: stacked gate+up N=28672 K=4096, down N=4096 "
                      "K=14336; A = 0.5 * Student-t(4), one draw per projection",
                      [Projection("gate_up", 4096, 28672, 4096, 2, "student_t", (-4, 2), SCALE2_1_448, 0),
                       Projection("down", 4096, 4096, 14336, 2, "student_t", (-4, 2), SCALE2_1_448, 10)]))
    dec = []
    for mm in (1, 2, 4, 8):
        dec.append(Projection(f"decode_m{mm}_n14336_k4096", mm, 14336, 4096, 3, "normal", (-4, 2),
                              SCALE2_1_448, 0))
        dec.append(Projection(f"decode_m{mm}_n4096_k14336", mm, 4096, 14336, 3, "normal", (-4, 2),
                              SCALE2_1_448, 10))
    w.append(Workload("decode", "decode GEMV M in {1,2,4,8} x (N=14336,K=4096), (N=4096,K=14336)", dec))
    w.append(Workload("large", "large prefill M=8192 N=28672 K=8192, A ~ N(0,1) with 8 fixed columns x100, "
                      "W scales 2^U{-6..4}, scale2 = fl32(1/448)",
                      [Projection("large", 8192, 28672, 8192, 4, "outlier_cols", (-6, 4), SCALE2_1_448)]))
    return w


@dataclass
class SiluMulInput:
    """The down projection's input before quantization: the gate and up halves
    [M, I] of a gate+up GEMM output, as BF16 bits (gate ~ N(0, gate_scale^2),
    up ~ N(0, 1), independent draws)."""
    name: str
    m: int
    k: int
    seed: int
    tensor_base: int
    gate_scale: float = 2.0

    def gate(self, m=None):
        m = self.m if m is None else m
        return bf16_normal(rng_for(self.seed, self.tensor_base + 1), m, self.k, scale=self.gate_scale)

    def up(self, m=None):
        m = self.m if m is None else m
        return bf16_normal(rng_for(self.seed, self.tensor_base + 2), m, self.k)


def silu_mul_input():
    """SiLU product feeding the dense FFN's down projection: M=4096, I=14336."""
    return SiluMulInput("ffn_down_input", 4096, 14336, 2, 20)


def workload(name):
    for w in workloads():
        if w.name == name:
            return w
    raise KeyError(name)
