"""Calls on two streams at once: the entry points keep no state between calls
apart from a per-device cache of the device check, so two independent
pipelines enqueued on two streams and left to overlap on the GPU give the bits
each gives run alone.  (The allocation-free GEMM entry point is the exception
its header names: its calls share one scratch buffer per GPU, so it is not
run here.)"""
import numpy as np
import pytest
import torch

from block_scaled_precision_requant_amd import bsr, inputs
from gpu_util import DEV, host, say, to_dev

pytestmark = pytest.mark.gpu


def _bf16(rng, m, k):
    return to_dev(inputs.bf16_normal(rng, m, k).view(np.int16))


class _Pipeline:
    """One stream's work: a weight requant, a big-grid prefill (256 x 128 tiles),
    a small-grid GEMM, a K-split GEMM into its own workspace, a decode GEMV, a
    W4A16 GEMV and a SiLU quantizer -- each on its own buffers."""

    def __init__(self, seed):
        rng = np.random.default_rng(seed)
        self.n, self.k = 4096, 4096
        packed, e4m3 = inputs.nvfp4_weight(rng, self.n, self.k, -4, 2)
        self.wp, self.we = to_dev(packed), to_dev(e4m3)
        self.a = _bf16(rng, 2048, self.k)
        self.a_small = _bf16(rng, 300, self.k)
        self.x = _bf16(rng, 8, self.k)
        self.gate, self.up = _bf16(rng, 512, self.k), _bf16(rng, 512, self.k)
        pk, ek = inputs.nvfp4_weight(rng, 1024, 14336, -4, 2)
        self.wp_long, self.we_long = to_dev(pk), to_dev(ek)
        self.a_long = _bf16(rng, 64, 14336)
        self.ws = torch.empty(bsr.int8_gemm_blockscaled_ws_bytes(64, 1024, 14336) // 4 + 4, dtype=torch.float32,
                              device=DEV)
        assert self.ws.numel() > 4, "the long-K shape splits K"

    def run(self, stream):
        n, k = self.n, self.k
        e = lambda *s, dt: torch.empty(s, dtype=dt, device=DEV)  # noqa: E731
        r = {}
        with torch.cuda.stream(stream):
            w_i8, w_s = e(n, k, dt=torch.int8), e(n, k // 32, dt=torch.float32)
            bsr.requant_w_nvfp4_int8(self.wp, self.we, float(inputs.SCALE2_1_448), w_i8, w_s)
            a_i8, a_s = e(2048, k, dt=torch.int8), e(2048, k // 32, dt=torch.float32)
            r["prefill"] = e(2048, n, dt=torch.int16)
            bsr.prefill(self.a, w_i8, w_s, a_i8, a_s, r["prefill"])
            s_i8, s_s = e(300, k, dt=torch.int8), e(300, k // 32, dt=torch.float32)
            r["small"] = e(300, n, dt=torch.int16)
            bsr.prefill(self.a_small, w_i8, w_s, s_i8, s_s, r["small"])
            wl_i8, wl_s = e(1024, 14336, dt=torch.int8), e(1024, 14336 // 32, dt=torch.float32)
            bsr.requant_w_nvfp4_int8(self.wp_long, self.we_long, float(inputs.SCALE2_1_448), wl_i8, wl_s)
            l_i8, l_s = e(64, 14336, dt=torch.int8), e(64, 14336 // 32, dt=torch.float32)
            bsr.requant_a_int8(self.a_long, l_i8, l_s)
            r["split"] = e(64, 1024, dt=torch.int16)
            bsr.int8_gemm_blockscaled_ws(l_i8, wl_i8, l_s, wl_s, r["split"], self.ws)
            x_i8, x_s = e(8, k, dt=torch.int8), e(8, k // 32, dt=torch.float32)
            bsr.requant_a_int8(self.x, x_i8, x_s)
            r["gemv"] = e(8, n, dt=torch.int16)
            bsr.int8_gemm_blockscaled(x_i8, w_i8, x_s, w_s, r["gemv"])
            r["w4a16"] = e(8, n, dt=torch.int16)
            bsr.w4a16_gemv(self.x, self.wp, self.we, float(inputs.SCALE2_1_448), r["w4a16"])
            q, qs = e(512, k, dt=torch.int8), e(512, k // 32, dt=torch.float32)
            bsr.silu_mul_requant_int8(self.gate, self.up, q, qs)
            r["silu_q"], r["silu_s"] = q, qs
        return r


def test_two_streams_overlapping_give_the_bits_of_each_alone():
    p0, p1 = _Pipeline(201), _Pipeline(202)
    torch.cuda.synchronize()  # inputs were copied in on the default stream
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    # alone, one after the other
    alone0 = {k: host(v) for k, v in p0.run(s0).items()}
    torch.cuda.synchronize()
    alone1 = {k: host(v) for k, v in p1.run(s1).items()}
    torch.cuda.synchronize()
    for rep in range(3):
        # both enqueued before either is waited for, so their kernels overlap
        r0 = p0.run(s0)
        r1 = p1.run(s1)
        torch.cuda.synchronize()
        for name in alone0:
            say(f"rep {rep}: {name}")
            assert np.array_equal(host(r0[name]), alone0[name]), ("stream 0", rep, name)
            assert np.array_equal(host(r1[name]), alone1[name]), ("stream 1", rep, name)
