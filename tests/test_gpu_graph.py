"""The entry points inside a captured HIP graph: they launch kernels on the
given stream and nothing else (no allocation, no synchronisation, no memset),
so a graph of the prefill and of a decode step replays them.  Each replay
follows new inputs written in place, with eager work between the replays, and
must give the eager launches' bits."""
import numpy as np
import pytest
import torch

from block_scaled_precision_requant_amd import bsr, inputs
from gpu_util import DEV, gpu_requant_w, say, to_dev

pytestmark = pytest.mark.gpu


def _bf16(rng, m, k):
    return to_dev(inputs.bf16_normal(rng, m, k).view(np.int16))


def test_prefill_and_decode_replay_in_graph():
    rng = np.random.default_rng(91)
    m, md, n, k = 300, 8, 1000, 2048
    packed, e4m3 = inputs.nvfp4_weight(rng, n, k, -4, 2)
    w_i8, w_s = gpu_requant_w(packed, e4m3, inputs.SCALE2_1_448)
    wp, we = to_dev(packed), to_dev(e4m3)

    # graph-owned buffers: inputs written in place before each replay
    a = _bf16(rng, m, k)
    x = _bf16(rng, md, k)
    a_i8 = torch.empty((m, k), dtype=torch.int8, device=DEV)
    a_s = torch.empty((m, k // 32), dtype=torch.float32, device=DEV)
    x_i8 = torch.empty((md, k), dtype=torch.int8, device=DEV)
    x_s = torch.empty((md, k // 32), dtype=torch.float32, device=DEV)
    out = torch.empty((m, n), dtype=torch.int16, device=DEV)
    dec = torch.empty((md, n), dtype=torch.int16, device=DEV)
    w4 = torch.empty((md, n), dtype=torch.int16, device=DEV)

    def step():
        bsr.prefill(a, w_i8, w_s, a_i8, a_s, out)
        bsr.requant_a_int8(x, x_i8, x_s)
        bsr.int8_gemm_blockscaled(x_i8, w_i8, x_s, w_s, dec)  # GEMV
        bsr.w4a16_gemv(x, wp, we, float(inputs.SCALE2_1_448), w4)

    # warm up on a side stream (first calls cache the device check), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        a.copy_(_bf16(rng, m, k))
        x.copy_(_bf16(rng, md, k))
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (out, dec, w4, a_i8, a_s, x_i8, x_s)]
        # eager work between replays overwrites the same buffers, then restores the inputs' results
        out.zero_()
        dec.zero_()
        w4.zero_()
        step()
        torch.cuda.synchronize()
        want = (out, dec, w4, a_i8, a_s, x_i8, x_s)
        for i, (g, e) in enumerate(zip(got, want)):
            assert torch.equal(g.view(torch.int8), e.view(torch.int8)), f"replay {rep}, tensor {i}"
        say(f"graph replay {rep}: prefill, GEMV and W4A16 outputs equal the eager launches")


def test_split_k_and_noalloc_replay_in_graph():
    """The K-split GEMM through a caller workspace and through the allocation-free
    entry point's static scratch, captured in one graph (the no-alloc call is the
    one callers under capture use): four replays on new activations, each equal to
    eager launches of the same calls, bit for bit."""
    rng = np.random.default_rng(92)
    m, n, k = 64, 1024, 8192
    need = bsr.int8_gemm_blockscaled_ws_bytes(m, n, k)
    assert need > 0
    packed, e4m3 = inputs.nvfp4_weight(rng, n, k, -4, 2)
    w_i8, w_s = gpu_requant_w(packed, e4m3, inputs.SCALE2_1_448)
    a = _bf16(rng, m, k)
    a_i8 = torch.empty((m, k), dtype=torch.int8, device=DEV)
    a_s = torch.empty((m, k // 32), dtype=torch.float32, device=DEV)
    ws = torch.empty(need // 4, dtype=torch.float32, device=DEV)
    out_ws = torch.empty((m, n), dtype=torch.int16, device=DEV)
    out_na = torch.empty((m, n), dtype=torch.int16, device=DEV)

    def step():
        bsr.requant_a_int8(a, a_i8, a_s)
        bsr.int8_gemm_blockscaled_ws(a_i8, w_i8, a_s, w_s, out_ws, ws)
        bsr.int8_gemm_blockscaled_noalloc(a_i8, w_i8, a_s, w_s, out_na)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # first calls look up the device check and the scratch address
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        a.copy_(_bf16(rng, m, k))
        graph.replay()
        torch.cuda.synchronize()
        got = (out_ws.clone(), out_na.clone())
        out_ws.zero_()
        out_na.zero_()
        ws.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        assert torch.equal(got[0], out_ws) and torch.equal(got[1], out_na), f"replay {rep}"
        assert torch.equal(out_ws, out_na)
        say(f"graph replay {rep}: split-K GEMM (workspace and static scratch) equals the eager launches")


def test_big_grid_prefill_replays_in_graph():
    """A prefill on a grid of two 128 x 128 tiles per CU (the 256 x 128 tile) and
    one whose M a 256-row tiling would pad (the 128 x 128 tile), captured in one
    graph: three replays on new activations, each equal to eager launches."""
    rng = np.random.default_rng(93)
    n, k = 4096, 1024
    packed, e4m3 = inputs.nvfp4_weight(rng, n, k, -4, 2)
    w_i8, w_s = gpu_requant_w(packed, e4m3, inputs.SCALE2_1_448)
    bufs = []
    for m in (2048, 2112):
        bufs.append(dict(a=_bf16(rng, m, k), a_i8=torch.empty((m, k), dtype=torch.int8, device=DEV),
                         a_s=torch.empty((m, k // 32), dtype=torch.float32, device=DEV),
                         out=torch.empty((m, n), dtype=torch.int16, device=DEV)))

    def step():
        for b in bufs:
            bsr.prefill(b["a"], w_i8, w_s, b["a_i8"], b["a_s"], b["out"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for b in bufs:
            b["a"].copy_(_bf16(rng, b["a"].shape[0], k))
        graph.replay()
        torch.cuda.synchronize()
        got = [b["out"].clone() for b in bufs]
        for b in bufs:
            b["out"].zero_()
        step()
        torch.cuda.synchronize()
        for g, b in zip(got, bufs):
            assert torch.equal(g, b["out"]), f"replay {rep}, m = {b['out'].shape[0]}"
        say(f"graph replay {rep}: big-grid prefills equal the eager launches")
