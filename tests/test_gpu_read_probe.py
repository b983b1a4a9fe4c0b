"""The streaming-read kernel bench.py reports as bandwidth context reads every
byte it is given: the XOR of its per-workgroup words equals the XOR of all
32-bit words of the buffer, for several grids and a size that is no multiple
of the grid's stride."""
import ctypes
import os

import numpy as np
import pytest
import torch

from block_scaled_precision_requant_amd import bsr
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("grid", [1, 7, 1024, 4096])
def test_read_probe_reads_every_word(grid):
    path = os.path.join(os.path.dirname(bsr.LIB_PATH), "libbsr_read.so")
    L = ctypes.CDLL(path)
    L.read_probe.restype = ctypes.c_int
    L.read_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]
    rng = np.random.default_rng(grid)
    nbytes = 16 * 262147  # not a multiple of 256 lanes x any grid here
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    out = torch.zeros(grid, dtype=torch.int32, device=DEV)
    assert L.read_probe(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()), grid,
                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host)
    say(f"read_probe grid={grid}: {got:#010x} vs {want:#010x}")
    assert got == want
