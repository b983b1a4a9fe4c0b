"""The allocation-free GEMM entry point (int8_gemm_blockscaled_noalloc, the
library's static per-GPU scratch as K-split workspace) against the workspace
entry point int8_gemm_blockscaled_ws and the oracle, on calls in a row: a
split that fills the whole 8 MiB scratch, then a smaller one (over the first
call's leftover scratch contents), then a problem with no split."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_requant_amd import bsr
from gpu_util import DEV, canary_out, host, say, to_dev
from oracle.compare import check_bf16

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 8 << 20


def _operands(seed, m, n, k):
    rng = np.random.default_rng(seed)
    a = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    w = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    a_s = (rng.uniform(0.5, 2.0, size=(m, k // 32)) * 2.0 ** -8).astype(np.float32)
    w_s = (rng.uniform(0.5, 2.0, size=(n, k // 32)) * 2.0 ** -10).astype(np.float32)
    return a, w, a_s, w_s


def test_noalloc_equals_workspace_entry_point():
    cases = [(64, 4096, 14336), (40, 300, 8192), (300, 512, 1024)]
    needs = [bsr.int8_gemm_blockscaled_ws_bytes(*c) for c in cases]
    assert needs[0] == SCRATCH_BYTES and 0 < needs[1] < needs[0] and needs[2] == 0
    for (m, n, k), need in zip(cases, needs):
        say(f"no-alloc GEMM m={m} n={n} k={k}, split workspace {need} bytes")
        a, w, a_s, w_s = _operands(m + 7 * n + k, m, n, k)
        da, dw, das, dws = to_dev(a), to_dev(w), to_dev(a_s), to_dev(w_s)
        ws = torch.empty(need // 4, dtype=torch.float32, device=DEV) if need else None
        ref = canary_out(m, n)
        bsr.int8_gemm_blockscaled_ws(da, dw, das, dws, ref, ws)
        got = canary_out(m, n)
        bsr.int8_gemm_blockscaled_noalloc(da, dw, das, dws, got)
        ref_h, got_h = host(ref), host(got)
        assert np.array_equal(got_h, ref_h), f"{np.count_nonzero(got_h != ref_h)} outputs differ"
        y, t = oracle.gemm_ref(a, w, a_s, w_s)
        res = check_bf16(got_h, y, t, k)
        say(f"  {res}")
        assert res.ok, str(res)
