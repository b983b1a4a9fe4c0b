"""A seeded sweep of random shapes through every GEMM entry point, each output
compared in full with the CPU oracle's FP64 reference (pass rule in
oracle/compare.py; outputs start as a NaN canary, so an element no launch wrote
fails).  The shapes fall in the row ranges the dispatch separates (the GEMV's
one 16-row tile, the streamed GEMV's up to four, the GEMM's small-grid K
groups, the 64 x 64 tiles, the workspace K split at long K), with ragged N and
any K that is a multiple of 32, so combinations no hand-picked case names are
covered too."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_requant_amd import bsr
from gpu_util import DEV, canary_out, host, say, to_dev
from oracle.compare import check_bf16

pytestmark = pytest.mark.gpu

ENTRIES = ("auto", "ws", "noalloc", "invariant", "gemm", "gemv", "agroup128", "agroup_row")


def _cases(seed=20240611, per_entry=12):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(per_entry * len(ENTRIES)):
        entry = ENTRIES[i % len(ENTRIES)]
        while True:
            band = int(rng.integers(0, 3))
            m = int((rng.integers(1, 17), rng.integers(17, 65), rng.integers(65, 301))[band])
            n = int(rng.integers(1, 2600))
            k = 32 * int(rng.integers(1, 301))
            if entry in ("ws", "noalloc") and (i // len(ENTRIES)) % 2 == 0:
                # long K at few tiles: where the K split applies
                m, n, k = int(rng.integers(33, 129)), int(rng.integers(64, 1200)), 32 * int(rng.integers(256, 301))
            if entry == "gemv":
                m = int(rng.integers(1, 65))
                if m > 16:
                    k = 256 * max(1, k // 256)
            if entry == "agroup128":
                k = 128 * max(1, k // 128)
            if m * n * k <= 6e8:
                break
        cases.append((i, entry, m, n, k))
    return cases


@pytest.mark.parametrize("i,entry,m,n,k", _cases(), ids=lambda v: str(v))
def test_sweep(i, entry, m, n, k):
    say(f"sweep case {i}: {entry} m={m} n={n} k={k}")
    rng = np.random.default_rng(1000 + i)
    a = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    w = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    group = {"agroup128": 128, "agroup_row": k}.get(entry, 32)
    a_s = (rng.uniform(0.5, 2.0, size=(m, k // group)) * 2.0 ** rng.integers(-12, -2, size=(m, k // group))
           ).astype(np.float32)
    w_s = (rng.uniform(0.5, 2.0, size=(n, k // 32)) * 2.0 ** rng.integers(-14, -4, size=(n, k // 32))
           ).astype(np.float32)
    a_s[rng.random(a_s.shape) < 0.03] = 0.0
    da, dw, das, dws = to_dev(a), to_dev(w), to_dev(a_s), to_dev(w_s)
    out = canary_out(m, n)
    if entry == "auto":
        bsr.int8_gemm_blockscaled(da, dw, das, dws, out)
    elif entry == "ws":
        need = bsr.int8_gemm_blockscaled_ws_bytes(m, n, k)
        ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device=DEV)
        say(f"  workspace {need} bytes")
        bsr.int8_gemm_blockscaled_ws(da, dw, das, dws, out, ws)
    elif entry == "noalloc":
        bsr.int8_gemm_blockscaled_noalloc(da, dw, das, dws, out)
    elif entry in ("invariant", "gemm", "gemv"):
        path = {"invariant": bsr.PATH_INVARIANT, "gemm": bsr.PATH_GEMM, "gemv": bsr.PATH_GEMV}[entry]
        bsr.int8_gemm_blockscaled_ex(da, dw, das, dws, out, path=path)
    else:
        bsr.int8_gemm_blockscaled_agroup(da, dw, das, 128 if entry == "agroup128" else 0, dws, out)
    got = host(out)
    if group == 32:
        y, t = oracle.gemm_ref(a, w, a_s, w_s)
    else:
        y, t = oracle.gemm_ref_agroup(a, w, a_s, w_s, group)
    res = check_bf16(got, y, t, k)
    say(f"  {res}")
    assert res.ok, f"case {i} {entry} {m}x{n}x{k}: {res}"
