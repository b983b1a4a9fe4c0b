"""The C-ABI library loads and exports every entry point include/bsr.h declares,
and argument validation answers before any GPU work (CPU only: no kernel runs)."""
import ctypes
import os
import re
import subprocess

import pytest

from block_scaled_precision_requant_amd import bsr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsr.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:BSR_API\s+)?(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))


def test_header_declares_the_entry_points():
    assert _declared_functions() == set(bsr.SIGNATURES)


def test_library_exports_exactly_the_declared_symbols():
    out = subprocess.run(["nm", "-D", "--defined-only", bsr.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    # every dynamic symbol the library defines is a declared entry point: no
    # internal launcher, helper or compiler-generated symbol leaks out
    assert exported == _declared_functions(), (exported ^ _declared_functions())
    L = bsr.lib()
    for name in _declared_functions():
        assert getattr(L, name) is not None


def test_status_strings():
    for st in range(6):
        assert bsr.status_string(st).startswith("BSR_")
    assert "unknown" in bsr.status_string(99)


FAKE = ctypes.c_void_p(1 << 20)       # never dereferenced: every call below fails validation first


def _fake(off=0):
    return ctypes.c_void_p((1 << 20) + off)


def test_bad_k_is_rejected_before_anything_else():
    L = bsr.lib()
    for k in (0, 16, 48, 33):
        assert L.requant_a_int8(FAKE, FAKE, FAKE, 4, k, None) == bsr.BSR_EINVAL
        assert L.requant_w_nvfp4_int8(FAKE, FAKE, 1.0, FAKE, FAKE, 4, k, None) == bsr.BSR_EINVAL
        assert L.int8_gemm_blockscaled(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, k, None) == bsr.BSR_EINVAL


def test_empty_problems_are_noops():
    L = bsr.lib()
    null = ctypes.c_void_p(0)
    assert L.requant_a_int8(null, null, null, 0, 64, None) == bsr.BSR_OK
    assert L.requant_w_nvfp4_int8(null, null, 1.0, null, null, 0, 64, None) == bsr.BSR_OK
    assert L.int8_gemm_blockscaled(null, null, null, null, null, 0, 7, 64, None) == bsr.BSR_OK
    assert L.int8_gemm_blockscaled(null, null, null, null, null, 7, 0, 64, None) == bsr.BSR_OK


def test_null_and_alignment_errors():
    L = bsr.lib()
    null = ctypes.c_void_p(0)
    assert L.requant_a_int8(null, FAKE, FAKE, 4, 64, None) == bsr.BSR_ENULL
    assert L.requant_a_int8(_fake(8), FAKE, FAKE, 4, 64, None) == bsr.BSR_EALIGN
    assert L.requant_a_int8(FAKE, FAKE, _fake(2), 4, 64, None) == bsr.BSR_EALIGN
    assert L.requant_w_nvfp4_int8(FAKE, _fake(1), 1.0, FAKE, FAKE, 4, 64, None) == bsr.BSR_EALIGN
    assert L.requant_w_nvfp4_int8(FAKE, FAKE, 1.0, null, FAKE, 4, 64, None) == bsr.BSR_ENULL
    assert L.int8_gemm_blockscaled(FAKE, _fake(4), FAKE, FAKE, FAKE, 4, 4, 64, None) == bsr.BSR_EALIGN
    assert L.int8_gemm_blockscaled(FAKE, FAKE, FAKE, FAKE, _fake(1), 4, 4, 64, None) == bsr.BSR_EALIGN
    assert L.int8_gemm_blockscaled(FAKE, FAKE, FAKE, FAKE, null, 4, 4, 64, None) == bsr.BSR_ENULL


def test_silu_requant_validation():
    L = bsr.lib()
    null = ctypes.c_void_p(0)
    assert L.silu_mul_requant_int8(FAKE, FAKE, 64, FAKE, FAKE, 4, 48, None) == bsr.BSR_EINVAL   # k
    assert L.silu_mul_requant_int8(FAKE, FAKE, 32, FAKE, FAKE, 4, 64, None) == bsr.BSR_EINVAL   # ld < k
    assert L.silu_mul_requant_int8(FAKE, FAKE, 68, FAKE, FAKE, 4, 64, None) == bsr.BSR_EINVAL   # ld % 8
    assert L.silu_mul_requant_int8(FAKE, FAKE, 64, FAKE, FAKE, 0, 64, None) == bsr.BSR_OK       # empty
    assert L.silu_mul_requant_int8(null, FAKE, 64, FAKE, FAKE, 4, 64, None) == bsr.BSR_ENULL
    assert L.silu_mul_requant_int8(FAKE, _fake(8), 64, FAKE, FAKE, 4, 64, None) == bsr.BSR_EALIGN
    assert L.silu_mul_requant_int8(FAKE, FAKE, 64, FAKE, _fake(2), 4, 64, None) == bsr.BSR_EALIGN


def test_w4a16_validation():
    L = bsr.lib()
    null = ctypes.c_void_p(0)
    assert L.w4a16_gemv(FAKE, FAKE, FAKE, 1.0, FAKE, 17, 4, 256, None) == bsr.BSR_EINVAL   # m > 16
    assert L.w4a16_gemv(FAKE, FAKE, FAKE, 1.0, FAKE, 1, 4, 48, None) == bsr.BSR_EINVAL     # k
    assert L.w4a16_gemv(FAKE, FAKE, FAKE, float("nan"), FAKE, 1, 4, 256, None) == bsr.BSR_EINVAL
    assert L.w4a16_gemv(FAKE, FAKE, FAKE, 1.0, FAKE, 0, 4, 256, None) == bsr.BSR_OK
    assert L.w4a16_gemv(null, FAKE, FAKE, 1.0, FAKE, 1, 4, 256, None) == bsr.BSR_ENULL
    assert L.w4a16_gemv(FAKE, FAKE, _fake(2), 1.0, FAKE, 1, 4, 256, None) == bsr.BSR_EALIGN  # k % 256 == 0
    assert L.w4a16_gemv(FAKE, _fake(8), FAKE, 1.0, FAKE, 1, 4, 96, None) == bsr.BSR_EALIGN


def test_bad_scale2_and_path():
    L = bsr.lib()
    for s2 in (float("nan"), float("inf"), -float("inf")):
        assert L.requant_w_nvfp4_int8(FAKE, FAKE, s2, FAKE, FAKE, 4, 64, None) == bsr.BSR_EINVAL
    assert L.int8_gemm_blockscaled_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 64, None, 4) == bsr.BSR_EINVAL
    assert L.int8_gemm_blockscaled_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 64, None, -1) == bsr.BSR_EINVAL
    assert L.int8_gemm_blockscaled_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 17, 4, 64, None,
                                      bsr.PATH_GEMV) == bsr.BSR_EINVAL  # m > 16, k % 256 != 0
    assert L.int8_gemm_blockscaled_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 65, 4, 256, None,
                                      bsr.PATH_GEMV) == bsr.BSR_EINVAL  # m > 64
    assert L.int8_gemm_blockscaled_ex(None, FAKE, FAKE, FAKE, FAKE, 64, 4, 256, None,
                                      bsr.PATH_GEMV) == bsr.BSR_ENULL   # m <= 64, k % 256 == 0: accepted


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU may be present")
def test_no_device_is_reported():
    L = bsr.lib()
    assert L.requant_a_int8(FAKE, FAKE, FAKE, 4, 64, None) == bsr.BSR_EDEVICE


def test_quantize_act_validation():
    L = bsr.lib()
    null = None
    assert L.quantize_act(FAKE, FAKE, FAKE, 4, 48, 32, 0, None) == bsr.BSR_EINVAL     # k
    assert L.quantize_act(FAKE, FAKE, FAKE, 4, 96, 128, 0, None) == bsr.BSR_EINVAL    # k % 128
    assert L.quantize_act(FAKE, FAKE, FAKE, 4, 128, 64, 0, None) == bsr.BSR_EINVAL    # group
    assert L.quantize_act(FAKE, FAKE, FAKE, 4, 128, 32, 2, None) == bsr.BSR_EINVAL    # format
    assert L.quantize_act(FAKE, FAKE, FAKE, 0, 128, 0, 1, None) == bsr.BSR_OK         # empty
    assert L.quantize_act(null, FAKE, FAKE, 4, 128, 0, 1, None) == bsr.BSR_ENULL
    assert L.quantize_act(FAKE, _fake(4), FAKE, 4, 128, 0, 1, None) == bsr.BSR_EALIGN
    assert L.quantize_act(_fake(8), FAKE, FAKE, 4, 128, 32, 0, None) == bsr.BSR_EALIGN


def test_gemm_agroup_validation():
    L = bsr.lib()
    args = (FAKE, FAKE, FAKE)
    assert L.int8_gemm_blockscaled_agroup(*args, 64, FAKE, FAKE, 4, 4, 128, None, 0) == bsr.BSR_EINVAL
    assert L.int8_gemm_blockscaled_agroup(*args, 128, FAKE, FAKE, 4, 4, 96, None, 0) == bsr.BSR_EINVAL
    assert L.int8_gemm_blockscaled_agroup(*args, 0, FAKE, FAKE, 4, 4, 48, None, 0) == bsr.BSR_EINVAL
    assert L.int8_gemm_blockscaled_agroup(*args, 0, FAKE, FAKE, 17, 4, 96, None, 2) == bsr.BSR_EINVAL  # gemv m>16
    assert L.int8_gemm_blockscaled_agroup(*args, 0, FAKE, FAKE, 65, 4, 256, None, 2) == bsr.BSR_EINVAL  # gemv m>64
    assert L.int8_gemm_blockscaled_agroup(*args, 0, FAKE, FAKE, 4, 4, 96, None, 7) == bsr.BSR_EINVAL  # path
    assert L.int8_gemm_blockscaled_agroup(*args, 128, FAKE, FAKE, 0, 4, 256, None, 0) == bsr.BSR_OK
    assert L.int8_gemm_blockscaled_agroup(FAKE, FAKE, None, 128, FAKE, FAKE, 4, 4, 256, None, 0) == bsr.BSR_ENULL
    assert L.int8_gemm_blockscaled_agroup(FAKE, FAKE, _fake(2), 0, FAKE, FAKE, 4, 4, 256, None, 0) == bsr.BSR_EALIGN


def test_binding_rejects_wrong_element_types():
    """The binding checks each argument's element type before anything reaches the
    library: a 1-byte output where BF16 is written, or 16-bit scales where binary32
    scales are read, would make a kernel access memory past the tensor's end."""
    import torch
    m, n, k = 4, 8, 64
    a = torch.zeros((m, k), dtype=torch.int8)
    w = torch.zeros((n, k), dtype=torch.int8)
    a_s = torch.zeros((m, k // 32), dtype=torch.float32)
    w_s = torch.zeros((n, k // 32), dtype=torch.float32)
    out = torch.zeros((m, n), dtype=torch.int16)
    bad_cases = [
        (dict(out=torch.zeros((m, n), dtype=torch.uint8)), "out"),
        (dict(a_scale=torch.zeros((m, k // 32), dtype=torch.bfloat16)), "a_scale"),
        (dict(w_scale=torch.zeros((n, k // 32), dtype=torch.float64)), "w_scale"),
        (dict(a_i8=torch.zeros((m, k), dtype=torch.int16)), "a_i8"),
    ]
    for change, what in bad_cases:
        args = dict(a_i8=a, w_i8=w, a_scale=a_s, w_scale=w_s, out=out)
        args.update(change)
        with pytest.raises(ValueError, match=f"{what}: dtype"):
            bsr.int8_gemm_blockscaled(**args)
    with pytest.raises(ValueError, match="a_scale: dtype"):
        bsr.requant_a_int8(torch.zeros((m, k), dtype=torch.bfloat16), a,
                           torch.zeros((m, k // 32), dtype=torch.float16))
    with pytest.raises(ValueError, match="w_scale: dtype"):
        bsr.requant_w_nvfp4_int8(torch.zeros((n, k // 2), dtype=torch.uint8),
                                 torch.zeros((n, k // 16), dtype=torch.uint8), 1.0, w,
                                 torch.zeros((n, k // 32), dtype=torch.int32))
    with pytest.raises(ValueError, match="out: dtype"):
        bsr.w4a16_gemv(torch.zeros((m, k), dtype=torch.bfloat16), torch.zeros((n, k // 2), dtype=torch.uint8),
                       torch.zeros((n, k // 16), dtype=torch.uint8), 1.0, torch.zeros((m, n), dtype=torch.float32))
    # the right element types pass the checks and stop only at the device check
    with pytest.raises(ValueError, match="device tensor"):
        bsr.int8_gemm_blockscaled(a, w, a_s, w_s, out)


def test_gemm_k_limit():
    """The GEMM (m > 16, or the GEMM path forced) needs k < 2^25: its staging
    addresses a tile's 128 rows with 32-bit offsets.  The GEMV (m <= 16) has no
    such limit, so there validation passes and only the device check answers."""
    L = bsr.lib()
    k = 1 << 25
    assert L.int8_gemm_blockscaled(FAKE, FAKE, FAKE, FAKE, FAKE, 17, 8, k, None) == bsr.BSR_EINVAL
    assert L.int8_gemm_blockscaled_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, k, None, bsr.PATH_GEMM) == bsr.BSR_EINVAL
    assert L.int8_gemm_blockscaled_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 40, 8, k, None, bsr.PATH_INVARIANT) == \
        bsr.BSR_EINVAL
    assert L.int8_gemm_blockscaled(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, k, None) != bsr.BSR_EINVAL
    assert L.int8_gemm_blockscaled(FAKE, FAKE, FAKE, FAKE, FAKE, 17, 8, k - 32, None) != bsr.BSR_EINVAL


def test_read_probe_library_exports_one_symbol():
    """The bandwidth-context read kernel (bench.py) lives in a library of its own
    that defines read_probe and nothing else; invalid arguments are refused
    before any launch."""
    path = os.path.join(os.path.dirname(bsr.LIB_PATH), "libbsr_read.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    assert {line.split()[-1] for line in out.splitlines() if line.strip()} == {"read_probe"}
    L = ctypes.CDLL(path)
    L.read_probe.restype = ctypes.c_int
    L.read_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]
    assert L.read_probe(None, 16, FAKE, 1, None) == 1           # null buffer
    assert L.read_probe(FAKE, 15, FAKE, 1, None) == 1           # not whole 16-byte words
    assert L.read_probe(FAKE, 16, FAKE, 0, None) == 1           # empty grid
