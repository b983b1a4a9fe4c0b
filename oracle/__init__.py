"""CPU oracle of the block-scaled int8 projection -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library and never takes a value
the GPU produced as input.

The arithmetic lives in plain C (``bsr_oracle.c``); this module only marshals
numpy arrays through ctypes.  Functions and what they follow (page
"metrale_model_layers/layers/ops/gemm_dense_int8.rs"):

* ``requant_w``   -- doc of ``requant_w_nvfp4_int8``: NVFP4 (packed E2M1, E4M3
  per 16, F32 scale2) -> int8 ``[N,K]`` + F32 ``[N,K/32]``.
* ``requant_a``   -- doc of ``int8_gemm_faith2_prefill``, first launch: BF16
  ``[M,K]`` -> int8 + F32 per 32.
* ``block_partials`` -- the exact int32 dot product of each 32-wide K block.
* ``gemm_ref``    -- FP64 sum over blocks of a_s * w_s * P (and the sum of the
  terms' magnitudes, which the FP32 error bound scales with).

Every function is pinned by tests that do not re-use this code (format tables
from the OCP specs, torch's E4M3 and BF16 conversions, an exact-rational
quantizer, numpy integer/FP64 matmuls, power-of-two exact GEMMs).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i8p = ctypes.POINTER(ctypes.c_int8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def lib():
    """Load oracle/liboracle.so, compiling it first only if it is absent."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.orc_e2m1_value.restype = ctypes.c_float
        L.orc_e2m1_value.argtypes = [ctypes.c_uint32]
        L.orc_e4m3_value.restype = ctypes.c_float
        L.orc_e4m3_value.argtypes = [ctypes.c_uint32]
        L.orc_requant_w.restype = ctypes.c_int
        L.orc_requant_w.argtypes = [_u8p, _u8p, ctypes.c_float, _i8p, _f32p, _i64, _i64]
        L.orc_requant_a.restype = ctypes.c_int
        L.orc_requant_a.argtypes = [_u16p, _i8p, _f32p, _i64, _i64]
        L.orc_bf16_round.restype = ctypes.c_float
        L.orc_bf16_round.argtypes = [ctypes.c_float]
        L.orc_exp_neg_f32.restype = ctypes.c_float
        L.orc_exp_neg_f32.argtypes = [ctypes.c_float]
        L.orc_silu_mul.restype = ctypes.c_float
        L.orc_silu_mul.argtypes = [ctypes.c_float, ctypes.c_float]
        L.orc_silu_mul_requant.restype = ctypes.c_int
        L.orc_silu_mul_requant.argtypes = [_u16p, _u16p, _i64, _i8p, _f32p, _i64, _i64]
        L.orc_block_partials.restype = ctypes.c_int
        L.orc_block_partials.argtypes = [_i8p, _i8p, _i32p, _i64, _i64, _i64]
        L.orc_gemm_ref.restype = ctypes.c_int
        L.orc_gemm_ref.argtypes = [_i8p, _i8p, _f32p, _f32p, _i64p, _i64, _f64p, _f64p, _i64, _i64]
        L.orc_e4m3_encode.restype = ctypes.c_uint32
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_quant_act.restype = ctypes.c_int
        L.orc_quant_act.argtypes = [_u16p, _u8p, _f32p, _i64, _i64, _i64, ctypes.c_int]
        L.orc_gemm_ref_agroup.restype = ctypes.c_int
        L.orc_gemm_ref_agroup.argtypes = [_i8p, _i8p, _f32p, _f32p, _i64p, _i64, _f64p, _f64p, _i64, _i64, _i64]
        L.orc_w4a16_ref.restype = ctypes.c_int
        L.orc_w4a16_ref.argtypes = [_u16p, _u8p, _u8p, ctypes.c_float, _i64p, _i64, _f64p, _f64p, _i64, _i64]
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [ctypes.c_int]
        _LIB = L
    return _LIB


def _ptr(a, t):
    return a.ctypes.data_as(t)


def _check(rc, what):
    if rc == -1:
        raise ValueError(f"{what}: k must be a positive multiple of 32")
    if rc == -2:
        raise ValueError(f"{what}: non-finite input or dequantized value (outside the contract)")
    if rc != 0:
        raise RuntimeError(f"{what}: status {rc}")


def e2m1_value(code: int) -> float:
    return float(lib().orc_e2m1_value(code))


def e4m3_value(code: int) -> float:
    return float(lib().orc_e4m3_value(code))


def requant_w(w_packed, w_e4m3, scale2):
    """NVFP4 weight -> (w_i8 [N,K] int8, w_scale [N,K/32] float32)."""
    w_packed = np.ascontiguousarray(w_packed, dtype=np.uint8)
    w_e4m3 = np.ascontiguousarray(w_e4m3, dtype=np.uint8)
    n, half_k = w_packed.shape
    k = 2 * half_k
    if w_e4m3.shape != (n, k // 16):
        raise ValueError(f"w_e4m3 shape {w_e4m3.shape} != {(n, k // 16)}")
    w_i8 = np.empty((n, k), np.int8)
    w_scale = np.empty((n, k // 32), np.float32)
    rc = lib().orc_requant_w(_ptr(w_packed, _u8p), _ptr(w_e4m3, _u8p), float(np.float32(scale2)),
                             _ptr(w_i8, _i8p), _ptr(w_scale, _f32p), n, k)
    _check(rc, "requant_w")
    return w_i8, w_scale


def requant_a(a_bf16_bits):
    """BF16 activations (raw uint16 bits) -> (a_i8 [M,K] int8, a_scale [M,K/32] float32)."""
    a = np.ascontiguousarray(a_bf16_bits, dtype=np.uint16)
    m, k = a.shape
    a_i8 = np.empty((m, k), np.int8)
    a_scale = np.empty((m, max(k // 32, 0)), np.float32)
    rc = lib().orc_requant_a(_ptr(a, _u16p), _ptr(a_i8, _i8p), _ptr(a_scale, _f32p), m, k)
    _check(rc, "requant_a")
    return a_i8, a_scale


def bf16_round(x: float) -> float:
    """Nearest BF16 value of a binary32 (ties to even), as a float."""
    return float(lib().orc_bf16_round(float(np.float32(x))))


def exp_neg_f32(g: float) -> float:
    """exp(-g) rounded once to binary32."""
    return float(lib().orc_exp_neg_f32(float(np.float32(g))))


def silu_mul(g: float, u: float) -> float:
    """BF16 value of fl32(fl32(g / fl32(1 + exp(-g))) * u)."""
    return float(lib().orc_silu_mul(float(np.float32(g)), float(np.float32(u))))


def silu_mul_requant(gate_bits, up_bits, k=None):
    """SiLU(gate) * up (BF16 raw bits, [M, ld]) over the first k columns ->
    (q [M,k] int8, scale [M,k/32] float32)."""
    g = np.ascontiguousarray(gate_bits, dtype=np.uint16)
    u = np.ascontiguousarray(up_bits, dtype=np.uint16)
    if g.shape != u.shape:
        raise ValueError(f"gate {g.shape} and up {u.shape} differ")
    m, ld = g.shape
    k = ld if k is None else k
    q = np.empty((m, k), np.int8)
    s = np.empty((m, max(k // 32, 0)), np.float32)
    rc = lib().orc_silu_mul_requant(_ptr(g, _u16p), _ptr(u, _u16p), ld, _ptr(q, _i8p), _ptr(s, _f32p), m, k)
    _check(rc, "silu_mul_requant")
    return q, s


def block_partials(a_i8, w_i8):
    """Exact int32 P[m, n, b] = sum over the 32 elements of block b of a_i8 * w_i8."""
    a = np.ascontiguousarray(a_i8, dtype=np.int8)
    w = np.ascontiguousarray(w_i8, dtype=np.int8)
    m, k = a.shape
    n = w.shape[0]
    p = np.empty((m, n, max(k // 32, 0)), np.int32)
    rc = lib().orc_block_partials(_ptr(a, _i8p), _ptr(w, _i8p), _ptr(p, _i32p), m, n, k)
    _check(rc, "block_partials")
    return p


def gemm_ref(a_i8, w_i8, a_scale, w_scale, rows=None):
    """FP64 reference (y, t) for the given activation rows (all rows by default)."""
    a = np.ascontiguousarray(a_i8, dtype=np.int8)
    w = np.ascontiguousarray(w_i8, dtype=np.int8)
    a_s = np.ascontiguousarray(a_scale, dtype=np.float32)
    w_s = np.ascontiguousarray(w_scale, dtype=np.float32)
    m, k = a.shape
    n = w.shape[0]
    if rows is None:
        rows = np.arange(m, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= m):
        raise IndexError("row index out of range")
    y = np.empty((rows.size, n), np.float64)
    t = np.empty((rows.size, n), np.float64)
    rc = lib().orc_gemm_ref(_ptr(a, _i8p), _ptr(w, _i8p), _ptr(a_s, _f32p), _ptr(w_s, _f32p),
                            _ptr(rows, _i64p), rows.size, _ptr(y, _f64p), _ptr(t, _f64p), n, k)
    _check(rc, "gemm_ref")
    return y, t


def e4m3_encode(x: float) -> int:
    """Nearest OCP E4M3 code of a binary32 (ties to even, saturating at 448)."""
    return int(lib().orc_e4m3_encode(float(np.float32(x))))


def quant_act(a_bf16_bits, group, e4m3=False):
    """BF16 activations -> (codes [M,K] uint8 (int8 or E4M3 bytes), scales [M,K/group] float32);
    group 32, 128 or K (one scale per row)."""
    a = np.ascontiguousarray(a_bf16_bits, dtype=np.uint16)
    m, k = a.shape
    q = np.empty((m, k), np.uint8)
    s = np.empty((m, max(k // group, 0)), np.float32)
    rc = lib().orc_quant_act(_ptr(a, _u16p), _ptr(q, _u8p), _ptr(s, _f32p), m, k, group, int(bool(e4m3)))
    _check(rc, "quant_act")
    return q, s


def gemm_ref_agroup(a_i8, w_i8, a_scale, w_scale, group, rows=None):
    """FP64 reference (y, t) with activation scales per `group` (32, 128 or K) and per-32 weight scales."""
    a = np.ascontiguousarray(a_i8, dtype=np.int8)
    w = np.ascontiguousarray(w_i8, dtype=np.int8)
    a_s = np.ascontiguousarray(a_scale, dtype=np.float32)
    w_s = np.ascontiguousarray(w_scale, dtype=np.float32)
    m, k = a.shape
    n = w.shape[0]
    if rows is None:
        rows = np.arange(m, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    y = np.empty((rows.size, n), np.float64)
    t = np.empty((rows.size, n), np.float64)
    rc = lib().orc_gemm_ref_agroup(_ptr(a, _i8p), _ptr(w, _i8p), _ptr(a_s, _f32p), _ptr(w_s, _f32p),
                                   _ptr(rows, _i64p), rows.size, _ptr(y, _f64p), _ptr(t, _f64p), n, k, group)
    _check(rc, "gemm_ref_agroup")
    return y, t


def w4a16_ref(x_bf16_bits, w_packed, w_e4m3, scale2, rows=None):
    """FP64 reference (y, t) of BF16 activations times the dequantized NVFP4 weight."""
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    wp = np.ascontiguousarray(w_packed, dtype=np.uint8)
    we = np.ascontiguousarray(w_e4m3, dtype=np.uint8)
    m, k = x.shape
    n = wp.shape[0]
    if wp.shape != (n, k // 2) or we.shape != (n, k // 16):
        raise ValueError("weight shapes do not match k")
    if rows is None:
        rows = np.arange(m, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    y = np.empty((rows.size, n), np.float64)
    t = np.empty((rows.size, n), np.float64)
    rc = lib().orc_w4a16_ref(_ptr(x, _u16p), _ptr(wp, _u8p), _ptr(we, _u8p), float(np.float32(scale2)),
                             _ptr(rows, _i64p), rows.size, _ptr(y, _f64p), _ptr(t, _f64p), n, k)
    _check(rc, "w4a16_ref")
    return y, t


def max_threads() -> int:
    return int(lib().orc_max_threads())


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))
