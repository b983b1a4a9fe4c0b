"""Python binding of libbsr: the C-ABI entry points under the same names.

Argument marshalling only -- every step runs in the HIP kernels of libbsr.so.
Tensors must be CUDA (HIP) tensors; their data pointers, sizes derived from
their shapes, and a stream (default: torch's current stream on the tensors'
device) are passed straight through.  A non-zero status raises ``BsrError``.
There is no fallback: if libbsr.so is missing, the first call raises.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsr.so")

BSR_OK, BSR_EINVAL, BSR_ENULL, BSR_EALIGN, BSR_EDEVICE, BSR_ELAUNCH = range(6)
PATH_AUTO, PATH_GEMM, PATH_GEMV, PATH_INVARIANT = 0, 1, 2, 3
GEMV_MAX_ROWS = 16          # any K
GEMV_STREAM_MAX_ROWS = 64   # K a multiple of 256

# Exported symbols and their C signatures (kept in step with include/bsr.h).
_vp, _u32, _f32, _int = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_float, ctypes.c_int
SIGNATURES = {
    "requant_w_nvfp4_int8": (_int, [_vp, _vp, _f32, _vp, _vp, _u32, _u32, _vp]),
    "requant_a_int8": (_int, [_vp, _vp, _vp, _u32, _u32, _vp]),
    "int8_gemm_blockscaled": (_int, [_vp, _vp, _vp, _vp, _vp, _u32, _u32, _u32, _vp]),
    "int8_gemm_blockscaled_ex": (_int, [_vp, _vp, _vp, _vp, _vp, _u32, _u32, _u32, _vp, _int]),
    "silu_mul_requant_int8": (_int, [_vp, _vp, _u32, _vp, _vp, _u32, _u32, _vp]),
    "w4a16_gemv": (_int, [_vp, _vp, _vp, _f32, _vp, _u32, _u32, _u32, _vp]),
    "quantize_act": (_int, [_vp, _vp, _vp, _u32, _u32, _u32, _int, _vp]),
    "int8_gemm_blockscaled_agroup": (_int, [_vp, _vp, _vp, _u32, _vp, _vp, _u32, _u32, _u32, _vp, _int]),
    "int8_gemm_blockscaled_ws_bytes": (ctypes.c_uint64, [_u32, _u32, _u32]),
    "int8_gemm_blockscaled_ws": (_int, [_vp, _vp, _vp, _vp, _vp, _u32, _u32, _u32, _vp, ctypes.c_uint64, _vp]),
    "int8_gemm_blockscaled_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _u32, _u32, _u32, _vp]),
    "bsr_status_string": (ctypes.c_char_p, [_int]),
}

_LIB = None


class BsrError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def lib():
    """The loaded libbsr.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; "
                               f"g.build()'` or `python block_scaled_precision_requant_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().bsr_status_string(int(status)).decode()


def _ptr(t):
    # runs after every argument's shape and element checks
    if t is None:
        return ctypes.c_void_p(0)
    if not t.is_cuda:
        raise ValueError("arguments must be device tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, like):
    if stream is None:
        stream = torch.cuda.current_stream(like.device)
    return ctypes.c_void_p(stream.cuda_stream)


# Element kinds the kernels read and write: byte codes (int8, packed E2M1,
# E4M3), 16-bit BF16 bits (any 2-byte dtype: torch.bfloat16, int16, uint16)
# and binary32 scales.
BYTES, BF16, F32 = "1-byte", "2-byte", "float32"


def _shape(t, shape, what, kind):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    _kind(t, what, kind)


def _kind(t, what, kind):
    ok = (t.dtype == torch.float32 if kind == F32 else
          t.element_size() == (1 if kind == BYTES else 2) and not t.dtype.is_complex)
    if not ok:
        raise ValueError(f"{what}: dtype {t.dtype}, expected {kind} elements")


def _done(status, what):
    if status != BSR_OK:
        raise BsrError(status, what)


def requant_w_nvfp4_int8(w_packed, w_e4m3, scale2, w_i8, w_scale, stream=None):
    """NVFP4 weight (w_packed [N,K/2] u8, w_e4m3 [N,K/16] u8, scale2 float) ->
    w_i8 [N,K] int8 and w_scale [N,K/32] float32 (both preallocated)."""
    n, half_k = w_packed.shape
    k = 2 * half_k
    _shape(w_packed, (n, k // 2), "w_packed", BYTES)
    _shape(w_e4m3, (n, k // 16), "w_e4m3", BYTES)
    _shape(w_i8, (n, k), "w_i8", BYTES)
    _shape(w_scale, (n, k // 32), "w_scale", F32)
    st = lib().requant_w_nvfp4_int8(_ptr(w_packed), _ptr(w_e4m3), float(scale2), _ptr(w_i8),
                                    _ptr(w_scale), n, k, _stream(stream, w_i8))
    _done(st, "requant_w_nvfp4_int8")


def requant_a_int8(a_bf16, a_i8, a_scale, stream=None):
    """BF16 activations a_bf16 [M,K] -> a_i8 [M,K] int8 and a_scale [M,K/32] float32."""
    m, k = a_bf16.shape
    _shape(a_bf16, (m, k), "a_bf16", BF16)
    _shape(a_i8, (m, k), "a_i8", BYTES)
    _shape(a_scale, (m, k // 32), "a_scale", F32)
    st = lib().requant_a_int8(_ptr(a_bf16), _ptr(a_i8), _ptr(a_scale), m, k, _stream(stream, a_i8))
    _done(st, "requant_a_int8")


def silu_mul_requant_int8(gate, up, a_i8, a_scale, stream=None):
    """SiLU(gate) * up -> a_i8 [M,K] int8 and a_scale [M,K/32] float32.

    gate and up are [M,K] BF16 (raw 16-bit) views with unit column stride and
    the same row stride (for instance the two halves of one [M, 2K] buffer)."""
    m, k = gate.shape
    if tuple(up.shape) != (m, k):
        raise ValueError(f"up: shape {tuple(up.shape)}, expected {(m, k)}")
    for t, what in ((gate, "gate"), (up, "up")):
        _kind(t, what, BF16)
        if (m > 1 and t.stride(1) != 1) or (m > 1 and t.stride(0) != gate.stride(0)):
            raise ValueError(f"{what}: 16-bit rows with unit column stride and the gate's row stride")
    ld = gate.stride(0) if m > 1 else k
    _shape(a_i8, (m, k), "a_i8", BYTES)
    _shape(a_scale, (m, k // 32), "a_scale", F32)
    st = lib().silu_mul_requant_int8(_ptr(gate), _ptr(up), ld, _ptr(a_i8), _ptr(a_scale), m, k,
                                     _stream(stream, a_i8))
    _done(st, "silu_mul_requant_int8")


def w4a16_gemv(x_bf16, w_packed, w_e4m3, scale2, out, stream=None):
    """out [M,N] BF16 = x_bf16 [M,K] (M <= 16) times the NVFP4 weight (w_packed [N,K/2] u8,
    w_e4m3 [N,K/16] u8, scale2), dequantized on the fly."""
    m, k = x_bf16.shape
    n = w_packed.shape[0]
    _shape(x_bf16, (m, k), "x_bf16", BF16)
    _shape(w_packed, (n, k // 2), "w_packed", BYTES)
    _shape(w_e4m3, (n, k // 16), "w_e4m3", BYTES)
    _shape(out, (m, n), "out", BF16)
    st = lib().w4a16_gemv(_ptr(x_bf16), _ptr(w_packed), _ptr(w_e4m3), float(scale2), _ptr(out), m, n, k,
                          _stream(stream, out))
    _done(st, "w4a16_gemv")


def int8_gemm_blockscaled_ex(a_i8, w_i8, a_scale, w_scale, out, path=PATH_AUTO, stream=None):
    """out [M,N] BF16 = block-scaled int8 GEMM of a_i8 [M,K] and w_i8 [N,K]."""
    m, k = a_i8.shape
    n = w_i8.shape[0]
    _shape(a_i8, (m, k), "a_i8", BYTES)
    _shape(w_i8, (n, k), "w_i8", BYTES)
    _shape(a_scale, (m, k // 32), "a_scale", F32)
    _shape(w_scale, (n, k // 32), "w_scale", F32)
    _shape(out, (m, n), "out", BF16)
    st = lib().int8_gemm_blockscaled_ex(_ptr(a_i8), _ptr(w_i8), _ptr(a_scale), _ptr(w_scale), _ptr(out),
                                        m, n, k, _stream(stream, out), int(path))
    _done(st, "int8_gemm_blockscaled_ex")


def int8_gemm_blockscaled(a_i8, w_i8, a_scale, w_scale, out, stream=None):
    """As int8_gemm_blockscaled_ex with the automatic path (the GEMV for M <= 16, and for
    M <= 48 when K % 256 == 0 and N <= 4096; else the GEMM)."""
    m, k = a_i8.shape
    n = w_i8.shape[0]
    _shape(a_i8, (m, k), "a_i8", BYTES)
    _shape(w_i8, (n, k), "w_i8", BYTES)
    _shape(a_scale, (m, k // 32), "a_scale", F32)
    _shape(w_scale, (n, k // 32), "w_scale", F32)
    _shape(out, (m, n), "out", BF16)
    st = lib().int8_gemm_blockscaled(_ptr(a_i8), _ptr(w_i8), _ptr(a_scale), _ptr(w_scale), _ptr(out),
                                     m, n, k, _stream(stream, out))
    _done(st, "int8_gemm_blockscaled")


def int8_gemm_blockscaled_ws_bytes(m, n, k):
    """Workspace bytes int8_gemm_blockscaled_ws needs for (m, n, k); 0 if it runs without a K split."""
    return int(lib().int8_gemm_blockscaled_ws_bytes(int(m), int(n), int(k)))


def int8_gemm_blockscaled_ws(a_i8, w_i8, a_scale, w_scale, out, workspace, stream=None):
    """int8_gemm_blockscaled with a caller workspace (a 16-byte aligned device
    tensor of at least int8_gemm_blockscaled_ws_bytes(M, N, K) bytes, or None when
    that is 0), which lets small grids split K across workgroups."""
    m, k = a_i8.shape
    n = w_i8.shape[0]
    _shape(a_i8, (m, k), "a_i8", BYTES)
    _shape(w_i8, (n, k), "w_i8", BYTES)
    _shape(a_scale, (m, k // 32), "a_scale", F32)
    _shape(w_scale, (n, k // 32), "w_scale", F32)
    _shape(out, (m, n), "out", BF16)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace: must be contiguous")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().int8_gemm_blockscaled_ws(_ptr(a_i8), _ptr(w_i8), _ptr(a_scale), _ptr(w_scale), _ptr(out), m, n, k,
                                        _ptr(workspace), ws_bytes, _stream(stream, out))
    _done(st, "int8_gemm_blockscaled_ws")


def int8_gemm_blockscaled_noalloc(a_i8, w_i8, a_scale, w_scale, out, stream=None):
    """int8_gemm_blockscaled_ws with the library's static per-GPU scratch as the
    workspace: allocates nothing; calls that overlap in time on one GPU race."""
    m, k = a_i8.shape
    n = w_i8.shape[0]
    _shape(a_i8, (m, k), "a_i8", BYTES)
    _shape(w_i8, (n, k), "w_i8", BYTES)
    _shape(a_scale, (m, k // 32), "a_scale", F32)
    _shape(w_scale, (n, k // 32), "w_scale", F32)
    _shape(out, (m, n), "out", BF16)
    st = lib().int8_gemm_blockscaled_noalloc(_ptr(a_i8), _ptr(w_i8), _ptr(a_scale), _ptr(w_scale), _ptr(out),
                                             m, n, k, _stream(stream, out))
    _done(st, "int8_gemm_blockscaled_noalloc")


FMT_INT8, FMT_E4M3 = 0, 1


def _scale_cols(k, group):
    return 1 if group == 0 else k // group


def quantize_act(a_bf16, q, scale, group=32, fmt=FMT_INT8, stream=None):
    """BF16 a_bf16 [M,K] -> codes q [M,K] (uint8: int8 or E4M3 bits) and float32
    scales [M, K/group] (group 32 or 128) or [M, 1] (group 0: one per row)."""
    m, k = a_bf16.shape
    _shape(a_bf16, (m, k), "a_bf16", BF16)
    _shape(q, (m, k), "q", BYTES)
    _shape(scale, (m, _scale_cols(k, group)), "scale", F32)
    st = lib().quantize_act(_ptr(a_bf16), _ptr(q), _ptr(scale), m, k, int(group), int(fmt), _stream(stream, q))
    _done(st, "quantize_act")


def int8_gemm_blockscaled_agroup(a_i8, w_i8, a_scale, a_group, w_scale, out, path=PATH_AUTO, stream=None):
    """int8_gemm_blockscaled_ex with activation scales a_scale [M, K/a_group]
    (a_group 32 or 128) or [M, 1] (a_group 0: one per row)."""
    m, k = a_i8.shape
    n = w_i8.shape[0]
    _shape(a_i8, (m, k), "a_i8", BYTES)
    _shape(w_i8, (n, k), "w_i8", BYTES)
    _shape(a_scale, (m, _scale_cols(k, a_group)), "a_scale", F32)
    _shape(w_scale, (n, k // 32), "w_scale", F32)
    _shape(out, (m, n), "out", BF16)
    st = lib().int8_gemm_blockscaled_agroup(_ptr(a_i8), _ptr(w_i8), _ptr(a_scale), int(a_group), _ptr(w_scale),
                                            _ptr(out), m, n, k, _stream(stream, out), int(path))
    _done(st, "int8_gemm_blockscaled_agroup")


def prefill(a_bf16, w_i8, w_scale, a_i8_scratch, a_scale_scratch, out, stream=None):
    """The two-launch projection: requant_a_int8 then int8_gemm_blockscaled on one stream."""
    requant_a_int8(a_bf16, a_i8_scratch, a_scale_scratch, stream=stream)
    int8_gemm_blockscaled(a_i8_scratch, w_i8, a_scale_scratch, w_scale, out, stream=stream)
