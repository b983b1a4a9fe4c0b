"""MI355X-native block-scaled int8 projection: NVFP4/BF16 -> int8 per-32 requant
and the int8 x int8 block-scaled GEMM / small-M GEMV, as hand-written HIP for
gfx950 behind a C-ABI library (``libbsr.so``).

Importing the package loads nothing; ``block_scaled_precision_requant_amd.bsr``
loads the HIP library on first use and fails loudly when it is missing.
"""
__all__ = ["bsr", "inputs"]
