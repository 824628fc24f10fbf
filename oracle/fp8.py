"""FP8 weight-only decoding for the CPU oracle (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/block.py``).

The inference-research page on Gemma-4-26B-A4B quotes the weight footprint
of the 26B model as 57.7 GB in BF16 and 28.8 GB at SFP8: one byte per weight,
with scales too few to show.  The page defines neither the 8-bit format nor
its scaling.  Reading taken here: OCP float8_e4m3fn codes (the 8-bit float
that the gfx950 matrix and conversion units take natively) with one fp32
scale per matrix, and the matrices keep the bf16 weights' [K, N] layout:

    w[k, n] = e4m3fn(q[k, n]) * tensor_scale

The element format is decoded by ``oracle.nvfp4.e4m3fn_value`` (its table is
pinned against torch's float8_e4m3fn for all 256 codes).
"""
from __future__ import annotations

import numpy as np

from .nvfp4 import E4M3_TABLE


def dequant_matrix_fp8(q: np.ndarray, tensor_scale) -> np.ndarray:
    """One FP8 matrix -> fp64 [K, N] weights: q [K, N] uint8 (e4m3fn bits),
    tensor_scale fp32."""
    return E4M3_TABLE[np.asarray(q, dtype=np.uint8)] * float(np.float32(tensor_scale))
