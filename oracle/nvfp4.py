"""NVFP4 weight-only decoding for the CPU oracle (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/block.py``).

The NVFP4 checkpoint config of the 26B-A4B model (``quantization_config``,
``config_groups.group_0.weights``) fixes: 4-bit float values
(``num_bits: 4``, ``type: float``), groups of 16 (``group_size: 16``),
``float8_e4m3fn`` group scales, strategy ``tensor_group`` (one scale per
tensor on top of the group scales), symmetric, static, format
``nvfp4-pack-quantized``; the router (``router.proj``) is in ``ignore`` and
stays unquantised.

The element formats are written out here from their definitions:

* e2m1 (OCP Microscaling Formats v1.0, FP4): bit 3 sign, bits 2..1 exponent
  with bias 1, bit 0 mantissa; exponent 0 is subnormal (0.m x 2^0).
* e4m3fn (OCP 8-bit Floating Point, E4M3): bit 7 sign, bits 6..3 exponent
  with bias 7, bits 2..0 mantissa; exponent 0 is subnormal (0.mmm x 2^-6);
  S.1111.111 is NaN and there is no infinity (max 448).

Packing reading: matrices are stored in the Linear [out, in] convention,
value (n, k) of a [K, N] matrix in byte q[n, k // 2], low nibble for even
k; group scales scale[n, k // 16]; w = e2m1 * e4m3(scale) * tensor_scale.
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code: int) -> float:
    """Value of one 4-bit e2m1 code."""
    code = int(code) & 0xF
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = (m / 2.0) * 2.0 ** (1 - 1)          # subnormal: 0.m x 2^(1-bias)
    else:
        mag = (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return sign * mag


def e4m3fn_value(byte: int) -> float:
    """Value of one float8_e4m3fn byte (NaN for S.1111.111)."""
    b = int(byte) & 0xFF
    sign = -1.0 if (b >> 7) & 1 else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3fn_value(b) for b in range(256)], dtype=np.float64)


def unpack_codes(q: np.ndarray) -> np.ndarray:
    """[N, K/2] bytes -> [N, K] 4-bit codes (low nibble is the even k)."""
    q = np.asarray(q, dtype=np.uint8)
    N, KH = q.shape
    codes = np.empty((N, 2 * KH), dtype=np.uint8)
    codes[:, 0::2] = q & 0xF
    codes[:, 1::2] = q >> 4
    return codes


def dequant_matrix(q: np.ndarray, scale: np.ndarray, tensor_scale) -> np.ndarray:
    """One packed matrix -> fp64 [K, N] weights.

    q [N, K/2] uint8, scale [N, K/16] uint8 (e4m3fn bits), tensor_scale fp32.
    """
    codes = unpack_codes(q)
    N, K = codes.shape
    vals = E2M1_TABLE[codes]                                   # [N, K]
    gs = np.repeat(E4M3_TABLE[np.asarray(scale, dtype=np.uint8)], 16, axis=1)
    w_nk = vals * gs * float(np.float32(tensor_scale))
    return np.ascontiguousarray(w_nk.T)
