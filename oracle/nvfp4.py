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


# ---------------------------------------------------------------------------
# W4A4: NVFP4 activations
# ---------------------------------------------------------------------------
#
# The checkpoint config's ``input_activations`` (same group): 4-bit float
# values, groups of 16, float8_e4m3fn group scales, strategy tensor_group,
# symmetric, ``dynamic: local`` (the group scales are computed from each
# call's activations) with a static global scale (``observer:
# static_minmax``: a calibrated constant).  Readings taken here:
#
# * one global scale s_in per activation tensor that a group of Linear layers
#   reads (the block input x for every gate/up projection, the routed hidden
#   h for every expert's down projection, the dense hidden h_d for the dense
#   down projection);
# * each 16-element group along K of a token row:
#       s_g  = e4m3(amax / (6 * s_in))          (round to nearest even, saturating)
#       code = e2m1(v / (s_g * s_in))           (round to nearest even, saturating)
#       dequantised value = e2m1(code) * s_g * s_in
#   with s_g = 0 (all-zero group or a vanishing scale) giving zeros;
# * a quantisation decision (a scale or a code) is taken in fp32, the
#   precision of the activations' arithmetic: 6 * s_in, amax / (6 * s_in),
#   s_g * s_in and v / (s_g * s_in) are each one correctly rounded fp32
#   operation, in that order.


def round_e4m3_sat(r) -> np.ndarray:
    """Nearest float8_e4m3fn value of non-negative fp32 values (ties to an
    even mantissa), saturating at 448; from the format definition: normal
    values keep 3 mantissa bits, below 2^-6 the step is 2^-9."""
    r = np.asarray(r, dtype=np.float64)
    out = np.empty_like(r)
    sub = r < 2.0 ** -6
    out[sub] = np.rint(r[sub] * 2.0 ** 9) * 2.0 ** -9          # subnormal grid
    rn = r[~sub]
    _, e = np.frexp(rn)                                         # rn = m * 2^e, m in [0.5, 1)
    step = np.ldexp(1.0, e - 4)                                 # 2^(floor(log2 rn) - 3)
    out[~sub] = np.rint(rn / step) * step                       # 3 mantissa bits
    return np.minimum(out, 448.0)


def round_e2m1_sat(r) -> np.ndarray:
    """Nearest e2m1 value of fp32 values (ties to an even mantissa),
    saturating at +-6: steps of 0.5 below 2, 1 up to 4, 2 up to 6.  The sign
    is kept, also for a result of zero (e2m1 has a negative zero, code 8)."""
    r = np.asarray(r, dtype=np.float64)
    a = np.abs(r)
    v = np.where(a < 2.0, np.rint(a * 2.0) / 2.0, np.where(a < 4.0, np.rint(a), 2.0 * np.rint(a / 2.0)))
    return np.copysign(np.minimum(v, 6.0), r)


def quant_act_nvfp4(v, s_in) -> np.ndarray:
    """Quantise-dequantise activations [..., K] (bf16 values) in 16-groups
    along K with global scale s_in (fp32); returns e2m1(code) * s_g, the
    dequantised values without the global factor s_in (exact in bf16)."""
    v = np.asarray(v, dtype=np.float64)
    sh = v.shape
    g = v.reshape(*sh[:-1], sh[-1] // 16, 16)
    f32 = np.float32
    s_in = f32(s_in)
    amax = np.max(np.abs(g), axis=-1).astype(f32)                # bf16 values: exact in fp32
    six = f32(f32(6.0) * s_in)
    ratio = (amax / six).astype(f32)                             # one fp32 division
    sg = round_e4m3_sat(ratio)                                   # group scale value
    denom = (sg.astype(f32) * s_in).astype(f32)                  # one fp32 product
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (g.astype(f32) / denom[..., None]).astype(f32)       # one fp32 division
    q = np.where(denom[..., None] > 0, round_e2m1_sat(r), 0.0)
    return (q * sg[..., None]).reshape(sh)
