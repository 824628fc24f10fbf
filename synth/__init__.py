"""Seeded synthetic inputs for the MoE feed-forward block.

This module is shared by the CPU oracle (``oracle/``) and the HIP path
(``sparse_moe_transformer_amd``); it holds no arithmetic of the block itself
(no routing, no GeGLU, no dequantisation).  It only draws numbers and stores
them in the byte formats the block consumes:

* bf16 tensors as ``uint16`` arrays of raw bits (round-to-nearest-even from
  fp32 draws), shaped exactly like the device buffers;
* the NVFP4 weight-only packing (e2m1 codes two per byte, e4m3 group scales,
  one fp32 scale per tensor) and the FP8 weight-only packing (e4m3fn codes,
  one fp32 scale per matrix), used as *checkpoint producers*: both sides read
  the same packed bytes, so the rounding choices made here cannot affect
  parity.

Random streams: ``numpy.random.default_rng([seed, layer, tensor_id, chunk])``
with a fixed id per tensor, so any tensor can be regenerated alone and the
result does not depend on the thread count.

Shapes and distributions follow the Gemma 4 26B-A4B configuration (gemma-llm
API page ``gm.nn.Gemma4_26B_A4B``, ``TransformerConfig``: embed_dim 2816,
num_experts 128, top_k_experts 8, expert_dim 704, moe_dense_hidden_dim 2112):
activations x ~ N(0, 1); every weight ~ N(0, 1/fan_in) with fan_in the
contracted dimension.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

# ---------------------------------------------------------------------------
# configurations
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class FFNShape:
    """Shape of one MoE feed-forward block and of one call on it."""

    name: str
    tokens: int          # T
    hidden: int          # H  (embed_dim)
    experts: int         # E  (num_experts)
    top_k: int           # k  (top_k_experts)
    expert_dim: int      # I  (expert_dim)
    dense_dim: int       # D  (moe_dense_hidden_dim)
    layers: int = 1
    skew: bool = False   # add a per-expert logit bias with Zipf-shaped loads
    nvfp4: bool = False  # weight-only NVFP4 packing of every expert/dense matrix
    fp8: bool = False    # weight-only FP8 (e4m3fn + per-matrix scale) packing

    def with_tokens(self, t: int) -> "FFNShape":
        return replace(self, tokens=int(t))


# the five workloads of the block: a tiny case, then the 26B-A4B layer shape
TINY = FFNShape("tiny", 32, 256, 8, 2, 64, 128)
DECODE = FFNShape("decode", 8, 2816, 128, 8, 704, 2112)
PREFILL = FFNShape("prefill", 4096, 2816, 128, 8, 704, 2112)
SKEW = FFNShape("skew", 16384, 2816, 128, 8, 704, 2112, skew=True)
NVFP4_STACK = FFNShape("nvfp4_stack", 1024, 2816, 128, 8, 704, 2112, layers=30,
                       nvfp4=True)
# the dense GeGLU FFN of the Gemma 4 E4B sibling (gemma-llm API page
# gm.nn.Gemma4_E4B: embed_dim 2560, hidden_dim 10240, enable_moe False,
# num_experts 0, expert_dim 0): no router and no experts
E4B_TINY = FFNShape("e4b_tiny", 32, 256, 0, 0, 0, 512)
E4B_DECODE = FFNShape("e4b_decode", 8, 2560, 0, 0, 0, 10240)
E4B_PREFILL = FFNShape("e4b_prefill", 4096, 2560, 0, 0, 0, 10240)
SHAPES = {s.name: s for s in (TINY, DECODE, PREFILL, SKEW, NVFP4_STACK, E4B_TINY, E4B_DECODE,
                              E4B_PREFILL)}

# tensor ids of the random streams
TID_X, TID_ROUTER, TID_GATE, TID_UP, TID_DOWN = 0, 1, 2, 3, 4
TID_DGATE, TID_DUP, TID_DDOWN, TID_ZIPF = 5, 6, 7, 8

# Zipf exponent of the skewed expert load and the logit-bias scale that gives
# a realised load with that log-log slope over ranks 9..128 at T=16384, seed 0.
# The value was found by bisection with tests/golden/calibrate_skew.py, which
# routes through the CPU oracle; tests/test_oracle_pins.py re-checks it.
ZIPF_S = 1.2
SKEW_LAMBDA = 0.4727793

_CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------------------
# bf16 storage
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return raw uint16 bits.

    Inputs here are finite normal draws, so NaN handling is not needed.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits to fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, layer: int, tid: int, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draws rounded to bf16, as uint16 bits of the given shape."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(c: int) -> None:
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = np.random.default_rng([seed, layer, tid, c])
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(v)

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


# ---------------------------------------------------------------------------
# one layer of inputs
# ---------------------------------------------------------------------------


def make_x(shape: FFNShape, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Activations x [T, H], bf16 bits."""
    return normal_bf16(seed, layer, TID_X, (shape.tokens, shape.hidden))


def make_weights(shape: FFNShape, seed: int = 0, layer: int = 0) -> dict:
    """bf16 weights of one block, row-major [K, N] per matrix (N contiguous).

    router [H, E]; gate, up [E, H, I]; down [E, I, H]; dgate, dup [H, D];
    ddown [D, H] (None where the shape has no experts or no dense branch).
    std = fan_in ** -0.5 with fan_in = the contracted size.
    """
    H, E, I, D = shape.hidden, shape.experts, shape.expert_dim, shape.dense_dim
    if E > 0:
        w = {
            "router": normal_bf16(seed, layer, TID_ROUTER, (H, E), H ** -0.5),
            "gate": normal_bf16(seed, layer, TID_GATE, (E, H, I), H ** -0.5),
            "up": normal_bf16(seed, layer, TID_UP, (E, H, I), H ** -0.5),
            "down": normal_bf16(seed, layer, TID_DOWN, (E, I, H), I ** -0.5),
        }
    else:  # a dense FFN: no router, no experts
        w = {"router": None, "gate": None, "up": None, "down": None}
    if D > 0:
        w["dgate"] = normal_bf16(seed, layer, TID_DGATE, (H, D), H ** -0.5)
        w["dup"] = normal_bf16(seed, layer, TID_DUP, (H, D), H ** -0.5)
        w["ddown"] = normal_bf16(seed, layer, TID_DDOWN, (D, H), D ** -0.5)
    else:
        w["dgate"] = w["dup"] = w["ddown"] = None
    return w


def zipf_bias(experts: int, lam: float = SKEW_LAMBDA, s: float = ZIPF_S,
              seed: int = 0, layer: int = 0) -> np.ndarray:
    """Per-expert fp32 logit bias b_e = lam * ln p_e, p_e ∝ (pi_e + 1)^-s.

    pi is a seeded permutation of the experts, so the hot experts are spread
    over the id range rather than sitting at the low ids.
    """
    g = np.random.default_rng([seed, layer, TID_ZIPF, 0])
    pi = g.permutation(experts)
    p = (pi + 1.0) ** (-s)
    p /= p.sum()
    return (lam * np.log(p)).astype(np.float32)


# ---------------------------------------------------------------------------
# NVFP4 weight-only packing (checkpoint producer)
# ---------------------------------------------------------------------------

_FP8_MAX = 448.0
_FP4_MAX = 6.0


def _e2m1_codes(v: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code of each value (ties to the even mantissa), saturating."""
    a = np.abs(v)
    # midpoints between neighbouring grid values; at a tie, the code with an
    # even mantissa bit (0, 1.0, 2.0, 4.0 -> codes 0, 2, 4, 6) wins
    mag = np.zeros(a.shape, dtype=np.uint8)
    mag[a > 0.25] = 1
    mag[a >= 0.75] = 2
    mag[a > 1.25] = 3
    mag[a >= 1.75] = 4
    mag[a > 2.5] = 5
    mag[a >= 3.5] = 6
    mag[a > 5.0] = 7
    sign = ((v < 0) & (mag > 0)).astype(np.uint8) << 3
    return mag | sign


def _to_e4m3_bits(v: np.ndarray) -> np.ndarray:
    import torch  # the float8_e4m3fn cast rounds to nearest even

    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _e4m3_bits_to_f64(b: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def nvfp4_pack(w_kn: np.ndarray) -> tuple:
    """Pack one [K, N] weight matrix (fp32 values) as NVFP4, weight only.

    Returns (q [N, K/2] uint8, scale [N, K/16] uint8 e4m3fn bits,
    tensor_scale float).  The layout is the Linear [out, in] convention:
    value (n, k) sits in byte q[n, k // 2], low nibble for even k.  Groups of
    16 run along K.  tensor_scale = amax / (6 * 448); group scale =
    e4m3(amax_group / (6 * tensor_scale)); code = nearest e2m1 of
    w / (group_scale * tensor_scale).
    """
    K, N = w_kn.shape
    assert K % 16 == 0
    w = np.ascontiguousarray(np.asarray(w_kn, dtype=np.float64).T)  # [N, K]
    amax = float(np.max(np.abs(w))) if w.size else 0.0
    st = np.float32(amax / (_FP4_MAX * _FP8_MAX)) if amax > 0 else np.float32(1.0)
    st64 = float(st)
    grp = w.reshape(N, K // 16, 16)
    gmax = np.max(np.abs(grp), axis=2)
    sbits = _to_e4m3_bits(gmax / (_FP4_MAX * st64))
    sval = _e4m3_bits_to_f64(sbits)
    denom = sval * st64
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(denom[:, :, None] > 0, grp / denom[:, :, None], 0.0)
    codes = _e2m1_codes(v).reshape(N, K)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return q, sbits, float(st)


def nvfp4_pack_stack(w_ekn_bits: np.ndarray) -> dict:
    """Pack a stack [G, K, N] of bf16-bit matrices; one tensor scale per matrix."""
    G, K, N = w_ekn_bits.shape
    q = np.empty((G, N, K // 2), dtype=np.uint8)
    s = np.empty((G, N, K // 16), dtype=np.uint8)
    st = np.empty((G,), dtype=np.float32)

    def work(g: int) -> None:
        q[g], s[g], st[g] = nvfp4_pack(bf16_bits_to_f32(w_ekn_bits[g]))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(G)))
    return {"q": q, "scale": s, "tensor_scale": st}


def make_nvfp4_weights(shape: FFNShape, seed: int = 0, layer: int = 0) -> dict:
    """bf16 N(0, 1/fan_in) weights of one layer, then NVFP4-packed.

    The router stays bf16 (it is excluded from quantisation in the NVFP4
    checkpoint's ``quantization_config.ignore`` list).  Dense matrices are
    packed as stacks of one.
    """
    w = make_weights(shape, seed, layer)
    out = {"router": w["router"]}
    for name in ("gate", "up", "down"):
        out[name] = nvfp4_pack_stack(w[name]) if w[name] is not None else None
    for name in ("dgate", "dup", "ddown"):
        out[name] = nvfp4_pack_stack(w[name][None]) if w[name] is not None else None
    return out


def bf16_bits(x) -> np.ndarray:
    """Convenience: accept fp32 values or uint16 bits, return uint16 bits."""
    x = np.asarray(x)
    return x if x.dtype == np.uint16 else f32_to_bf16_bits(x.astype(np.float32))



# ---------------------------------------------------------------------------
# FP8 weight-only packing (checkpoint producer)
# ---------------------------------------------------------------------------


def fp8_pack(w_kn: np.ndarray) -> tuple:
    """Pack one [K, N] weight matrix (fp32 values) as e4m3fn codes with one
    fp32 scale: returns (q [K, N] uint8, tensor_scale float).

    tensor_scale = amax / 448 (1 for an all-zero matrix); code = nearest
    e4m3fn value of w / tensor_scale (ties to even), clamped to +-448 first.
    The layout stays [K, N] (N contiguous), like the bf16 weights.
    """
    w = np.asarray(w_kn, dtype=np.float32)
    amax = float(np.max(np.abs(w))) if w.size else 0.0
    st = np.float32(amax / _FP8_MAX) if amax > 0 else np.float32(1.0)
    v = np.clip(w / st, -_FP8_MAX, _FP8_MAX)
    return _to_e4m3_bits(v).reshape(w.shape), float(st)


def fp8_pack_stack(w_ekn_bits: np.ndarray) -> dict:
    """Pack a stack [G, K, N] of bf16-bit matrices; one scale per matrix."""
    G, K, N = w_ekn_bits.shape
    q = np.empty((G, K, N), dtype=np.uint8)
    st = np.empty((G,), dtype=np.float32)

    def work(g: int) -> None:
        q[g], st[g] = fp8_pack(bf16_bits_to_f32(w_ekn_bits[g]))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(G)))
    return {"q8": q, "tensor_scale": st}


def make_fp8_weights(shape: FFNShape, seed: int = 0, layer: int = 0) -> dict:
    """bf16 N(0, 1/fan_in) weights of one layer, then FP8-packed; the router
    stays bf16 and dense matrices are packed as stacks of one."""
    w = make_weights(shape, seed, layer)
    out = {"router": w["router"]}
    for name in ("gate", "up", "down"):
        out[name] = fp8_pack_stack(w[name]) if w[name] is not None else None
    for name in ("dgate", "dup", "ddown"):
        out[name] = fp8_pack_stack(w[name][None]) if w[name] is not None else None
    return out
