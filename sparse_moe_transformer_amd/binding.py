"""ctypes binding of libmoe_ffn.so (argument marshalling only).

Every function here has the name of the C entry point it calls and takes
plain integers for device pointers (e.g. ``tensor.data_ptr()``) and for the
stream (``torch.cuda.current_stream().cuda_stream``).  No arithmetic of the
block happens in Python: every step runs in the HIP kernels of the library.
If the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_FFN_LIB selects another build of the library (the host-sanitized one of
# the CPU ABI tests); the default is the in-tree build
LIB_PATH = os.environ.get("MOE_FFN_LIB") or os.path.join(_PKG, "libmoe_ffn.so")

MOE_FFN_OK = 0
MOE_FFN_ERR_INVALID_ARG = -1
MOE_FFN_ERR_UNSUPPORTED = -2
MOE_FFN_ERR_HIP = -3
MOE_FFN_ERR_OOM = -4

MOE_FFN_W_BF16 = 0
MOE_FFN_W_NVFP4 = 1
MOE_FFN_W_FP8 = 2
MOE_FFN_ACCUMULATE = 1

MOE_FFN_VARIANT_AUTO = 0
MOE_FFN_VARIANT_STREAM = 1
MOE_FFN_VARIANT_MFMA = 2

EXPORTS = (
    "moe_ffn_workspace_bytes", "moe_ffn_create", "moe_ffn_destroy", "moe_ffn_set_variant",
    "moe_ffn_forward", "moe_ffn_forward_nvfp4", "moe_ffn_forward_fp8", "moe_ffn_forward_w4a4",
    "moe_ffn_quant_act_nvfp4",
    "moe_ffn_forward_block",
    "moe_ffn_get_routing",
    "moe_ffn_get_intermediates", "moe_ffn_align_only", "moe_ffn_profile_begin",
    "moe_ffn_profile_end", "moe_ffn_forward_noalloc", "moe_ffn_last_error",
)
MOE_FFN_STAGE_ROUTE, MOE_FFN_STAGE_ALIGN, MOE_FFN_STAGE_GATEUP = 0, 1, 2
MOE_FFN_STAGE_DOWN, MOE_FFN_STAGE_COMBINE, MOE_FFN_STAGE_GEGLU = 3, 4, 5
MOE_FFN_NUM_STAGES = 6


class moe_ffn_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("expert_dim", ctypes.c_int32),
                ("dense_dim", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("weight_format", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class moe_ffn_nvfp4_t(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


class moe_ffn_fp8_t(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("tensor_scale", ctypes.c_void_p)]


class MoeFFNError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moe_ffn error {code}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_moe_transformer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER
        L.moe_ffn_workspace_bytes.argtypes = [P(moe_ffn_config), P(sz)]
        L.moe_ffn_create.argtypes = [P(moe_ffn_config), P(vp)]
        L.moe_ffn_destroy.argtypes = [vp]
        L.moe_ffn_set_variant.argtypes = [vp, i32]
        L.moe_ffn_forward.argtypes = [vp, i32] + [vp] * 11
        L.moe_ffn_forward_noalloc.argtypes = [P(moe_ffn_config), i32] + [vp] * 11
        L.moe_ffn_forward_nvfp4.argtypes = [vp, i32, vp, vp, vp] + [P(moe_ffn_nvfp4_t)] * 6 + [vp, vp]
        L.moe_ffn_quant_act_nvfp4.argtypes = [ctypes.c_int64, i32, vp, vp, vp, vp]
        L.moe_ffn_forward_w4a4.argtypes = [vp, i32, vp, vp, vp] + [P(moe_ffn_nvfp4_t)] * 6 + [vp, vp, vp]
        L.moe_ffn_forward_fp8.argtypes = [vp, i32, vp, vp, vp] + [P(moe_ffn_fp8_t)] * 6 + [vp, vp]
        L.moe_ffn_forward_block.argtypes = [vp, i32, vp, vp, vp, ctypes.c_float] + [vp] * 10
        L.moe_ffn_get_routing.argtypes = [vp] + [vp] * 7
        L.moe_ffn_get_intermediates.argtypes = [vp] + [vp] * 5
        L.moe_ffn_align_only.argtypes = [vp, i32, vp, vp]
        L.moe_ffn_profile_begin.argtypes = [vp, ctypes.c_uint32, i32]
        L.moe_ffn_profile_end.argtypes = [vp, vp, vp]
        L.moe_ffn_last_error.argtypes = []
        L.moe_ffn_last_error.restype = ctypes.c_char_p
        for name in EXPORTS[:-1]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def moe_ffn_last_error() -> str:
    return lib().moe_ffn_last_error().decode()


def check(rc: int) -> int:
    if rc != MOE_FFN_OK:
        raise MoeFFNError(rc, moe_ffn_last_error())
    return rc


def make_config(hidden, num_experts, top_k, expert_dim, dense_dim, max_tokens,
                weight_format=MOE_FFN_W_BF16, flags=0) -> moe_ffn_config:
    return moe_ffn_config(hidden, num_experts, top_k, expert_dim, dense_dim, max_tokens,
                          weight_format, flags)


def moe_ffn_workspace_bytes(cfg: moe_ffn_config) -> tuple:
    n = ctypes.c_size_t(0)
    rc = lib().moe_ffn_workspace_bytes(ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(n))
    return rc, n.value


def moe_ffn_create(cfg: moe_ffn_config) -> tuple:
    h = ctypes.c_void_p(0)
    rc = lib().moe_ffn_create(ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(h))
    return rc, h.value


def moe_ffn_destroy(h) -> int:
    return lib().moe_ffn_destroy(h)


def moe_ffn_set_variant(h, variant: int) -> int:
    return lib().moe_ffn_set_variant(h, variant)


def moe_ffn_forward(h, T, x, router_w, router_bias, w_gate, w_up, w_down, d_gate, d_up, d_down,
                    out, stream) -> int:
    return lib().moe_ffn_forward(h, T, x, router_w, router_bias, w_gate, w_up, w_down, d_gate,
                                 d_up, d_down, out, stream)


def moe_ffn_forward_noalloc(cfg, T, x, router_w, router_bias, w_gate, w_up, w_down, d_gate, d_up, d_down,
                            out, stream) -> int:
    """cfg: a moe_ffn_config (host structure) or None."""
    return lib().moe_ffn_forward_noalloc(ctypes.byref(cfg) if cfg is not None else None, T, x, router_w,
                                         router_bias, w_gate, w_up, w_down, d_gate, d_up, d_down, out, stream)


def moe_ffn_forward_nvfp4(h, T, x, router_w, router_bias, w_gate, w_up, w_down, d_gate, d_up,
                          d_down, out, stream) -> int:
    """Weight descriptors are (q_ptr, scale_ptr, tensor_scale_ptr) tuples or None."""
    def desc(d):
        if d is None:
            return None
        return ctypes.byref(moe_ffn_nvfp4_t(*d))
    return lib().moe_ffn_forward_nvfp4(h, T, x, router_w, router_bias, desc(w_gate), desc(w_up),
                                       desc(w_down), desc(d_gate), desc(d_up), desc(d_down),
                                       out, stream)


def moe_ffn_quant_act_nvfp4(rows, K, inp, out, in_scale, stream) -> int:
    return lib().moe_ffn_quant_act_nvfp4(rows, K, inp, out, in_scale, stream)


def moe_ffn_forward_w4a4(h, T, x, router_w, router_bias, w_gate, w_up, w_down, d_gate, d_up,
                         d_down, in_scale, out, stream) -> int:
    """Weight descriptors as for moe_ffn_forward_nvfp4; in_scale a device pointer to 3 fp32."""
    def desc(d):
        if d is None:
            return None
        return ctypes.byref(moe_ffn_nvfp4_t(*d))
    return lib().moe_ffn_forward_w4a4(h, T, x, router_w, router_bias, desc(w_gate), desc(w_up),
                                      desc(w_down), desc(d_gate), desc(d_up), desc(d_down), in_scale,
                                      out, stream)


def moe_ffn_forward_fp8(h, T, x, router_w, router_bias, w_gate, w_up, w_down, d_gate, d_up,
                        d_down, out, stream) -> int:
    """Weight descriptors are (q_ptr, tensor_scale_ptr) tuples or None."""
    def desc(d):
        if d is None:
            return None
        return ctypes.byref(moe_ffn_fp8_t(*d))
    return lib().moe_ffn_forward_fp8(h, T, x, router_w, router_bias, desc(w_gate), desc(w_up),
                                     desc(w_down), desc(d_gate), desc(d_up), desc(d_down), out, stream)


def moe_ffn_forward_block(h, T, x, pre_scale, post_scale, eps, router_w, router_bias, w_gate, w_up,
                          w_down, d_gate, d_up, d_down, out, stream) -> int:
    return lib().moe_ffn_forward_block(h, T, x, pre_scale, post_scale, eps, router_w, router_bias, w_gate,
                                       w_up, w_down, d_gate, d_up, d_down, out, stream)


def moe_ffn_get_routing(h, topk_idx, topk_w, counts, offsets, perm, pos, stream) -> int:
    return lib().moe_ffn_get_routing(h, topk_idx, topk_w, counts, offsets, perm, pos, stream)


def moe_ffn_get_intermediates(h, h_rows, y_rows, h_dense, y_dense, stream) -> int:
    return lib().moe_ffn_get_intermediates(h, h_rows, y_rows, h_dense, y_dense, stream)


def moe_ffn_align_only(h, T, topk_idx, stream) -> int:
    return lib().moe_ffn_align_only(h, T, topk_idx, stream)


def moe_ffn_profile_begin(h, stage_mask: int, max_samples: int) -> int:
    return lib().moe_ffn_profile_begin(h, stage_mask, max_samples)


def moe_ffn_profile_end(h) -> tuple:
    """Returns (rc, [total ms per stage], [timed launches per stage])."""
    ms = (ctypes.c_float * MOE_FFN_NUM_STAGES)()
    n = (ctypes.c_int32 * MOE_FFN_NUM_STAGES)()
    rc = lib().moe_ffn_profile_end(h, ctypes.cast(ms, ctypes.c_void_p), ctypes.cast(n, ctypes.c_void_p))
    return rc, list(ms), list(n)
