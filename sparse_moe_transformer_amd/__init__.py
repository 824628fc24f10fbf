"""MI355X-native MoE feed-forward block (Gemma 4 26B-A4B shape).

The compute lives in ``libmoe_ffn.so`` (hand-written HIP kernels for gfx950
behind the C ABI in ``include/moe_ffn.h``).  ``binding`` mirrors the C entry
points one to one; ``MoeFFN`` below is a small convenience layer that takes
torch tensors, passes their device pointers and torch's current stream, and
raises on error codes.  torch is used for device memory and streams only.
"""
from __future__ import annotations

from . import binding
from .binding import (MOE_FFN_ACCUMULATE, MOE_FFN_VARIANT_AUTO, MOE_FFN_VARIANT_MFMA,
                      MOE_FFN_VARIANT_STREAM, MOE_FFN_W_BF16, MOE_FFN_W_FP8, MOE_FFN_W_NVFP4, MoeFFNError,
                      check)

__all__ = ["MoeFFN", "binding", "MoeFFNError", "MOE_FFN_ACCUMULATE", "MOE_FFN_VARIANT_AUTO",
           "MOE_FFN_VARIANT_MFMA", "MOE_FFN_VARIANT_STREAM", "MOE_FFN_W_BF16", "MOE_FFN_W_FP8", "MOE_FFN_W_NVFP4"]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


class MoeFFN:
    """One handle of the block: a fixed shape and its device workspace."""

    def __init__(self, hidden, num_experts, top_k, expert_dim, dense_dim, max_tokens,
                 weight_format=MOE_FFN_W_BF16, accumulate=False, variant=MOE_FFN_VARIANT_AUTO):
        self.cfg = binding.make_config(hidden, num_experts, top_k, expert_dim, dense_dim, max_tokens,
                                       weight_format, MOE_FFN_ACCUMULATE if accumulate else 0)
        rc, h = binding.moe_ffn_create(self.cfg)
        check(rc)
        self.h = h
        self.set_variant(variant)

    @classmethod
    def for_shape(cls, shape, max_tokens=None, **kw):
        fmt = (MOE_FFN_W_NVFP4 if getattr(shape, "nvfp4", False)
               else MOE_FFN_W_FP8 if getattr(shape, "fp8", False) else MOE_FFN_W_BF16)
        return cls(shape.hidden, shape.experts, shape.top_k, shape.expert_dim, shape.dense_dim,
                   max_tokens or shape.tokens, weight_format=fmt, **kw)

    def set_variant(self, variant):
        check(binding.moe_ffn_set_variant(self.h, variant))

    def close(self):
        if self.h:
            binding.moe_ffn_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward(self, x, w, out, bias=None):
        """x [T, H] bf16; w: dict of bf16 tensors router, gate, up, down, dgate, dup, ddown
        (missing or None: absent, as in a config without experts)."""
        T = x.shape[0]
        check(binding.moe_ffn_forward(self.h, T, _ptr(x), _ptr(w.get("router")), _ptr(bias),
                                      _ptr(w.get("gate")), _ptr(w.get("up")), _ptr(w.get("down")),
                                      _ptr(w.get("dgate")), _ptr(w.get("dup")), _ptr(w.get("ddown")),
                                      _ptr(out), _stream()))
        return out

    def forward_block(self, x, w, pre_scale, post_scale, out, eps=1e-6, bias=None):
        """The sub-block with sandwich norms: out = x + RMSNorm(FFN(bf16(RMSNorm(x) * pre))) * post.
        pre_scale/post_scale: [H] fp32 tensors; out may be x."""
        T = x.shape[0]
        check(binding.moe_ffn_forward_block(self.h, T, _ptr(x), _ptr(pre_scale), _ptr(post_scale), float(eps),
                                            _ptr(w.get("router")), _ptr(bias), _ptr(w.get("gate")), _ptr(w.get("up")),
                                            _ptr(w.get("down")), _ptr(w.get("dgate")), _ptr(w.get("dup")),
                                            _ptr(w.get("ddown")), _ptr(out), _stream()))
        return out

    def forward_nvfp4(self, x, w, out, bias=None):
        """w: router bf16 tensor; gate/up/down/dgate/dup/ddown dicts of q, scale, tensor_scale."""
        def d(m):
            if m is None:
                return None
            return (m["q"].data_ptr(), m["scale"].data_ptr(), m["tensor_scale"].data_ptr())
        T = x.shape[0]
        check(binding.moe_ffn_forward_nvfp4(self.h, T, _ptr(x), _ptr(w.get("router")), _ptr(bias),
                                            d(w.get("gate")), d(w.get("up")), d(w.get("down")),
                                            d(w.get("dgate")), d(w.get("dup")), d(w.get("ddown")),
                                            _ptr(out), _stream()))
        return out

    def forward_w4a4(self, x, w, in_scale, out, bias=None):
        """NVFP4 weights (as forward_nvfp4) and NVFP4 activations; in_scale: fp32 device
        tensor [3] (global scales of x, h, h_d)."""
        def d(m):
            if m is None:
                return None
            return (m["q"].data_ptr(), m["scale"].data_ptr(), m["tensor_scale"].data_ptr())
        T = x.shape[0]
        check(binding.moe_ffn_forward_w4a4(self.h, T, _ptr(x), _ptr(w.get("router")), _ptr(bias),
                                           d(w.get("gate")), d(w.get("up")), d(w.get("down")),
                                           d(w.get("dgate")), d(w.get("dup")), d(w.get("ddown")),
                                           _ptr(in_scale), _ptr(out), _stream()))
        return out

    def forward_fp8(self, x, w, out, bias=None):
        """w: router bf16 tensor; gate/up/down/dgate/dup/ddown dicts of q8 (uint8 [G, K, N])
        and tensor_scale (fp32 [G]), or None where the config has no such matrices."""
        def d(m):
            if m is None:
                return None
            return (m["q8"].data_ptr(), m["tensor_scale"].data_ptr())
        T = x.shape[0]
        check(binding.moe_ffn_forward_fp8(self.h, T, _ptr(x), _ptr(w.get("router")), _ptr(bias),
                                          d(w.get("gate")), d(w.get("up")), d(w.get("down")),
                                          d(w.get("dgate")), d(w.get("dup")), d(w.get("ddown")),
                                          _ptr(out), _stream()))
        return out

    def routing(self, T):
        """Routing tables of the last forward (or align_only) as new device tensors."""
        import torch
        k, E = self.cfg.top_k, self.cfg.num_experts
        dev = torch.device("cuda", torch.cuda.current_device())
        r = {"topk_idx": torch.empty((T, k), dtype=torch.int32, device=dev),
             "topk_w": torch.empty((T, k), dtype=torch.float32, device=dev),
             "counts": torch.empty((E,), dtype=torch.int32, device=dev),
             "offsets": torch.empty((E + 1,), dtype=torch.int32, device=dev),
             "perm": torch.empty((T * k,), dtype=torch.int32, device=dev),
             "pos": torch.empty((T, k), dtype=torch.int32, device=dev)}
        check(binding.moe_ffn_get_routing(self.h, *(_ptr(r[n]) for n in
                                                     ("topk_idx", "topk_w", "counts", "offsets",
                                                      "perm", "pos")), _stream()))
        return r

    def intermediates(self, T):
        import torch
        c = self.cfg
        dev = torch.device("cuda", torch.cuda.current_device())
        bf = torch.bfloat16
        r = {"h": torch.empty((T * c.top_k, c.expert_dim), dtype=bf, device=dev),
             "y": torch.empty((T * c.top_k, c.hidden), dtype=bf, device=dev),
             "h_d": torch.empty((T, max(c.dense_dim, 1)), dtype=bf, device=dev),
             "y_d": torch.empty((T, c.hidden), dtype=bf, device=dev)}
        check(binding.moe_ffn_get_intermediates(self.h, _ptr(r["h"]), _ptr(r["y"]),
                                                _ptr(r["h_d"]) if c.dense_dim else None,
                                                _ptr(r["y_d"]), _stream()))
        return r

    def align_only(self, topk_idx):
        check(binding.moe_ffn_align_only(self.h, topk_idx.shape[0], _ptr(topk_idx), _stream()))
