"""CPU oracle of the MoE feed-forward block — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against brute force, closed forms, library routines and the parameter counts
printed on the pages; see the docstring of each test.
"""
from .block import (NEAR_TIE_GAP, align, dense_block, dense_ffn, gelu_tanh, geglu, geglu_hidden,
                    moe_block, moe_ffn, moe_ffn_w4a4,
                      moe_ffn_layer_residual, rms_norm, round_bf16, route, router_logits,
                      routed_mixture_dense_mask, select_topk, softmax, widen_bf16)
from .fp8 import dequant_matrix_fp8
from .nvfp4 import (E2M1_TABLE, E4M3_TABLE, dequant_matrix, e2m1_value, e4m3fn_value, quant_act_nvfp4,
                    round_e2m1_sat, round_e4m3_sat)

__all__ = [
    "NEAR_TIE_GAP", "align", "dense_block", "dense_ffn", "gelu_tanh", "geglu", "geglu_hidden", "moe_block", "moe_ffn",
    "moe_ffn_layer_residual", "moe_ffn_w4a4", "quant_act_nvfp4", "round_e2m1_sat",
    "round_e4m3_sat", "rms_norm", "round_bf16", "route", "router_logits",
    "routed_mixture_dense_mask",
    "select_topk", "softmax", "widen_bf16", "E2M1_TABLE", "E4M3_TABLE",
    "dequant_matrix", "dequant_matrix_fp8", "e2m1_value", "e4m3fn_value",
]
