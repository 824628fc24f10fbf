"""Planted mistakes in the CPU oracle must be caught by its pins.

Each case swaps one oracle function for a plausibly wrong version (a sign
flip, a dropped term, a swapped operand or index, a wrong tie-break, a wrong
bit field) on the CPU, runs the pins that should notice, and expects at least
one of them to fail.  Nothing here touches the GPU path.
"""
import numpy as np
import pytest

import oracle
import oracle.block as om
import oracle.nvfp4 as on
from tests import test_oracle_pins as pins


def _patch(monkeypatch, name, fn, module=om):
    monkeypatch.setattr(module, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)


def _expect_caught(tests):
    failures = 0
    for t in tests:
        try:
            t()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, "planted mistake went unnoticed"


ROUTING_PINS = [pins.test_routing_sets_match_brute_force_tiny,
                pins.test_routing_tie_break_lowest_index,
                pins.test_routing_weights_closed_form,
                pins.test_routing_k1_and_kE]
BLOCK_PINS = [pins.test_routed_branch_equals_dense_mask_brute_force,
              pins.test_dense_branch_is_torch_geglu_mlp,
              pins.test_single_expert_is_torch_geglu_mlp,
              pins.test_identical_experts_give_one_expert,
              pins.test_k_equals_E_is_full_softmax_mixture,
              pins.test_zero_input_gives_zero_output]


def test_gelu_cubic_sign(monkeypatch):
    _patch(monkeypatch, "gelu_tanh", lambda v: 0.5 * np.asarray(v) * (
        1 + np.tanh(om.SQRT_2_OVER_PI * (np.asarray(v) - om.GELU_CUBIC * np.asarray(v) ** 3))))
    _expect_caught([pins.test_gelu_matches_torch_tanh_gelu] + BLOCK_PINS)


def test_gelu_on_up_instead_of_gate(monkeypatch):
    _patch(monkeypatch, "geglu_hidden", lambda X, g, u: (X @ g) * om.gelu_tanh(X @ u))
    _expect_caught(BLOCK_PINS)


def test_missing_renormalisation(monkeypatch):
    real = om.route

    def bad(*a, **k):
        r = real(*a, **k)
        r["topk_w"] = np.take_along_axis(r["p"], r["topk_idx"].astype(np.int64), axis=1)
        return r

    _patch(monkeypatch, "route", bad)
    _expect_caught(ROUTING_PINS + BLOCK_PINS)


def test_bottom_k_selection(monkeypatch):
    def bad(z, k):
        zd = np.asarray(z).astype(np.float32)
        order = np.lexsort((np.broadcast_to(np.arange(zd.shape[1]), zd.shape), zd), axis=-1)
        return order[:, :k], order

    _patch(monkeypatch, "select_topk", bad)
    _expect_caught(ROUTING_PINS)


def test_highest_index_tie_break(monkeypatch):
    def bad(z, k):
        zd = np.asarray(z).astype(np.float32)
        order = np.lexsort((-np.broadcast_to(np.arange(zd.shape[1]), zd.shape), -zd), axis=-1)
        return order[:, :k], order

    _patch(monkeypatch, "select_topk", bad)
    _expect_caught(ROUTING_PINS)


def test_align_descending_tokens(monkeypatch):
    real = om.align

    def bad(idx, E):
        a = real(idx, E)
        perm = a["perm"].copy()
        for e in range(E):
            lo, hi = a["offsets"][e], a["offsets"][e + 1]
            perm[lo:hi] = perm[lo:hi][::-1]
        a["perm"] = perm
        return a

    _patch(monkeypatch, "align", bad)
    _expect_caught([lambda: pins.test_align_matches_stable_argsort(32, 8, 2)])


def test_combine_uses_perm_not_pos(monkeypatch):
    real_align = om.align

    def bad(idx, E):
        a = real_align(idx, E)
        T, k = np.asarray(idx).shape
        a["pos"] = np.arange(T * k).reshape(T, k).astype(np.int32)
        return a

    _patch(monkeypatch, "align", bad)
    _expect_caught(BLOCK_PINS)


def test_dropped_dense_term(monkeypatch):
    real = om.geglu
    calls = {"n": 0}

    def bad(X, g, u, d):
        h, y = real(X, g, u, d)
        # the dense branch is the call with the whole token batch and a
        # dense-width hidden layer; drop its output
        if np.asarray(g).shape[1] == 128:
            calls["n"] += 1
            return h, np.zeros_like(y)
        return h, y

    _patch(monkeypatch, "geglu", bad)
    _expect_caught([pins.test_dense_branch_is_torch_geglu_mlp])
    assert calls["n"] > 0


def test_transposed_down_operand(monkeypatch):
    real = om._matrix

    def bad(w, g):
        m = real(w, g)
        if m.shape[0] == m.shape[1]:
            return m.T
        return m

    # on a square-shaped variant the slip is silent to numpy; use the tiny
    # block with I == H to make it plausible and check the pins catch it
    monkeypatch.setattr(om, "_matrix", bad)
    import synth
    shape = synth.FFNShape("sq", 16, 64, 4, 2, 64, 64)
    x = synth.make_x(shape)
    w = synth.make_weights(shape)
    r = om.moe_ffn(x, w["router"], w["gate"], w["up"], w["down"], top_k=2)
    monkeypatch.undo()
    bf = om.routed_mixture_dense_mask(x, w["router"], w["gate"], w["up"], w["down"], 2)
    assert np.max(np.abs(r["out"] - bf)) > 1e-6


def test_e4m3_wrong_bias(monkeypatch):
    def bad(b):
        b = int(b) & 0xFF
        e, m = (b >> 3) & 0xF, b & 7
        s = -1.0 if b >> 7 else 1.0
        if e == 15 and m == 7:
            return float("nan")
        return s * ((m / 8) * 2.0 ** -7 if e == 0 else (1 + m / 8) * 2.0 ** (e - 8))

    table = np.array([bad(b) for b in range(256)])
    monkeypatch.setattr(on, "E4M3_TABLE", table)
    monkeypatch.setattr(oracle, "E4M3_TABLE", table)
    _expect_caught([pins.test_e4m3_decoder_matches_torch_all_codes,
                    pins.test_nvfp4_dequant_layout_and_roundtrip])


def test_nibble_order_swapped(monkeypatch):
    def bad(q):
        q = np.asarray(q, dtype=np.uint8)
        N, KH = q.shape
        c = np.empty((N, 2 * KH), dtype=np.uint8)
        c[:, 0::2] = q >> 4
        c[:, 1::2] = q & 0xF
        return c

    monkeypatch.setattr(on, "unpack_codes", bad)
    _expect_caught([pins.test_nvfp4_dequant_layout_and_roundtrip])


@pytest.mark.parametrize("exp_bias", [0, 2])
def test_e2m1_wrong_exponent_bias(monkeypatch, exp_bias):
    def bad(code):
        code = int(code) & 0xF
        s = -1.0 if code >> 3 else 1.0
        e, m = (code >> 1) & 3, code & 1
        return s * ((m / 2) * 2.0 ** (1 - exp_bias) if e == 0 else (1 + m / 2) * 2.0 ** (e - exp_bias))

    monkeypatch.setattr(on, "e2m1_value", bad)
    monkeypatch.setattr(oracle, "e2m1_value", bad)
    _expect_caught([pins.test_e2m1_decoder_matches_ocp_table])


NORM_PINS = [pins.test_rms_norm_matches_torch_rms_norm,
             pins.test_rms_norm_unit_rms_and_constant_rows]
SANDWICH_PINS = [pins.test_block_with_zero_post_gain_is_identity,
                 pins.test_block_prenorm_removes_input_scale,
                 pins.test_block_is_norm_ffn_norm_residual_with_torch_norms]


def test_rms_norm_sum_instead_of_mean(monkeypatch):
    def bad(v, scale, eps):
        V = np.asarray(v, dtype=np.float64)
        return V / np.sqrt(np.sum(V * V, axis=-1, keepdims=True) + eps) * np.asarray(scale)

    _patch(monkeypatch, "rms_norm", bad)
    _expect_caught(NORM_PINS + SANDWICH_PINS)


def test_rms_norm_dropped_eps(monkeypatch):
    def bad(v, scale, eps):
        V = np.asarray(v, dtype=np.float64)
        return V / np.sqrt(np.mean(V * V, axis=-1, keepdims=True)) * np.asarray(scale)

    _patch(monkeypatch, "rms_norm", bad)
    _expect_caught(NORM_PINS)


def test_bf16_truncation_instead_of_nearest(monkeypatch):
    def bad(v):
        f = np.asarray(v, dtype=np.float64).astype(np.float32)
        b = f.view(np.uint32) & np.uint32(0xFFFF0000)
        return b.view(np.float32).astype(np.float64)

    _patch(monkeypatch, "round_bf16", bad)
    _expect_caught([pins.test_round_bf16_matches_torch_cast] + SANDWICH_PINS)


def test_post_norm_after_the_residual(monkeypatch):
    real = om.moe_block

    def bad(x, pre, post, eps, *a, **k):
        r = real(x, pre, np.ones_like(np.asarray(post, dtype=np.float64)), eps, *a, **k)
        X = om.widen_bf16(x)
        rows = X if k.get("tokens") is None else X[np.asarray(k["tokens"], dtype=np.int64)]
        r["out"] = om.rms_norm(rows + r["ffn"], post, eps)
        return r

    _patch(monkeypatch, "moe_block", bad)
    _expect_caught(SANDWICH_PINS)


def test_missing_pre_norm(monkeypatch):
    real_round = om.round_bf16

    def bad(x, pre, post, eps, router_w, w_gate, w_up, w_down, d_gate=None, d_up=None, d_down=None,
            top_k=8, bias=None, force_routing=None, tokens=None):
        X = om.widen_bf16(x)
        xn = real_round(X)
        r = om.moe_ffn(xn, router_w, w_gate, w_up, w_down, d_gate, d_up, d_down, top_k=top_k, bias=bias,
                       force_routing=force_routing, tokens=tokens)
        rows = X if tokens is None else X[np.asarray(tokens, dtype=np.int64)]
        r["xn"], r["ffn"] = xn, r["out"]
        r["out"] = rows + om.rms_norm(r["ffn"], post, eps)
        return r

    _patch(monkeypatch, "moe_block", bad)
    _expect_caught(SANDWICH_PINS)


DENSE_FFN_PINS = [pins.test_dense_ffn_is_torch_geglu_mlp,
                  pins.test_dense_ffn_token_rows_and_independence,
                  pins.test_dense_ffn_is_moe_block_dense_branch,
                  pins.test_dense_block_torch_norms_and_zero_post_gain]


def test_dense_ffn_gate_and_up_swapped(monkeypatch):
    real = om.dense_ffn

    def bad(x, d_gate, d_up, d_down, tokens=None):
        return real(x, d_up, d_gate, d_down, tokens=tokens)

    _patch(monkeypatch, "dense_ffn", bad)
    _expect_caught(DENSE_FFN_PINS)


def test_dense_ffn_erf_gelu(monkeypatch):
    from math import erf

    verf = np.vectorize(erf)

    def bad(x, d_gate, d_up, d_down, tokens=None):
        X = om.widen_bf16(x)
        if tokens is not None:
            X = X[np.asarray(tokens, dtype=np.int64)]
        G = X @ om._dense_matrix(d_gate)
        h = 0.5 * G * (1.0 + verf(G / np.sqrt(2.0))) * (X @ om._dense_matrix(d_up))
        y = h @ om._dense_matrix(d_down)
        return {"h_d": h, "y_d": y, "out": y, "tokens": tokens}

    _patch(monkeypatch, "dense_ffn", bad)
    _expect_caught(DENSE_FFN_PINS)


def test_dense_ffn_row_mixing(monkeypatch):
    real = om.dense_ffn

    def bad(x, d_gate, d_up, d_down, tokens=None):
        r = real(x, d_gate, d_up, d_down, tokens=tokens)
        r["out"] = r["out"] + 1e-3 * np.roll(r["out"], 1, axis=0)
        return r

    _patch(monkeypatch, "dense_ffn", bad)
    _expect_caught(DENSE_FFN_PINS)


def test_fp8_scale_dropped(monkeypatch):
    import oracle.fp8 as of

    _patch(monkeypatch, "dequant_matrix_fp8", lambda q, st: on.E4M3_TABLE[np.asarray(q, dtype=np.uint8)],
           module=of)
    _expect_caught([pins.test_fp8_dequant_matches_torch_and_layout])


def test_fp8_transposed_layout(monkeypatch):
    import oracle.fp8 as of

    real = of.dequant_matrix_fp8

    def bad(q, st):
        q = np.asarray(q)
        return real(q.reshape(q.shape[::-1]).T, st)  # reads the bytes as [N, K]

    _patch(monkeypatch, "dequant_matrix_fp8", bad, module=of)
    _expect_caught([pins.test_fp8_dequant_matches_torch_and_layout])


W4A4_PINS = [pins.test_e2m1_rounding_is_nearest_with_even_ties,
             pins.test_activation_quantiser_worked_group,
             pins.test_activation_quantiser_properties,
             pins.test_w4a4_block_composition_with_torch]


def test_e2m1_ties_away_from_zero(monkeypatch):
    def bad(r):
        r = np.asarray(r, dtype=np.float64)
        a = np.abs(r)
        up = np.floor  # ties (and everything) rounded half up
        v = np.where(a < 2.0, up(a * 2.0 + 0.5) / 2.0, np.where(a < 4.0, up(a + 0.5), 2.0 * up(a / 2.0 + 0.5)))
        return np.sign(r) * np.minimum(v, 6.0)

    _patch(monkeypatch, "round_e2m1_sat", bad, module=on)
    _expect_caught(W4A4_PINS)


def test_activation_scale_ignores_global_scale(monkeypatch):
    real = on.round_e4m3_sat

    def bad_quant(v, s_in):
        v = np.asarray(v, dtype=np.float64)
        sh = v.shape
        g = v.reshape(*sh[:-1], sh[-1] // 16, 16)
        sg = real(np.max(np.abs(g), axis=-1) / 6.0)              # global scale left out
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(sg[..., None] > 0, on.round_e2m1_sat(g / sg[..., None]), 0.0)
        return (q * sg[..., None]).reshape(sh)

    _patch(monkeypatch, "quant_act_nvfp4", bad_quant, module=on)
    _expect_caught(W4A4_PINS)


def test_w4a4_hidden_not_rounded_to_bf16(monkeypatch):
    monkeypatch.setattr(om, "round_bf16", lambda v: np.asarray(v, dtype=np.float64))
    _expect_caught([pins.test_w4a4_block_composition_with_torch])
