"""CPU oracle of the Gemma 4 26B-A4B MoE feed-forward block (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module; only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
kernels and imports nothing from the product package or from the input
generators.

What the block computes, with the passage each step follows:

* Router logits z = x . W_r (one bias-free [H, E] matrix; the NVFP4
  checkpoint config lists it as ``router.proj`` and keeps it unquantised) —
  plus an optional per-expert logit bias, which only the skewed-load workload
  uses to shape expert loads.
* Gating: softmax over all expert logits (archdb page "Gemma-4-26B-A4B",
  field "Gating function over expert logits": softmax).
* Selection: the top_k_experts = 8 of num_experts = 128 (gemma-llm API page
  ``gm.nn.Gemma4_26B_A4B``, ``TransformerConfig``; archdb fields "Routed
  experts per MoE layer", "Routed experts selected per token").  Equal logits
  go to the lower expert id.
* Renormalisation: the selected softmax weights are divided by their sum
  (archdb field "Selected expert weights are renormalized to sum to 1": Yes).
* Each routed expert is a bias-free GeGLU MLP H -> I -> H with the
  tanh-approximate GELU on the gate projection (archdb fields "FFN
  activation": GeGLU (tanh-approximate GELU), "FFN projections have bias
  terms": No, "Intermediate width of one routed expert": 704; NVFP4 config
  ``hidden_activation: gelu_pytorch_tanh``).
* The always-on dense branch is the same GeGLU form H -> D -> H with
  D = 2112 (API page, model description: one dense MLP branch of
  intermediate width 2112 beside the experts;
  archdb fields "Always-on experts per MoE layer": 1, "Total intermediate
  width of the shared expert(s)": 2,112).
* The block output is the plain sum of the routed mixture and the dense
  branch (the API page lists both branches in every layer; no weighting of
  the dense branch is stated, so its weight is 1).

Precision.  Inputs are bf16 and are widened exactly; all arithmetic is fp64.
One decision is not arithmetic: which experts win.  The HIP path ranks fp32
logits, so the oracle ranks its logits rounded to fp32 too (a decision taken
in the kernel's precision); tokens whose k-th/(k+1)-th logit gap is at most
1e-3 are reported as near-ties because either side may legitimately pick a
different set there.
"""
from __future__ import annotations

import math

import numpy as np

SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_CUBIC = 0.044715
NEAR_TIE_GAP = 1e-3


# ---------------------------------------------------------------------------
# element formats
# ---------------------------------------------------------------------------


def widen_bf16(bits) -> np.ndarray:
    """bf16 raw bits (uint16) -> fp64.  A bf16 value is the top half of an fp32."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        return np.asarray(b, dtype=np.float64)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_bf16(v) -> np.ndarray:
    """Value -> the nearest bf16 value (ties to even), returned as fp64.

    The value is first taken to fp32 (nearest), then its low 16 bits are
    rounded away: a stored bf16 activation is decided in the precision the
    kernels compute it in (fp32).  Finite inputs only.
    """
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def gelu_tanh(v: np.ndarray) -> np.ndarray:
    """tanh approximation of GELU (Hendrycks & Gimpel 2016, eq. for GELU(x)
    ~ 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))))."""
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * (1.0 + np.tanh(SQRT_2_OVER_PI * (v + GELU_CUBIC * v * v * v)))


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------


def router_logits(x: np.ndarray, router_w: np.ndarray, bias=None) -> np.ndarray:
    """z[t, e] = sum_h x[t, h] W_r[h, e] (+ b[e]), fp64."""
    z = widen_bf16(x) @ widen_bf16(router_w)
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)[None, :]
    return z


def softmax(z: np.ndarray) -> np.ndarray:
    """Softmax over the last axis (shifted by the row maximum)."""
    m = np.max(z, axis=-1, keepdims=True)
    ez = np.exp(z - m)
    return ez / np.sum(ez, axis=-1, keepdims=True)


def select_topk(z: np.ndarray, k: int) -> tuple:
    """Top-k expert ids per row, ranked on fp32 logits, lower id wins ties.

    Returns (ids sorted by descending logit, the full ranking).
    """
    zd = np.asarray(z, dtype=np.float64).astype(np.float32)
    T, E = zd.shape
    ids = np.broadcast_to(np.arange(E), (T, E))
    # np.lexsort sorts by the last key first: descending logit, then ascending id
    order = np.lexsort((ids, -zd), axis=-1)
    return order[:, :k], order


def route(x, router_w, k: int, bias=None, force_routing=None) -> dict:
    """Router of the block: logits, top-k selection, softmax, renormalise.

    topk_idx[t] lists the selected experts in ascending id order and topk_w[t]
    their renormalised weights in the same order.  ``force_routing`` replaces
    the selected sets (used for near-tie tokens, where both sets are valid).
    """
    z = router_logits(x, router_w, bias)
    T, E = z.shape
    if force_routing is None:
        sel, order = select_topk(z, k)
    else:
        sel = np.asarray(force_routing, dtype=np.int64).reshape(T, k)
        _, order = select_topk(z, k)
    idx = np.sort(sel, axis=1)
    if k < E:
        rows = np.arange(T)
        gap = z[rows, order[:, k - 1]] - z[rows, order[:, k]]
    else:
        gap = np.full(T, np.inf)
    p = softmax(z)
    ps = np.take_along_axis(p, idx, axis=1)
    w = ps / np.sum(ps, axis=1, keepdims=True)
    return {"z": z, "p": p, "topk_idx": idx.astype(np.int32), "topk_w": w,
            "gap": gap, "near_tie": gap <= NEAR_TIE_GAP}


def align(topk_idx: np.ndarray, num_experts: int) -> dict:
    """Group the (token, slot) pairs by expert: a stable counting sort.

    counts[e]  = number of tokens that selected e
    offsets    = exclusive prefix sum of counts, offsets[E] = T*k
    perm[r]    = token id of row r; rows of expert e are
                 offsets[e] .. offsets[e+1]-1, tokens ascending
    pos[t, j]  = row of slot (t, j), i.e. where token t sits among the rows
                 of expert topk_idx[t, j]
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    counts = np.zeros(num_experts, dtype=np.int64)
    for e in idx.ravel():
        counts[e] += 1
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    for e in range(num_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1].copy()
    perm = np.empty(T * k, dtype=np.int64)
    pos = np.empty((T, k), dtype=np.int64)
    for t in range(T):              # token-major order keeps each expert's
        for j in range(k):          # rows in ascending token order
            e = idx[t, j]
            r = cursor[e]
            perm[r] = t
            pos[t, j] = r
            cursor[e] = r + 1
    return {"counts": counts.astype(np.int32), "offsets": offsets.astype(np.int32),
            "perm": perm.astype(np.int32), "pos": pos.astype(np.int32)}


# ---------------------------------------------------------------------------
# GeGLU MLPs
# ---------------------------------------------------------------------------


def geglu_hidden(X: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray) -> np.ndarray:
    """h = gelu_tanh(X W_gate) * (X W_up); weights are [K, N] matrices."""
    return gelu_tanh(X @ w_gate) * (X @ w_up)


def geglu(X: np.ndarray, w_gate, w_up, w_down) -> tuple:
    """One bias-free GeGLU MLP: returns (hidden, output)."""
    h = geglu_hidden(X, w_gate, w_up)
    return h, h @ w_down


def _matrix(w, g: int) -> np.ndarray:
    """fp64 [K, N] matrix g of a weight stack (bf16 bits, floats, NVFP4 or FP8)."""
    if isinstance(w, dict) and "q8" in w:
        from .fp8 import dequant_matrix_fp8
        return dequant_matrix_fp8(w["q8"][g], w["tensor_scale"][g])
    if isinstance(w, dict):
        from .nvfp4 import dequant_matrix
        return dequant_matrix(w["q"][g], w["scale"][g], w["tensor_scale"][g])
    return widen_bf16(w[g])


def _dense_matrix(w) -> np.ndarray:
    if isinstance(w, dict):
        return _matrix(w, 0)
    return widen_bf16(w)


# ---------------------------------------------------------------------------
# the block
# ---------------------------------------------------------------------------


def moe_ffn(x, router_w, w_gate, w_up, w_down, d_gate=None, d_up=None, d_down=None,
            top_k: int = 8, bias=None, force_routing=None, tokens=None,
            intermediates: bool = True) -> dict:
    """Forward of the MoE feed-forward block.

    x [T, H] (bf16 bits or floats); router_w [H, E]; w_gate, w_up [E, H, I];
    w_down [E, I, H]; d_gate, d_up [H, D]; d_down [D, H] (None: no dense
    branch).  Expert and dense matrices may be NVFP4 packs (dicts with q,
    scale, tensor_scale) or FP8 packs (dicts with q8, tensor_scale), which
    are dequantised first.

    out[t] = sum_j w[t, j] * Expert_{e_j}(x_t) + Dense(x_t), the j-sum in
    ascending j, then the dense term.  With ``tokens`` only those output rows
    are computed (routing is still evaluated for every token).
    """
    X = widen_bf16(x)
    T, H = X.shape
    E = np.asarray(router_w).shape[1]
    r = route(x, router_w, top_k, bias, force_routing)
    a = align(r["topk_idx"], E)
    res = dict(r)
    res.update(a)
    have_dense = d_gate is not None

    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        out = np.zeros((len(tokens), H))
        cache = {}  # expert -> its three fp64 matrices (each decoded once per call)

        def mats(e):
            if e not in cache:
                cache[e] = (_matrix(w_gate, e), _matrix(w_up, e), _matrix(w_down, e))
            return cache[e]

        dense_m = ((_dense_matrix(d_gate), _dense_matrix(d_up), _dense_matrix(d_down))
                   if have_dense else None)
        for i, t in enumerate(tokens):
            acc = np.zeros(H)
            for j in range(top_k):
                e = int(r["topk_idx"][t, j])
                _, ye = geglu(X[t:t + 1], *mats(e))
                acc += r["topk_w"][t, j] * ye[0]
            if have_dense:
                _, yd = geglu(X[t:t + 1], *dense_m)
                acc += yd[0]
            out[i] = acc
        res["out"] = out
        res["tokens"] = tokens
        return res

    if isinstance(w_down, dict) and "q8" in w_down:
        I = w_down["q8"].shape[1]
    elif isinstance(w_down, dict):
        I = w_down["q"].shape[2] * 2
    else:
        I = np.asarray(w_down).shape[1]
    rows = T * top_k
    h = np.zeros((rows, I)) if intermediates else None
    y = np.zeros((rows, H))
    offsets, perm = a["offsets"], a["perm"]
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        Xe = X[perm[lo:hi]]
        he, ye = geglu(Xe, _matrix(w_gate, e), _matrix(w_up, e), _matrix(w_down, e))
        if intermediates:
            h[lo:hi] = he
        y[lo:hi] = ye
    if have_dense:
        h_d, y_d = geglu(X, _dense_matrix(d_gate), _dense_matrix(d_up), _dense_matrix(d_down))
    else:
        h_d, y_d = None, np.zeros((T, H))
    out = np.zeros((T, H))
    pos, w = a["pos"], r["topk_w"]
    for j in range(top_k):
        out += w[:, j:j + 1] * y[pos[:, j]]
    out += y_d
    res.update({"out": out, "h": h, "y": y, "h_d": h_d, "y_d": y_d})
    return res


# ---------------------------------------------------------------------------
# the sub-block with its sandwich norms
# ---------------------------------------------------------------------------


def rms_norm(v, scale, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: v / sqrt(mean(v^2) + eps) * scale.

    archdb page "Gemma-4-26B-A4B", fields "Normalization layer type in the
    blocks" (RMSNorm) and "Epsilon of the block normalization layers" (1e-06).
    ``scale`` is the per-channel gain as applied (any offset a checkpoint
    stores it with is the caller's).
    """
    V = np.asarray(v, dtype=np.float64)
    return V / np.sqrt(np.mean(V * V, axis=-1, keepdims=True) + eps) * np.asarray(scale, dtype=np.float64)


def moe_block(x, pre_scale, post_scale, eps: float, router_w, w_gate, w_up, w_down, d_gate=None,
              d_up=None, d_down=None, top_k: int = 8, bias=None, force_routing=None, tokens=None) -> dict:
    """The feed-forward sub-block with sandwich norms and the residual.

    archdb field "Pre-norm, post-norm, or sandwich (pre and post)": sandwich;
    API page gm.nn.Gemma4_26B_A4B ``use_post_ffw_norm=True``.  Reading taken
    here (the pages show one norm before and one after the block, not one per
    branch): a single pre-norm feeds the router, the experts and the dense
    branch, a single post-norm acts on their sum, and the residual adds the
    block input:

        xn  = bf16(RMSNorm(x) * pre_scale)      (a stored bf16 activation)
        out = x + RMSNorm(moe_ffn(xn)) * post_scale

    Returns the moe_ffn details of xn plus ``xn``, ``ffn`` (the block's
    pre-norm output rows) and ``out``; with ``tokens`` only those rows.
    """
    X = widen_bf16(x)
    xn = round_bf16(rms_norm(X, pre_scale, eps))
    r = moe_ffn(xn, router_w, w_gate, w_up, w_down, d_gate, d_up, d_down, top_k=top_k, bias=bias,
                force_routing=force_routing, tokens=tokens, intermediates=tokens is None)
    f = r["out"]
    rows = X if tokens is None else X[np.asarray(tokens, dtype=np.int64)]
    r["xn"] = xn
    r["ffn"] = f
    r["out"] = rows + rms_norm(f, post_scale, eps)
    return r


# ---------------------------------------------------------------------------
# W4A4: NVFP4 weights and NVFP4 activations
# ---------------------------------------------------------------------------


def moe_ffn_w4a4(x, router_w, w_gate, w_up, w_down, d_gate, d_up, d_down, in_scale,
                 top_k: int = 8, bias=None, force_routing=None, tokens=None) -> dict:
    """The block with NVFP4 weights and NVFP4 activations at every Linear
    input (checkpoint config ``input_activations``; readings in
    ``oracle.nvfp4``).  The router is not quantised (``ignore`` lists
    ``router.proj``) and reads x as it is.

    in_scale = (s_x, s_h, s_hd): the static global scales of x (input of
    every gate/up projection), of the routed hidden rows h (bf16, as stored)
    and of the dense hidden rows h_d.  Each expert:
        h = bf16(gelu_tanh(q(x)·W_g[e]) ⊙ (q(x)·W_u[e])),  y = q(h)·W_d[e]
    with q the quantise-dequantise of ``quant_act_nvfp4`` times its scale.
    """
    from .nvfp4 import quant_act_nvfp4

    s_x, s_h, s_hd = (float(np.float32(s)) for s in in_scale)
    X = widen_bf16(x)
    T, H = X.shape
    E = np.asarray(router_w).shape[1]
    r = route(x, router_w, top_k, bias, force_routing)
    res = dict(r)
    XQ = quant_act_nvfp4(X, s_x) * s_x
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    cache = {}

    def mats(e):
        if e not in cache:
            cache[e] = (_matrix(w_gate, e), _matrix(w_up, e), _matrix(w_down, e))
        return cache[e]

    def hidden_q(xq, g, u, s):
        h = round_bf16(geglu_hidden(xq, g, u))                   # the stored bf16 hidden rows
        return quant_act_nvfp4(h, s) * s

    out = np.zeros((len(toks), H))
    have_dense = d_gate is not None
    if have_dense:
        dg, du, dd = _dense_matrix(d_gate), _dense_matrix(d_up), _dense_matrix(d_down)
        yd = hidden_q(XQ[toks], dg, du, s_hd) @ dd
    for i, t in enumerate(toks):
        acc = np.zeros(H)
        for j in range(top_k):
            e = int(r["topk_idx"][t, j])
            g, u, dwn = mats(e)
            acc += r["topk_w"][t, j] * (hidden_q(XQ[t:t + 1], g, u, s_h) @ dwn)[0]
        if have_dense:
            acc += yd[i]
        out[i] = acc
    res["out"] = out
    res["xq"] = XQ
    res["tokens"] = toks
    return res


# ---------------------------------------------------------------------------
# the dense FFN of the E4B sibling
# ---------------------------------------------------------------------------


def dense_ffn(x, d_gate, d_up, d_down, tokens=None) -> dict:
    """Feed-forward block of a model without experts: one GeGLU MLP H -> D -> H.

    gemma-llm API page gm.nn.Gemma4_E4B, ``TransformerConfig``: embed_dim
    2560, hidden_dim 10240, enable_moe False, num_experts 0, expert_dim 0.
    The page does not name the activation; the family's tanh-approximate GeGLU
    (the 26B-A4B's) is taken.  x [T, H]; d_gate, d_up [H, D]; d_down [D, H]
    (bf16 bits, floats or NVFP4 packs).  Returns h_d, y_d and out (= y_d);
    with ``tokens`` only those rows (and no h_d).
    """
    X = widen_bf16(x)
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        X = X[tokens]
    h_d, y_d = geglu(X, _dense_matrix(d_gate), _dense_matrix(d_up), _dense_matrix(d_down))
    return {"h_d": None if tokens is not None else h_d, "y_d": y_d, "out": y_d, "tokens": tokens}


def dense_block(x, pre_scale, post_scale, eps: float, d_gate, d_up, d_down, tokens=None) -> dict:
    """The dense FFN with the sandwich norms and the residual (API page
    gm.nn.Gemma4_E4B ``use_post_ffw_norm=True``), read as for the MoE block:

        xn  = bf16(RMSNorm(x) * pre_scale)
        out = x + RMSNorm(dense_ffn(xn)) * post_scale
    """
    X = widen_bf16(x)
    xn = round_bf16(rms_norm(X, pre_scale, eps))
    r = dense_ffn(xn, d_gate, d_up, d_down, tokens=tokens)
    f = r["out"]
    rows = X if tokens is None else X[np.asarray(tokens, dtype=np.int64)]
    r["xn"] = xn
    r["ffn"] = f
    r["out"] = rows + rms_norm(f, post_scale, eps)
    return r


def moe_ffn_layer_residual(x, weights: dict, top_k: int, bias=None) -> tuple:
    """One layer of a residual stack without attention: (x + FFN(x), details).

    ``weights`` holds router, gate, up, down, dgate, dup, ddown.  Normalisation
    layers around the block are not part of this stack.
    """
    r = moe_ffn(x, weights["router"], weights["gate"], weights["up"], weights["down"],
                weights.get("dgate"), weights.get("dup"), weights.get("ddown"),
                top_k=top_k, bias=bias, intermediates=False)
    return widen_bf16(x) + r["out"], r


def routed_mixture_dense_mask(x, router_w, w_gate, w_up, w_down, top_k: int,
                              bias=None) -> np.ndarray:
    """Routed branch by brute force: every expert on every token, weighted by a
    dense [T, E] weight matrix that is zero outside the selected set.

    Independent of ``align`` (no grouping or permutation); used to pin it.
    """
    X = widen_bf16(x)
    T, H = X.shape
    E = np.asarray(router_w).shape[1]
    r = route(x, router_w, top_k, bias)
    W = np.zeros((T, E))
    np.put_along_axis(W, r["topk_idx"].astype(np.int64), r["topk_w"], axis=1)
    acc = np.zeros((T, H))
    for e in range(E):
        _, ye = geglu(X, _matrix(w_gate, e), _matrix(w_up, e), _matrix(w_down, e))
        acc += W[:, e:e + 1] * ye
    return acc
