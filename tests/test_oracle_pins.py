"""Pins of the CPU oracle against things other than itself.

Each test fixes part of the oracle with brute force, a closed form, a library
routine, an invariant of the method, or values printed on the pages, chosen so
that a plausible slip (a dropped term, a wrong sign or index, a transposed
operand) fails at least one of them (``test_oracle_mutations.py`` plants such
slips and checks that these pins catch them).
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_inputs(seed=0, T=None, shape=synth.TINY):
    if T is not None:
        shape = shape.with_tokens(T)
    x = synth.make_x(shape, seed)
    w = synth.make_weights(shape, seed)
    return shape, x, w


def run(shape, x, w, **kw):
    return oracle.moe_ffn(x, w["router"], w["gate"], w["up"], w["down"], w["dgate"], w["dup"],
                          w["ddown"], top_k=kw.pop("top_k", shape.top_k), **kw)


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b)))


# ---------------------------------------------------------------------------
# GELU, softmax: library routines and closed forms
# ---------------------------------------------------------------------------


def test_gelu_matches_torch_tanh_gelu():
    """Pin: torch.nn.functional.gelu(approximate='tanh') in fp64 is the same
    function (the NVFP4 config names it gelu_pytorch_tanh)."""
    v = np.linspace(-12, 12, 20001)
    ref = torch.nn.functional.gelu(torch.from_numpy(v), approximate="tanh").numpy()
    assert np.max(np.abs(oracle.gelu_tanh(v) - ref)) < 1e-14


def test_gelu_odd_identity_and_limits():
    """Pin: gelu(v) - gelu(-v) = v exactly in real arithmetic (tanh is odd);
    gelu(0) = 0; gelu(v) -> v for large v and -> 0 for very negative v."""
    v = np.linspace(-30, 30, 6001)
    assert np.max(np.abs(oracle.gelu_tanh(v) - oracle.gelu_tanh(-v) - v)) < 1e-13
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert abs(oracle.gelu_tanh(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(oracle.gelu_tanh(np.array([-40.0]))[0]) < 1e-12
    # the cubic term: at v=1 the tanh argument is sqrt(2/pi) * 1.044715
    t = np.tanh(np.sqrt(2 / np.pi) * 1.044715)
    assert abs(oracle.gelu_tanh(np.array([1.0]))[0] - 0.5 * (1 + t)) < 1e-15


def test_softmax_matches_scipy():
    """Pin: scipy.special.softmax."""
    from scipy.special import softmax as sp_softmax
    z = np.random.default_rng(1).standard_normal((16, 128)) * 3
    assert np.max(np.abs(oracle.softmax(z) - sp_softmax(z, axis=-1))) < 1e-15


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------


def brute_force_sets(z, k):
    """Enumerate every k-subset; keep the one with the largest fp32 logit sum.

    Subsets are visited in lexicographic order and only a strictly larger sum
    replaces the incumbent, so equal sums go to the lexicographically smallest
    (lower-id) subset.
    """
    zd = z.astype(np.float32).astype(np.float64)
    T, E = zd.shape
    out = []
    for t in range(T):
        best, best_s = None, -np.inf
        for s in itertools.combinations(range(E), k):
            v = zd[t, list(s)].sum()
            if v > best_s:
                best, best_s = s, v
        out.append(best)
    return np.array(out)


def test_routing_sets_match_brute_force_tiny():
    """Pin: top-k = the subset with the largest logit sum (all C(8,2)=28
    subsets enumerated on the tiny workload, and C(8,3), C(8,4) variants)."""
    shape, x, w = tiny_inputs()
    for k in (2, 3, 4):
        r = oracle.route(x, w["router"], k)
        bf = brute_force_sets(r["z"], k)
        assert np.array_equal(r["topk_idx"], bf)


def test_routing_tie_break_lowest_index():
    """Pin: equal logits go to the lower expert id (x = 0 makes every logit
    0, so the selected set is {0..k-1}); duplicated router columns a < b at
    the k boundary select a."""
    shape, x, w = tiny_inputs()
    z0 = np.zeros_like(x)
    r = oracle.route(z0, w["router"], 2)
    assert np.all(r["topk_idx"] == np.array([0, 1]))
    assert np.allclose(r["topk_w"], 0.5)
    # duplicated router columns 2 and 5 plus an equal large bias, so that
    # they lead every token with bit-identical logits: k=1 must pick 2
    wr = w["router"].copy()
    wr[:, 5] = wr[:, 2]
    b = np.zeros(8, dtype=np.float32)
    b[[2, 5]] = 100.0
    r1 = oracle.route(x, wr, 1, bias=b)
    assert np.all(r1["z"][:, 2] == r1["z"][:, 5])
    assert np.all(r1["topk_idx"][:, 0] == 2)
    r2 = oracle.route(x, wr, 2, bias=b)
    assert np.all(r2["topk_idx"] == np.array([2, 5]))
    assert np.allclose(r2["topk_w"], 0.5)
    # ties on hand-made logits: ranks (-z, id)
    z = np.array([[1.0, 3.0, 3.0, 0.5, 3.0]])
    sel, _ = oracle.select_topk(z, 2)
    assert list(sel[0]) == [1, 2]


def test_routing_weights_closed_form():
    """Pin: renormalised weights sum to 1, and p_S / sum p_S equals the
    closed form softmax over the selected logits only."""
    shape, x, w = tiny_inputs()
    r = oracle.route(x, w["router"], 2)
    assert np.max(np.abs(r["topk_w"].sum(1) - 1)) < 1e-12
    zs = np.take_along_axis(r["z"], r["topk_idx"].astype(np.int64), axis=1)
    closed = np.exp(zs - zs.max(1, keepdims=True))
    closed /= closed.sum(1, keepdims=True)
    assert np.max(np.abs(r["topk_w"] - closed)) < 1e-12
    # ascending id order inside each set, weights aligned with it
    assert np.all(np.diff(r["topk_idx"], axis=1) > 0)


def test_routing_k1_and_kE():
    """Pin: k=1 gives weight exactly 1; k=E gives the full softmax."""
    shape, x, w = tiny_inputs()
    r1 = oracle.route(x, w["router"], 1)
    assert np.all(r1["topk_w"] == 1.0)
    assert np.array_equal(r1["topk_idx"][:, 0], np.argmax(r1["z"].astype(np.float32), axis=1))
    rE = oracle.route(x, w["router"], shape.experts)
    assert np.array_equal(rE["topk_idx"], np.broadcast_to(np.arange(8), (shape.tokens, 8)))
    assert np.max(np.abs(rE["topk_w"] - oracle.softmax(rE["z"]))) < 1e-15


def test_router_logits_library_matmul():
    """Pin: the logits are torch's fp64 matmul of the widened bf16 tensors
    (the bf16 widening itself is torch's bfloat16 -> float64 cast)."""
    shape, x, w = tiny_inputs()
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    wt = torch.from_numpy(w["router"].view(np.int16)).view(torch.bfloat16).to(torch.float64)
    assert np.max(np.abs(oracle.router_logits(x, w["router"]) - (xt @ wt).numpy())) < 1e-12
    b = np.linspace(-1, 1, 8).astype(np.float32)
    assert np.max(np.abs(oracle.router_logits(x, w["router"], b) - (xt @ wt).numpy() - b)) < 1e-12


# ---------------------------------------------------------------------------
# align (permutation)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("T,E,k", [(32, 8, 2), (257, 16, 4), (64, 128, 8), (1, 8, 8), (5, 3, 1)])
def test_align_matches_stable_argsort(T, E, k):
    """Pin: the counting sort equals numpy's stable argsort of the expert id
    of each token-major slot; counts sum to T*k; offsets are the cumulative
    counts; pos inverts perm slot by slot."""
    g = np.random.default_rng([T, E, k])
    idx = np.sort(np.stack([g.choice(E, k, replace=False) for _ in range(T)]), axis=1)
    a = oracle.align(idx, E)
    slot_expert = idx.reshape(-1)
    order = np.argsort(slot_expert, kind="stable")
    assert np.array_equal(a["perm"], order // k)
    assert np.array_equal(a["counts"], np.bincount(slot_expert, minlength=E))
    assert a["offsets"][0] == 0 and a["offsets"][-1] == T * k
    assert np.array_equal(np.diff(a["offsets"]), a["counts"])
    inv = np.empty(T * k, dtype=np.int64)
    inv[order] = np.arange(T * k)
    assert np.array_equal(a["pos"].reshape(-1), inv)
    for t in range(T):
        for j in range(k):
            assert a["perm"][a["pos"][t, j]] == t


# ---------------------------------------------------------------------------
# the block
# ---------------------------------------------------------------------------


def test_routed_branch_equals_dense_mask_brute_force():
    """Pin: the grouped computation (align, per-expert GEMMs, gather-sum)
    equals running every expert on every token with a dense weight matrix
    that is zero outside the selected set — no grouping code shared."""
    shape, x, w = tiny_inputs()
    r = run(shape, x, w)
    routed = r["out"] - r["y_d"]
    bf = oracle.routed_mixture_dense_mask(x, w["router"], w["gate"], w["up"], w["down"],
                                          shape.top_k)
    assert rel_err(routed, bf) < 1e-12


def test_dense_branch_is_torch_geglu_mlp():
    """Pin: zero every routed down matrix and the block is one GeGLU MLP,
    checked against torch fp64 matmuls and torch's tanh GELU."""
    shape, x, w = tiny_inputs()
    w2 = dict(w)
    w2["down"] = np.zeros_like(w["down"])
    r = run(shape, x, w2)

    def t(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(torch.float64)

    X = t(x)
    g = torch.nn.functional.gelu(X @ t(w["dgate"]), approximate="tanh")
    ref = ((g * (X @ t(w["dup"]))) @ t(w["ddown"])).numpy()
    assert rel_err(r["out"], ref) < 1e-12


def test_single_expert_is_torch_geglu_mlp():
    """Pin: with k=1 and no dense branch, each output row is its expert's
    GeGLU MLP (torch fp64), weight 1."""
    shape, x, w = tiny_inputs()
    r = oracle.moe_ffn(x, w["router"], w["gate"], w["up"], w["down"], top_k=1)

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(torch.float64)

    X = t(x)
    for tok in range(shape.tokens):
        e = int(r["topk_idx"][tok, 0])
        h = torch.nn.functional.gelu(X[tok] @ t(w["gate"][e]), approximate="tanh") * (X[tok] @ t(w["up"][e]))
        assert rel_err(r["out"][tok], (h @ t(w["down"][e])).numpy()) < 1e-12


def test_token_permutation_invariance():
    """Pin: permuting the tokens permutes the outputs the same way."""
    shape, x, w = tiny_inputs()
    r = run(shape, x, w)
    p = np.random.default_rng(3).permutation(shape.tokens)
    rp = run(shape, x[p], w)
    assert rel_err(rp["out"], r["out"][p]) < 1e-12


def test_expert_relabelling_invariance():
    """Pin: permuting the router columns together with the expert weight
    stacks leaves the output unchanged (no exact ties in this input)."""
    shape, x, w = tiny_inputs()
    r = run(shape, x, w)
    p = np.random.default_rng(4).permutation(shape.experts)
    w2 = dict(w)
    w2["router"] = w["router"][:, p]
    w2["gate"], w2["up"], w2["down"] = w["gate"][p], w["up"][p], w["down"][p]
    r2 = run(shape, x, w2)
    assert rel_err(r2["out"], r["out"]) < 1e-12


def test_identical_experts_give_one_expert():
    """Pin: with all experts identical, the routed output is that expert's
    output because the renormalised weights sum to 1."""
    shape, x, w = tiny_inputs()
    w2 = dict(w)
    for n in ("gate", "up", "down"):
        w2[n] = np.broadcast_to(w[n][3], w[n].shape).copy()
    r = oracle.moe_ffn(x, w2["router"], w2["gate"], w2["up"], w2["down"], top_k=2)
    _, ref = oracle.geglu(oracle.widen_bf16(x), oracle.widen_bf16(w["gate"][3]),
                          oracle.widen_bf16(w["up"][3]), oracle.widen_bf16(w["down"][3]))
    assert rel_err(r["out"], ref) < 1e-12


def test_k_equals_E_is_full_softmax_mixture():
    """Pin: with k = E the routed branch is the softmax-weighted sum of all
    experts (dense-mask brute force with the full softmax)."""
    shape, x, w = tiny_inputs()
    r = oracle.moe_ffn(x, w["router"], w["gate"], w["up"], w["down"], top_k=shape.experts)
    p = oracle.softmax(oracle.router_logits(x, w["router"]))
    X = oracle.widen_bf16(x)
    acc = 0
    for e in range(shape.experts):
        _, ye = oracle.geglu(X, oracle.widen_bf16(w["gate"][e]), oracle.widen_bf16(w["up"][e]),
                             oracle.widen_bf16(w["down"][e]))
        acc = acc + p[:, e:e + 1] * ye
    assert rel_err(r["out"], acc) < 1e-12


def test_zero_input_gives_zero_output():
    """Pin: x = 0 -> all logits 0 -> set {0..k-1}, w = 1/k, GELU(0)*0 = 0,
    output exactly 0."""
    shape, x, w = tiny_inputs()
    r = run(shape, np.zeros_like(x), w)
    assert np.all(r["out"] == 0.0)
    assert np.all(r["topk_idx"] == np.arange(shape.top_k))


def test_token_subset_mode_matches_full():
    """The sampled-token mode (used at full sizes) agrees with the full path."""
    shape, x, w = tiny_inputs()
    r = run(shape, x, w)
    toks = [0, 5, 31]
    rs = run(shape, x, w, tokens=toks)
    assert rel_err(rs["out"], r["out"][toks]) < 1e-12


def test_residual_layer_with_zero_down_is_identity():
    """Pin of the stack step x + FFN(x): with every down projection zero the
    block contributes exactly 0 (both branches end in a down matmul), so the
    layer returns its input; with the dense branch alone left on, the layer
    adds exactly the torch GeGLU MLP of x."""
    shape, x, w = tiny_inputs()
    wz = dict(w)
    wz["down"] = np.zeros_like(w["down"])
    wz["ddown"] = np.zeros_like(w["ddown"])
    y, _ = oracle.moe_ffn_layer_residual(x, wz, shape.top_k)
    assert np.array_equal(y, oracle.widen_bf16(x))
    wd = dict(w)
    wd["down"] = np.zeros_like(w["down"])
    y, _ = oracle.moe_ffn_layer_residual(x, wd, shape.top_k)
    X = torch.from_numpy(oracle.widen_bf16(x))
    g = X @ torch.from_numpy(oracle.widen_bf16(w["dgate"]))
    u = X @ torch.from_numpy(oracle.widen_bf16(w["dup"]))
    ref = X + (torch.nn.functional.gelu(g, approximate="tanh") * u) @ torch.from_numpy(
        oracle.widen_bf16(w["ddown"]))
    assert rel_err(y, ref.numpy()) < 1e-12


# ---------------------------------------------------------------------------
# sandwich norms and the residual (the block with its RMSNorms)
# ---------------------------------------------------------------------------


def test_rms_norm_matches_torch_rms_norm():
    """Pin: oracle.rms_norm against torch.nn.functional.rms_norm (a library
    routine) on random rows, random gains, two epsilons."""
    rng = np.random.default_rng(7)
    X = rng.standard_normal((9, 64)) * 3.0
    g = rng.standard_normal(64)
    for eps in (1e-6, 0.5):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(X), (64,), weight=torch.from_numpy(g), eps=eps)
        assert rel_err(oracle.rms_norm(X, g, eps), ref.numpy()) < 1e-12


def test_rms_norm_unit_rms_and_constant_rows():
    """Pins: with eps = 0 and unit gain every row has mean square exactly 1
    (up to rounding); a constant row c maps to c / sqrt(c^2 + eps) * g."""
    rng = np.random.default_rng(8)
    X = rng.standard_normal((5, 96)) * rng.uniform(0.01, 100.0, (5, 1))
    y = oracle.rms_norm(X, np.ones(96), 0.0)
    assert np.max(np.abs(np.mean(y * y, axis=1) - 1.0)) < 1e-12
    c, eps, g = -0.75, 1e-6, rng.standard_normal(96)
    y = oracle.rms_norm(np.full((1, 96), c), g, eps)
    assert rel_err(y[0], c / np.sqrt(c * c + eps) * g) < 1e-14


def test_round_bf16_matches_torch_cast():
    """Pin: oracle.round_bf16 against torch's float32 -> bfloat16 cast (round
    to nearest even), on random values and on exact halfway cases."""
    rng = np.random.default_rng(9)
    v = (rng.standard_normal(4096) * np.exp(rng.uniform(-20, 20, 4096))).astype(np.float32)
    half = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(2.0 + 2.0 ** -7), 3.0 + 2.0 ** -7],
                    dtype=np.float32)  # exactly between two bf16 values
    for a in (v, half):
        ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(oracle.round_bf16(a), ref)
    assert list(oracle.round_bf16(half)) == [1.0, 1.015625, -2.0, 3.0]


def block(shape, x, w, pre, post, eps, **kw):
    return oracle.moe_block(x, pre, post, eps, w["router"], w["gate"], w["up"], w["down"], w["dgate"],
                            w["dup"], w["ddown"], top_k=shape.top_k, **kw)


def test_block_with_zero_post_gain_is_identity():
    """Pin of the residual: with a zero post-norm gain the sub-block adds
    exactly 0, so it returns its input."""
    shape, x, w = tiny_inputs()
    g = np.random.default_rng(1).standard_normal(shape.hidden)
    r = block(shape, x, w, g, np.zeros(shape.hidden), 1e-6)
    assert np.array_equal(r["out"], oracle.widen_bf16(x))


def test_block_prenorm_removes_input_scale():
    """Pin: with eps = 0 the pre-norm makes the FFN blind to a power-of-two
    scale of x (doubling is exact in binary floating point, so xn and the FFN
    output are bit-identical); the block output then differs from the
    unscaled one only by the change of the residual."""
    shape, x, w = tiny_inputs()
    rng = np.random.default_rng(2)
    pre, post = rng.standard_normal(shape.hidden), rng.standard_normal(shape.hidden)
    X = oracle.widen_bf16(x)
    r1 = block(shape, X, w, pre, post, 0.0)
    r2 = block(shape, 4.0 * X, w, pre, post, 0.0)
    assert np.array_equal(r1["xn"], r2["xn"])
    assert np.array_equal(r1["ffn"], r2["ffn"])
    assert rel_err(r2["out"] - 4.0 * X, r1["out"] - X) < 1e-12


def test_block_is_norm_ffn_norm_residual_with_torch_norms():
    """Pin of the composition: pre-norm and post-norm taken from
    torch.nn.functional.rms_norm, the bf16 store from torch's cast, the FFN
    from oracle.moe_ffn (pinned above); sampled-token mode agrees too."""
    shape, x, w = tiny_inputs()
    rng = np.random.default_rng(3)
    pre, post, eps = rng.standard_normal(shape.hidden), rng.standard_normal(shape.hidden), 1e-6
    X = torch.from_numpy(oracle.widen_bf16(x))
    xn = torch.nn.functional.rms_norm(X, (shape.hidden,), weight=torch.from_numpy(pre), eps=eps)
    xn = xn.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    f = run(shape, xn.numpy(), w)["out"]
    ref = X + torch.nn.functional.rms_norm(torch.from_numpy(f), (shape.hidden,), weight=torch.from_numpy(post),
                                           eps=eps)
    r = block(shape, x, w, pre, post, eps)
    assert rel_err(r["out"], ref.numpy()) < 1e-12
    toks = [2, 17, 30]
    rs = block(shape, x, w, pre, post, eps, tokens=toks)
    assert rel_err(rs["out"], r["out"][toks]) < 1e-12


def test_force_routing_reproduces_own_routing():
    shape, x, w = tiny_inputs()
    r = run(shape, x, w)
    rf = run(shape, x, w, force_routing=r["topk_idx"])
    assert np.array_equal(rf["out"], r["out"])


# ---------------------------------------------------------------------------
# shapes: parameter counts printed on the pages
# ---------------------------------------------------------------------------


def test_parameter_counts_reproduce_printed_values():
    """Pin: with each expert = 3 bias-free [H, I] / [I, H] matrices, the
    router = one [H, E] matrix and the dense branch = 3 [H, D] / [D, H]
    matrices — the shapes the oracle consumes — the counts printed on the
    archdb page (total, embedding, backbone, largest layer group, active)
    are reproduced within their printed rounding.  Also the per-layer
    routed-expert count 128*3*2816*704 = 761,266,176."""
    with open(os.path.join(GOLDEN, "param_counts.json")) as f:
        g = json.load(f)
    c = g["config"]
    s = synth.DECODE
    H, E, I, D = s.hidden, s.experts, s.expert_dim, s.dense_dim
    assert (H, E, s.top_k, I, D) == (c["embed_dim"], c["num_experts"], c["top_k_experts"],
                                     c["expert_dim"], c["moe_dense_hidden_dim"])
    # shapes the oracle consumes (router [H,E]; gate/up [E,H,I]; down [E,I,H]; dense [H,D],[D,H])
    experts = E * (H * I + H * I + I * H)
    dense = H * D + H * D + D * H
    router = H * E
    assert experts == 761_266_176
    local_attn = H * c["num_heads"] * c["head_dim"] * 2 + H * c["num_kv_heads"] * c["head_dim"] * 2
    kv = 1 if c["k_eq_v_global"] else 2
    global_attn = (H * c["num_heads"] * c["global_key_size"] * 2
                   + H * c["num_global_kv_heads"] * c["global_key_size"] * kv)
    L, Lg = c["num_layers"], c["global_layers"]
    backbone = L * (experts + dense + router) + (L - Lg) * local_attn + Lg * global_attn
    embedding = c["num_embed"] * H
    largest = experts + dense + router + global_attn
    active = backbone - L * experts + L * experts * s.top_k // E
    got = {"counted_total": backbone + embedding, "counted_embedding": embedding,
           "counted_backbone": backbone, "largest_layer_group": largest,
           "counted_active": active}
    for key, val in got.items():
        p = g["printed"][key]
        assert abs(val - p["value"]) <= p["round_to"] / 2, (key, val, p)


# ---------------------------------------------------------------------------
# NVFP4 decoding
# ---------------------------------------------------------------------------


def test_e4m3_decoder_matches_torch_all_codes():
    """Pin: all 256 float8_e4m3fn bytes decode as torch.float8_e4m3fn does
    (NaN for S.1111.111)."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = oracle.E4M3_TABLE
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.all(both_nan | (ref == mine))
    assert np.sum(np.isnan(mine)) == 2
    assert np.nanmax(mine) == 448.0


def test_e2m1_decoder_matches_ocp_table():
    """Pin: the 16 e2m1 codes decode to the OCP MX FP4 table."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_values.txt"))
            if l.strip() and not l.startswith("#")]
    for code, val in rows:
        v = oracle.e2m1_value(int(code))
        assert v == float(val) and np.signbit(v) == np.signbit(float(val)) or (v == 0 and float(val) == 0)


def test_e2m1_times_e4m3_products_exact_in_bf16():
    """Every e2m1 x e4m3 product (finite) is exactly representable in bf16
    (8 significant bits), so a dequantised bf16 tile carries no rounding."""
    prods = np.outer(oracle.E2M1_TABLE, oracle.E4M3_TABLE[np.isfinite(oracle.E4M3_TABLE)]).ravel()
    t = torch.from_numpy(prods).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(t, prods)


def test_nvfp4_dequant_layout_and_roundtrip():
    """Pin: dequantise(pack(W)) is within the NVFP4 grid error of W, the
    layout puts value (n, k) in q[n, k//2] (low nibble = even k), and packing
    the dequantised matrix again reproduces the same bytes."""
    g = np.random.default_rng(7)
    K, N = 64, 48
    wv = g.standard_normal((K, N)).astype(np.float32) * 0.05
    q, s, st = synth.nvfp4_pack(wv)
    assert q.shape == (N, K // 2) and s.shape == (N, K // 16)
    deq = oracle.dequant_matrix(q, s, st)
    assert deq.shape == (K, N)
    # hand-decode one element from the bytes
    n, k = 7, 33
    code = (q[n, k // 2] >> 4) & 0xF
    val = oracle.e2m1_value(code) * oracle.e4m3fn_value(s[n, k // 16]) * float(np.float32(st))
    assert deq[k, n] == val
    # error bound: the largest e2m1 grid step is 2 (between 4 and 6), so a
    # code is off by at most 1 unit of s_g * s_t = gmax / 6 * (1 + d), where
    # |d| <= 1/16 is the e4m3 rounding of the group scale (3 mantissa bits)
    err = np.abs(deq - wv)
    gmax = np.repeat(np.abs(wv).reshape(K // 16, 16, N).max(1), 16, axis=0)
    assert np.all(err <= gmax / 6 * (1 + 1 / 16) + 1e-12)
    q2, s2, st2 = synth.nvfp4_pack(deq.astype(np.float32))
    assert np.array_equal(q2, q) and np.array_equal(s2, s) and st2 == st


def test_nvfp4_block_uses_dequantised_weights():
    """The NVFP4 block equals the bf16-weight path applied to the decoded
    matrices (only the weight format changes)."""
    shape, x, w = tiny_inputs()
    pk = {n: synth.nvfp4_pack_stack(w[n]) for n in ("gate", "up", "down")}
    pk.update({n: synth.nvfp4_pack_stack(w[n][None]) for n in ("dgate", "dup", "ddown")})
    r = oracle.moe_ffn(x, w["router"], pk["gate"], pk["up"], pk["down"], pk["dgate"],
                       pk["dup"], pk["ddown"], top_k=2)
    deq = {n: np.stack([oracle.dequant_matrix(pk[n]["q"][g], pk[n]["scale"][g],
                                              pk[n]["tensor_scale"][g])
                        for g in range(pk[n]["q"].shape[0])]) for n in pk}
    r2 = oracle.moe_ffn(x, w["router"], deq["gate"], deq["up"], deq["down"], deq["dgate"][0],
                        deq["dup"][0], deq["ddown"][0], top_k=2)
    assert np.array_equal(r["out"], r2["out"])


def test_fp8_dequant_matches_torch_and_layout():
    """Pin: the FP8 decode equals torch's float8_e4m3fn -> float64 cast times
    the fp32 scale (a library routine), value (k, n) sits at q[k, n]; the
    packing error is at most half an e4m3 step (3 mantissa bits, relative
    2^-4) of the scaled value, or half the subnormal step 2^-9 * scale; and
    packing the decoded matrix again reproduces the bytes."""
    g = np.random.default_rng(8)
    K, N = 64, 48
    wv = g.standard_normal((K, N)).astype(np.float32) * 0.05
    q, st = synth.fp8_pack(wv)
    assert q.shape == (K, N) and q.dtype == np.uint8
    deq = oracle.dequant_matrix_fp8(q, st)
    ref = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy() * float(np.float32(st))
    assert np.array_equal(deq, ref)
    k, n = 33, 7
    assert deq[k, n] == oracle.e4m3fn_value(q[k, n]) * float(np.float32(st))
    err = np.abs(deq - wv)
    bound = np.maximum(np.abs(wv) * 2.0 ** -4, 2.0 ** -10 * float(st)) + 1e-12
    assert np.all(err <= bound)
    assert np.max(np.abs(deq)) == 448.0 * float(np.float32(st))  # amax maps to the top code
    q2, st2 = synth.fp8_pack(deq.astype(np.float32))
    assert np.array_equal(q2, q) and st2 == st


def test_fp8_block_uses_dequantised_weights():
    """The FP8 block equals the bf16-weight path applied to the decoded
    matrices (only the weight format changes), dense-only config included."""
    shape, x, w = tiny_inputs()
    pk = {n: synth.fp8_pack_stack(w[n]) for n in ("gate", "up", "down")}
    pk.update({n: synth.fp8_pack_stack(w[n][None]) for n in ("dgate", "dup", "ddown")})
    r = oracle.moe_ffn(x, w["router"], pk["gate"], pk["up"], pk["down"], pk["dgate"],
                       pk["dup"], pk["ddown"], top_k=2)
    deq = {n: np.stack([oracle.dequant_matrix_fp8(pk[n]["q8"][g], pk[n]["tensor_scale"][g])
                        for g in range(pk[n]["q8"].shape[0])]) for n in pk}
    r2 = oracle.moe_ffn(x, w["router"], deq["gate"], deq["up"], deq["down"], deq["dgate"][0],
                        deq["dup"][0], deq["ddown"][0], top_k=2)
    assert np.array_equal(r["out"], r2["out"])
    d = oracle.dense_ffn(x, pk["dgate"], pk["dup"], pk["ddown"])
    assert np.array_equal(d["out"], r2["y_d"])


# ---------------------------------------------------------------------------
# the skewed-load workload's calibration
# ---------------------------------------------------------------------------


@pytest.mark.slow
def test_skew_lambda_gives_zipf_slope():
    """The stored logit-bias scale gives a realised sorted-load log-log slope
    of -1.2 over ranks 9..128 at T=16384 (seed 0), as the workload asks."""
    from tests.golden.calibrate_skew import load_slope
    slope, loads = load_slope(synth.SKEW_LAMBDA)
    assert abs(slope + synth.ZIPF_S) < 0.02, slope
    assert loads.sum() == synth.SKEW.tokens * synth.SKEW.top_k


# ---------------------------------------------------------------------------
# the dense FFN of the E4B sibling (no router, no experts)
# ---------------------------------------------------------------------------


def _torch_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(torch.float64)


def test_dense_ffn_is_torch_geglu_mlp():
    """Pin: the dense FFN is one GeGLU MLP, checked against torch fp64
    matmuls and torch's tanh GELU (a library routine) on the tiny E4B-like
    shape; the hidden rows h_d are the GELU(gate) * up product."""
    shape = synth.E4B_TINY
    x, w = synth.make_x(shape), synth.make_weights(shape)
    assert w["router"] is None and w["gate"] is None
    r = oracle.dense_ffn(x, w["dgate"], w["dup"], w["ddown"])
    X = _torch_bf16(x)
    h = torch.nn.functional.gelu(X @ _torch_bf16(w["dgate"]), approximate="tanh") * (X @ _torch_bf16(w["dup"]))
    assert rel_err(r["h_d"], h.numpy()) < 1e-12
    assert rel_err(r["out"], (h @ _torch_bf16(w["ddown"])).numpy()) < 1e-12


def test_dense_ffn_shape_of_e4b_page():
    """Pin of the shape: the E4B page gives embed_dim 2560 and hidden_dim
    10240 with no experts, i.e. 3 * 2560 * 10240 = 78,643,200 FFN weights per
    layer; the generated matrices have exactly those shapes."""
    s = synth.E4B_DECODE
    assert (s.hidden, s.dense_dim, s.experts, s.expert_dim) == (2560, 10240, 0, 0)
    shapes = {"dgate": (2560, 10240), "dup": (2560, 10240), "ddown": (10240, 2560)}
    assert sum(a * b for a, b in shapes.values()) == 78_643_200


def test_dense_ffn_token_rows_and_independence():
    """Pin: each output row depends on its own input row only (sampled-row
    mode and a token permutation agree with the full call), and x = 0 gives 0
    (GELU(0) = 0, no biases)."""
    shape = synth.E4B_TINY
    x, w = synth.make_x(shape), synth.make_weights(shape)
    full = oracle.dense_ffn(x, w["dgate"], w["dup"], w["ddown"])["out"]
    toks = [0, 5, 31]
    assert rel_err(oracle.dense_ffn(x, w["dgate"], w["dup"], w["ddown"], tokens=toks)["out"], full[toks]) < 1e-12
    p = np.random.default_rng(4).permutation(shape.tokens)
    assert rel_err(oracle.dense_ffn(x[p], w["dgate"], w["dup"], w["ddown"])["out"], full[p]) < 1e-12
    z = oracle.dense_ffn(np.zeros_like(x), w["dgate"], w["dup"], w["ddown"])["out"]
    assert np.array_equal(z, np.zeros_like(z))


def test_dense_ffn_is_moe_block_dense_branch():
    """Pin: the dense FFN equals the dense branch y_d of the MoE block (itself
    pinned against torch above) on the same input and dense matrices."""
    shape, x, w = tiny_inputs()
    r = run(shape, x, w)
    d = oracle.dense_ffn(x, w["dgate"], w["dup"], w["ddown"])
    assert np.array_equal(d["out"], r["y_d"])


def test_dense_block_torch_norms_and_zero_post_gain():
    """Pin of the sandwich around the dense FFN: pre- and post-norm from
    torch.nn.functional.rms_norm and the bf16 store from torch's cast; a zero
    post gain returns the input exactly."""
    shape = synth.E4B_TINY
    x, w = synth.make_x(shape), synth.make_weights(shape)
    rng = np.random.default_rng(5)
    pre, post, eps = rng.standard_normal(shape.hidden), rng.standard_normal(shape.hidden), 1e-6
    X = torch.from_numpy(oracle.widen_bf16(x))
    xn = torch.nn.functional.rms_norm(X, (shape.hidden,), weight=torch.from_numpy(pre), eps=eps)
    xn = xn.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    h = torch.nn.functional.gelu(xn @ _torch_bf16(w["dgate"]), approximate="tanh") * (xn @ _torch_bf16(w["dup"]))
    f = h @ _torch_bf16(w["ddown"])
    ref = X + torch.nn.functional.rms_norm(f, (shape.hidden,), weight=torch.from_numpy(post), eps=eps)
    r = oracle.dense_block(x, pre, post, eps, w["dgate"], w["dup"], w["ddown"])
    assert rel_err(r["out"], ref.numpy()) < 1e-12
    rs = oracle.dense_block(x, pre, post, eps, w["dgate"], w["dup"], w["ddown"], tokens=[3, 9])
    assert rel_err(rs["out"], r["out"][[3, 9]]) < 1e-12
    z = oracle.dense_block(x, pre, np.zeros(shape.hidden), eps, w["dgate"], w["dup"], w["ddown"])
    assert np.array_equal(z["out"], oracle.widen_bf16(x))


# ---------------------------------------------------------------------------
# W4A4: the NVFP4 activation quantiser
# ---------------------------------------------------------------------------


def test_e4m3_rounding_matches_torch_cast():
    """Pin: round_e4m3_sat equals torch's float8_e4m3fn cast (round to nearest
    even) on fp32 values in [0, 448], including every midpoint between
    neighbouring e4m3 values; above 448 it saturates."""
    vals = oracle.E4M3_TABLE[:127]                               # non-negative finite values
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(11)
    rand = np.concatenate([rng.uniform(0, 448, 4000), 2.0 ** rng.uniform(-12, 8.8, 4000)])
    x = np.concatenate([vals, mids, rand]).astype(np.float32)
    x = x[x <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_e4m3_sat(x), ref)
    assert np.all(oracle.round_e4m3_sat(np.float32([448.5, 470.0, 1e6])) == 448.0)


def test_e2m1_rounding_is_nearest_with_even_ties():
    """Pin: round_e2m1_sat is the nearest e2m1 value by brute force over the
    8 magnitudes, a tie going to the even mantissa (codes 0, 2, 4, 6), and
    values beyond 6 saturate."""
    mags = oracle.E2M1_TABLE[:8]
    rng = np.random.default_rng(12)
    r = np.concatenate([rng.uniform(-8, 8, 5000), (mags[:-1] + mags[1:]) / 2, -(mags[:-1] + mags[1:]) / 2, mags])
    got = oracle.round_e2m1_sat(r)
    for v, g in zip(r, got):
        d = np.abs(np.abs(v) - mags)
        best = np.flatnonzero(d == d.min())
        code = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
        assert g == np.sign(v) * mags[code] and np.signbit(g) == np.signbit(v), (v, g)
    assert np.signbit(oracle.round_e2m1_sat(np.array([-0.0, -0.2]))).all()


def test_activation_quantiser_worked_group():
    """Pin on a hand-worked group: with s_in = fp32(1/6), 6 * s_in rounds to
    exactly 1 in fp32, the group amax 6 gives s_g = 6, s_g * s_in rounds to 1,
    so each value is just rounded on the e2m1 grid (ties to the even
    mantissa) and the dequantised value is that times s_g = 6."""
    s_in = float(np.float32(1.0 / 6.0))
    v = np.array([0, 0.25, 0.3, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6, -1, -2.9, 4.4, 0.5, 1.5, 3.0])
    e2m1 = np.array([0, 0, 0.5, 1, 1, 2, 2, 4, 4, 6, -1, -3, 4, 0.5, 1.5, 3.0])
    assert np.array_equal(oracle.quant_act_nvfp4(v[None], s_in)[0], e2m1 * 6.0)


def test_activation_quantiser_properties():
    """Pins: groups are independent (permuting whole groups permutes the
    output), an all-zero group gives zeros, every output is an e2m1 x e4m3
    product and so exact in bf16, and |q * s_in - v| is at most one e2m1 half
    step at the top of the grid, s_g * s_in, per group."""
    rng = np.random.default_rng(13)
    v = oracle.round_bf16(rng.standard_normal((6, 64)) * np.array([1e-3, 0.1, 1, 10])[:, None].repeat(16, 1).T.reshape(-1)[None])
    v[2, 16:32] = 0.0
    s_in = float(np.float32(np.max(np.abs(v)) / (6 * 448)))
    q = oracle.quant_act_nvfp4(v, s_in)
    assert np.all(q[2, 16:32] == 0)
    assert np.array_equal(oracle.round_bf16(q), q)
    perm = np.array([2, 0, 3, 1])
    vp = v.reshape(6, 4, 16)[:, perm].reshape(6, 64)
    assert np.array_equal(oracle.quant_act_nvfp4(vp, s_in), q.reshape(6, 4, 16)[:, perm].reshape(6, 64))
    g = v.reshape(6, 4, 16)
    amax = np.abs(g).max(-1)
    sg = oracle.round_e4m3_sat(np.float32(amax / np.float32(6 * np.float32(s_in))))
    err = np.abs(q * s_in - v).reshape(6, 4, 16).max(-1)
    assert np.all(err <= sg * s_in * (1 + 1e-6) + 1e-30)


def test_w4a4_block_composition_with_torch():
    """Pin of the W4A4 block: routing of the unquantised x; each expert and
    the dense branch as torch fp64 matmuls and torch's tanh GELU on the
    quantised activations (quantiser pinned above), the hidden rows rounded
    to bf16 by torch's cast before their quantisation; sampled-token mode
    agrees."""
    shape, x, w = tiny_inputs()
    pk = {n: synth.nvfp4_pack_stack(w[n]) for n in ("gate", "up", "down")}
    pk.update({n: synth.nvfp4_pack_stack(w[n][None]) for n in ("dgate", "dup", "ddown")})
    s = (0.003, 0.002, 0.001)
    r = oracle.moe_ffn_w4a4(x, w["router"], pk["gate"], pk["up"], pk["down"], pk["dgate"], pk["dup"],
                            pk["ddown"], s, top_k=2)
    rt = oracle.route(x, w["router"], 2)
    assert np.array_equal(r["topk_idx"], rt["topk_idx"])

    def deq(n, g):
        return torch.from_numpy(oracle.dequant_matrix(pk[n]["q"][g], pk[n]["scale"][g], pk[n]["tensor_scale"][g]))

    def q(a, sc):
        sc = float(np.float32(sc))
        return torch.from_numpy(oracle.quant_act_nvfp4(a.numpy(), sc) * sc)

    def bf(t):
        return t.to(torch.float32).to(torch.bfloat16).to(torch.float64)

    X = q(torch.from_numpy(oracle.widen_bf16(x)), s[0])
    ref = np.zeros((shape.tokens, shape.hidden))
    for t in range(shape.tokens):
        for j in range(2):
            e = int(rt["topk_idx"][t, j])
            h = bf(torch.nn.functional.gelu(X[t:t + 1] @ deq("gate", e), approximate="tanh") * (X[t:t + 1] @ deq("up", e)))
            ref[t] += rt["topk_w"][t, j] * (q(h, s[1]) @ deq("down", e))[0].numpy()
    hd = bf(torch.nn.functional.gelu(X @ deq("dgate", 0), approximate="tanh") * (X @ deq("dup", 0)))
    ref += (q(hd, s[2]) @ deq("ddown", 0)).numpy()
    assert rel_err(r["out"], ref) < 1e-12
    rs = oracle.moe_ffn_w4a4(x, w["router"], pk["gate"], pk["up"], pk["down"], pk["dgate"], pk["dup"],
                             pk["ddown"], s, top_k=2, tokens=[1, 7, 30])
    assert rel_err(rs["out"], r["out"][[1, 7, 30]]) < 1e-12
