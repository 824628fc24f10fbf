"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Rules (bf16 block output): routing sets bit-exact on every token whose
k-th/(k+1)-th logit gap exceeds 1e-3 (near-ties are counted and compared
against the oracle re-run with the GPU's sets); counts, offsets, perm and pos
bit-exact against the oracle's grouping of the GPU's routing; outputs within
2e-2 * (|oracle| + rms(oracle)) element by element.  Every workload, the
full-size ones included, compares every routing/grouping entry, every output
element and every element of the intermediates h, y, h_d and y_d.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

STREAM = 1
MFMA = 2
AUTO = 0


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available()
    return _t


def ffn_for(shape, variant=AUTO, max_tokens=None, accumulate=False):
    from sparse_moe_transformer_amd import MoeFFN
    return MoeFFN.for_shape(shape, max_tokens=max_tokens or max(shape.tokens, 1), variant=variant,
                            accumulate=accumulate)


def run_gpu(torch, shape, x, w, bias, variant, nvfp4=False, ffn=None):
    T = x.shape[0]
    ffn = ffn or ffn_for(shape, variant, max_tokens=T)
    xd = G.up_bf16(x)
    bd = G.up(bias) if bias is not None else None
    out = torch.empty_like(xd)
    if nvfp4:
        ffn.forward_nvfp4(xd, G.up_nvfp4_weights(w), out, bd)
    else:
        ffn.forward(xd, G.up_weights(w), out, bd)
    torch.cuda.synchronize()
    r = {k: G.to_np(v) for k, v in ffn.routing(T).items()}
    inter = ffn.intermediates(T)
    torch.cuda.synchronize()
    return G.to_f64(out), r, inter, ffn


def full_check(shape, x, w, bias, out, r, inter=None, nvfp4_w=None, k=None):
    """Routing, grouping, every output element and (given) every element of
    the intermediates against the oracle.  The oracle runs once, on the GPU's
    sets: they equal its own on every token that is not a near-tie (checked
    first), and on near-ties both sets are correct."""
    k = k or shape.top_k
    wts = nvfp4_w or w
    rt = oracle.route(x, w["router"], k, bias)
    near = G.check_routing(r["topk_idx"], r["topk_w"], rt)
    G.check_align(r, r["topk_idx"], shape.experts)
    ref = oracle.moe_ffn(x, w["router"], wts["gate"], wts["up"], wts["down"], wts.get("dgate"),
                         wts.get("dup"), wts.get("ddown"), top_k=k, bias=bias,
                         force_routing=r["topk_idx"], intermediates=inter is not None)
    G.assert_block_close(out, ref["out"])
    if inter is not None:
        G.assert_block_close(G.to_f64(inter["h"]), ref["h"], what="h")
        G.assert_block_close(G.to_f64(inter["y"]), ref["y"], what="y")
        if shape.dense_dim:
            G.assert_block_close(G.to_f64(inter["h_d"]), ref["h_d"], what="h_d")
            G.assert_block_close(G.to_f64(inter["y_d"]), ref["y_d"], what="y_d")
    return ref, int(near.sum())


# ---------------------------------------------------------------------------
# tiny workload and ragged shapes
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("variant", [AUTO, MFMA, STREAM])
def test_tiny_block(torch, variant):
    s = synth.TINY
    x, w, bias = G.make_inputs(s)
    out, r, inter, _ = run_gpu(torch, s, x, w, bias, variant)
    ref, near = full_check(s, x, w, bias, out, r, inter)
    assert near == 0
    # with no near-ties the grouping equals the oracle's grouping of its own sets
    own = oracle.route(x, w["router"], s.top_k, bias)["topk_idx"]
    assert np.array_equal(r["perm"], oracle.align(own, s.experts)["perm"])


MID = synth.FFNShape("mid", 0, 512, 32, 4, 128, 192)
MID128 = synth.FFNShape("mid128", 0, 512, 128, 8, 128, 128)


@pytest.mark.parametrize("T", [1, 3, 8, 63, 64, 65, 200, 333])
@pytest.mark.parametrize("variant", [STREAM, MFMA])
def test_ragged_tokens(torch, T, variant):
    s = MID.with_tokens(T)
    x, w, bias = G.make_inputs(s, seed=T)
    out, r, inter, _ = run_gpu(torch, s, x, w, bias, variant)
    full_check(s, x, w, bias, out, r, inter)


def test_streaming_every_token_count(torch):
    """Every T the streaming path takes (1..64) on one handle, each checked in
    full: the down units' GeGLU staging sees every row-chunk remainder, and
    the router's token groups every ragged tail."""
    ffn = ffn_for(MID, STREAM, max_tokens=64)
    for T in range(1, 65):
        s = MID.with_tokens(T)
        x, w, bias = G.make_inputs(s, seed=100 + T)
        out, r, inter, _ = run_gpu(torch, s, x, w, bias, STREAM, ffn=ffn)
        full_check(s, x, w, bias, out, r, inter)


# the 26B router shape (two tokens per router group at H = 2816, E = 128)
# with narrow experts, so the oracle stays cheap
ROUTE_WIDE = synth.FFNShape("routewide", 0, 2816, 128, 8, 64, 64)


def test_alternating_token_counts_one_handle(torch):
    """Forwards of different T on one handle, each checked in full.  The
    router's arrival counters (one per group of two tokens here) must be
    back at zero after every forward whatever the group count, and the
    streaming (T <= 32) and MFMA variants share the workspace."""
    ffn = ffn_for(ROUTE_WIDE.with_tokens(64), AUTO, max_tokens=64)
    for i, T in enumerate([8, 64, 1, 33, 8, 17, 64, 3]):
        st = ROUTE_WIDE.with_tokens(T)
        x, w, bias = G.make_inputs(st, seed=100 + i)
        out, r, inter, _ = run_gpu(torch, st, x, w, bias, AUTO, ffn=ffn)
        full_check(st, x, w, bias, out, r, inter)


@pytest.mark.parametrize("T", [40, 300])
def test_mfma_router_and_bias(torch, T):
    """E = 128 takes the MFMA router tiles at T > 64; a logit bias shifts loads."""
    s = MID128.with_tokens(T)
    x, w, _ = G.make_inputs(s, seed=11)
    bias = synth.zipf_bias(s.experts, lam=0.5)
    for variant in (AUTO, MFMA):
        out, r, inter, _ = run_gpu(torch, s, x, w, bias, variant)
        full_check(s, x, w, bias, out, r, inter)


@pytest.mark.parametrize("H,E,k,T", [(512, 4, 2, 5), (2816, 256, 8, 8), (2816, 132, 8, 8), (512, 24, 3, 7), (512, 16, 4, 8),
                                     (256, 8, 8, 8), (2816, 172, 8, 8), (2304, 212, 8, 5), (512, 256, 8, 200),
                                     (512, 128, 8, 97), (512, 256, 8, 8200), (256, 128, 4, 8195),
                                     (512, 256, 8, 4099), (256, 128, 4, 4100)])
def test_router_shapes(torch, H, E, k, T):
    """Small-T router variants: 8-expert chunks (E/8 a power of two, several
    row batches at E = 256), and the per-expert path for other E.  Two
    shapes (wide H, E not a multiple of 8) do not fit the small-T router's
    launch shape: they route with the large-T kernels.  T >= 4096 with
    E = 128 or 256 takes the one-launch MFMA router (16 tokens per block
    below T = 8192, 32 from there; ragged last blocks).  E = 256 and E = 132
    (4-expert chunks) at H = 2816 do not fit the router's 16 K-slices and
    take 32."""
    s = synth.FFNShape("rt", T, H, E, k, 64, 64)
    x, w, _ = G.make_inputs(s, seed=E)
    out, r, inter, _ = run_gpu(torch, s, x, w, None, AUTO)
    full_check(s, x, w, None, out, r, inter)


def test_no_dense_branch(torch):
    s = synth.FFNShape("nodense", 70, 256, 8, 2, 64, 0)
    x, w, _ = G.make_inputs(s)
    for variant in (STREAM, MFMA):
        out, r, inter, _ = run_gpu(torch, s, x, w, None, variant)
        full_check(s, x, w, None, out, r, inter)


@pytest.mark.parametrize("shape", [MID.with_tokens(100), MID.with_tokens(8),
                                   synth.FFNShape("rt256", 3, 512, 256, 16, 64, 64)])
def test_zero_input(torch, shape):
    """x = 0: every logit is 0, the set is {0..k-1} with weights 1/k, out = 0
    (all experts tie: the small-T router's ranks and the large-T arg-max
    must both fall back to the lowest ids)."""
    s = shape
    _, w, _ = G.make_inputs(s)
    x = np.zeros((s.tokens, s.hidden), dtype=np.uint16)
    for variant in (STREAM, MFMA):
        out, r, _, _ = run_gpu(torch, s, x, w, None, variant)
        assert np.all(out == 0.0)
        assert np.all(r["topk_idx"] == np.arange(s.top_k))
        assert np.allclose(r["topk_w"], 1.0 / s.top_k, atol=1e-7)


def test_duplicate_router_columns_tie_break(torch):
    """Bit-identical logits for experts 2 and 5 (same column, same large
    bias): the lower id must win when only one fits."""
    s = MID.with_tokens(40)
    x, w, _ = G.make_inputs(s)
    w["router"] = w["router"].copy()
    w["router"][:, 5] = w["router"][:, 2]
    bias = np.zeros(s.experts, dtype=np.float32)
    bias[[2, 5]] = 100.0
    bias[7] = 200.0
    # k = 4: 7 first, then 2 and 5 (tied), then the best other; with k=2 only 2 fits
    from sparse_moe_transformer_amd import MoeFFN
    ffn = MoeFFN(s.hidden, s.experts, 2, s.expert_dim, s.dense_dim, 40)
    out, r, _, _ = run_gpu(torch, s, x, w, bias, AUTO, ffn=ffn)
    assert np.all(r["topk_idx"] == np.array([2, 7]))
    ref = oracle.moe_ffn(x, w["router"], w["gate"], w["up"], w["down"], w["dgate"], w["dup"],
                         w["ddown"], top_k=2, bias=bias)
    G.assert_block_close(out, ref["out"])


@pytest.mark.parametrize("T", [8, 333])
def test_determinism(torch, T):
    s = MID.with_tokens(T)
    x, w, bias = G.make_inputs(s)
    for variant in (STREAM, MFMA):
        ffn = ffn_for(s, variant)
        a, ra, _, _ = run_gpu(torch, s, x, w, bias, variant, ffn=ffn)
        b, rb, _, _ = run_gpu(torch, s, x, w, bias, variant, ffn=ffn)
        assert np.array_equal(a, b)
        for n in ra:
            assert np.array_equal(ra[n], rb[n]), n


def test_accumulate_in_place(torch):
    """MOE_FFN_ACCUMULATE with out == x: x <- x + block(x)."""
    s = MID.with_tokens(65)
    x, w, _ = G.make_inputs(s)
    for variant in (STREAM, MFMA):
        ffn = ffn_for(s, variant, accumulate=True)
        xd = G.up_bf16(x)
        ffn.forward(xd, G.up_weights(w), xd)
        torch.cuda.synchronize()
        got = G.to_f64(xd)
        ref = oracle.widen_bf16(x) + oracle.moe_ffn(x, w["router"], w["gate"], w["up"], w["down"],
                                                    w["dgate"], w["dup"], w["ddown"], top_k=s.top_k)["out"]
        G.assert_block_close(got, ref)


# ---------------------------------------------------------------------------
# grouping with injected routing
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("case", ["hot", "uniform", "sparse", "single"])
def test_align_only(torch, case):
    E, k = 32, 4
    rng = np.random.default_rng(5)
    T = {"hot": 300, "uniform": 1000, "sparse": 129, "single": 1}[case]
    if case == "hot":      # every token picks experts 0..3: one expert gets all T rows
        idx = np.broadcast_to(np.arange(k), (T, k)).copy()
    elif case == "sparse":  # only 5 experts used, many empty
        idx = np.sort(np.stack([rng.choice(5, k, replace=False) for _ in range(T)]), 1)
    else:
        idx = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]), 1)
    from sparse_moe_transformer_amd import MoeFFN
    ffn = MoeFFN(512, E, k, 128, 192, T)
    ffn.align_only(G.up(idx.astype(np.int32)))
    torch.cuda.synchronize()
    r = {n: G.to_np(v) for n, v in ffn.routing(T).items()}
    assert np.array_equal(r["topk_idx"], idx)
    G.check_align(r, idx, E)


# ---------------------------------------------------------------------------
# the 26B-A4B layer shape
# ---------------------------------------------------------------------------


@pytest.fixture(scope="module")
def w26():
    return synth.make_weights(synth.DECODE)


@pytest.mark.parametrize("variant", [AUTO, MFMA])
def test_decode_26b(torch, w26, variant):
    s = synth.DECODE
    x = synth.make_x(s)
    out, r, inter, _ = run_gpu(torch, s, x, w26, None, variant)
    _, near = full_check(s, x, w26, None, out, r, inter)
    print(f"decode near-ties: {near}, active experts: {int((r['counts'] > 0).sum())}")


def test_prefill_26b(torch, w26):
    s = synth.PREFILL
    x = synth.make_x(s)
    out, r, inter, _ = run_gpu(torch, s, x, w26, None, AUTO)
    _, near = full_check(s, x, w26, None, out, r, inter)
    print(f"prefill near-ties: {near}")


def test_skew_26b(torch, w26):
    """T = 16384 with Zipf(1.2) loads: the busiest experts hold ~11K rows
    (43 M-tiles of one expert), the coldest ~150; every element checked."""
    s = synth.SKEW
    x = synth.make_x(s)
    bias = synth.zipf_bias(s.experts)
    out, r, inter, _ = run_gpu(torch, s, x, w26, bias, AUTO)
    _, near = full_check(s, x, w26, bias, out, r, inter)
    loads = r["counts"]
    print(f"skew near-ties: {near}; max/mean load {loads.max() / loads.mean():.2f}")
    assert loads.max() / loads.mean() > 5


# A mid shape whose hot experts take more than 512 rows each (biased logits:
# 4 experts picked by nearly every token, 8 more by a large share), so the
# second and later M-tiles of an expert, their ragged last tile and the tile
# remap are compared in full; the other experts share the remaining slots.
HOT_T = 1200


def hot_bias(E, seed=0):
    rng = np.random.default_rng(seed)
    b = np.zeros(E, dtype=np.float32)
    hot = rng.choice(E, 12, replace=False)
    b[hot[:4]] = 4.0
    b[hot[4:]] = 1.5
    return b


@pytest.mark.parametrize("variant", [AUTO, MFMA])
def test_hot_experts_many_mtiles(torch, variant):
    s = MID128.with_tokens(HOT_T)
    x, w, _ = G.make_inputs(s, seed=21)
    bias = hot_bias(s.experts)
    out, r, inter, _ = run_gpu(torch, s, x, w, bias, variant)
    full_check(s, x, w, bias, out, r, inter)
    c = r["counts"]
    assert (c > 512).sum() >= 4 and (c > 0).sum() > 64, c


# ---------------------------------------------------------------------------
# NVFP4 weight-only
# ---------------------------------------------------------------------------


def nvfp4_inputs(shape, seed=0):
    x = synth.make_x(shape, seed)
    w = synth.make_weights(shape, seed)
    pk = {"router": w["router"]}
    for n in ("gate", "up", "down"):
        pk[n] = synth.nvfp4_pack_stack(w[n])
    for n in ("dgate", "dup", "ddown"):
        pk[n] = synth.nvfp4_pack_stack(w[n][None]) if w[n] is not None else None
    return x, w, pk


@pytest.mark.parametrize("T", [32, 65, 200])
def test_nvfp4_block(torch, T):
    s = synth.FFNShape("mid_fp4", T, 512, 32, 4, 128, 192, nvfp4=True)
    x, w, pk = nvfp4_inputs(s, seed=T)
    out, r, inter, _ = run_gpu(torch, s, x, pk, None, AUTO, nvfp4=True)
    full_check(s, x, w, None, out, r, inter, nvfp4_w=pk)


@pytest.mark.parametrize("variant", [AUTO, MFMA, STREAM])
def test_nvfp4_every_token_count(torch, variant):
    """NVFP4 weights at every T from 1 to 64 on one handle, each forward
    checked in full.  AUTO streams the packed weights (k_fs4_*) up to T = 32
    and runs the register-fed MFMA tiles (k_fp4mm) above; MFMA runs the tiles
    at every T (one 32-row tile per expert up to T = 32, 128-row tiles above);
    STREAM streams at every T."""
    s64 = synth.FFNShape("mid_fp4", 64, 512, 32, 4, 128, 192, nvfp4=True)
    _, w, pk = nvfp4_inputs(s64, seed=9)
    from sparse_moe_transformer_amd import MoeFFN
    ffn = MoeFFN.for_shape(s64, max_tokens=64, variant=variant)
    wd = G.up_nvfp4_weights(pk)
    for T in range(1, 65):
        s = s64.with_tokens(T)
        x = synth.make_x(s, seed=500 + T)
        xd = G.up_bf16(x)
        out = torch.empty_like(xd)
        ffn.forward_nvfp4(xd, wd, out)
        torch.cuda.synchronize()
        r = {k: G.to_np(v) for k, v in ffn.routing(T).items()}
        full_check(s, x, w, None, G.to_f64(out), r, ffn.intermediates(T), nvfp4_w=pk)


@pytest.mark.parametrize("T", [1, 16])
def test_nvfp4_stream_wide_expert(torch, T):
    """Streamed NVFP4 with an expert width of 1024: the down units' chunk
    loads take several batches per column (the 26B shape needs one)."""
    s = synth.FFNShape("wide_fp4", T, 512, 16, 2, 1024, 256, nvfp4=True)
    x, w, pk = nvfp4_inputs(s, seed=40 + T)
    out, r, inter, _ = run_gpu(torch, s, x, pk, None, STREAM, nvfp4=True)
    full_check(s, x, w, None, out, r, inter, nvfp4_w=pk)


@pytest.mark.parametrize("variant", [AUTO, MFMA])
def test_nvfp4_decode_26b(torch, variant):
    """The 26B NVFP4 layer at T = 8: streamed (AUTO) and on the MFMA tiles."""
    s = synth.NVFP4_STACK.with_tokens(8)
    x = synth.make_x(s)
    pk = synth.make_nvfp4_weights(s)
    out, r, inter, _ = run_gpu(torch, s, x, pk, None, variant, nvfp4=True)
    full_check(s, x, pk, None, out, r, inter, nvfp4_w=pk)


def test_nvfp4_hot_experts(torch):
    """NVFP4 B tiles on experts with more than 512 rows (several M-tiles each)."""
    s = synth.FFNShape("mid128_fp4", HOT_T, 512, 128, 8, 128, 128, nvfp4=True)
    x, w, pk = nvfp4_inputs(s, seed=22)
    bias = hot_bias(s.experts, seed=1)
    out, r, inter, _ = run_gpu(torch, s, x, pk, bias, AUTO, nvfp4=True)
    full_check(s, x, w, bias, out, r, inter, nvfp4_w=pk)
    assert (r["counts"] > 512).sum() >= 4


def test_nvfp4_26b(torch):
    s = synth.NVFP4_STACK
    x = synth.make_x(s)
    pk = synth.make_nvfp4_weights(s)
    out, r, inter, _ = run_gpu(torch, s, x, pk, None, AUTO, nvfp4=True)
    _, near = full_check(s, x, pk, None, out, r, inter, nvfp4_w=pk)
    print(f"nvfp4 26B layer near-ties: {near}")


@pytest.mark.parametrize("case", ["26b_t1024", "ragged"])
def test_nvfp4_repeatable(torch, case):
    """NVFP4 tiles give bit-identical, finite results on repeated calls.

    A block whose last column group lies partly past the matrix has waves
    without columns: they copy their share of every A stage for the other
    waves and compute nothing.  Such a wave must not reach a step's barrier
    before its own A copies of that step have landed, or the other waves read
    stale LDS.  At the 26B shape (T = 1024, 128-row tiles of 8 column waves)
    the last dense gate/up block has 2 of its 8 waves inside the 2112
    columns, the last routed gate/up block 6 of 8 and the last down blocks 4
    of 8; in the ragged case (T = 100, the same tiles) the last blocks keep
    2 of 8 waves (dense gate/up, D = 320), 6 of 8 (routed gate/up, I = 192)
    and 4 of 8 (down, H = 768)."""
    if case == "26b_t1024":
        s = synth.NVFP4_STACK
        x = synth.make_x(s)
        pk = synth.make_nvfp4_weights(s)
        w = pk
    else:
        s = synth.FFNShape("ragged_fp4", 100, 768, 16, 2, 192, 320, nvfp4=True)
        x, w, pk = nvfp4_inputs(s, seed=51)
    ffn = None
    first = None
    for rep in range(4):
        out, r, inter, ffn = run_gpu(torch, s, x, pk, None, MFMA, nvfp4=True, ffn=ffn)
        vals = [out] + [G.to_f64(inter[n]) for n in ("h", "y", "h_d", "y_d")]
        for v in vals:
            assert np.isfinite(v).all(), f"{case}: non-finite values on call {rep}"
        if first is None:
            first = vals
            if case != "26b_t1024":  # the 26B layer's oracle check is test_nvfp4_26b
                full_check(s, x, w, None, out, r, inter, nvfp4_w=pk)
        else:
            for name, a, b in zip(("out", "h", "y", "h_d", "y_d"), first, vals):
                assert np.array_equal(a, b), f"{case}: {name} differs between call 0 and call {rep}"


# Layers of the NVFP4 residual stack in this test (the stack has 30; set
# MOE_STACK_LAYERS=30 to run all of them, ~15 s of host work per layer).
STACK_LAYERS = int(os.environ.get("MOE_STACK_LAYERS", "4"))


def test_nvfp4_stack(torch):
    """The NVFP4 residual stack at T = 1024 (x <- x + FFN_l(x) in place, the
    accumulate flag, out == x), STACK_LAYERS distinct seeded layers.

    Each layer is checked teacher-forced on every token: the oracle takes the
    GPU's own layer input (the bf16 values the GPU stored) and the output
    must follow the bf16 rule.  Beside it the oracle runs its own chain in
    fp64 from the same x (never teacher-forced) and the end-to-end error of
    the GPU's chain against it is reported, over all tokens and over the
    tokens whose routing sets agree with the oracle chain's at every layer
    so far.  It is a report, not a bound: the GPU's residual stream is bf16
    (the model's activation type) and each layer's differences, which the
    teacher-forced check bounds, propagate through the later layers; a token
    whose set differs from the oracle chain's at some layer (a near-tie, or
    a gap the accumulated differences have closed) follows another, equally
    valid path.  Both oracle evaluations of a layer are one call on the
    stacked rows (the block is row-independent), so each layer's weights are
    decoded once."""
    from sparse_moe_transformer_amd import MoeFFN
    s = synth.NVFP4_STACK
    T = s.tokens
    ffn = MoeFFN.for_shape(s, accumulate=True)
    x0 = synth.make_x(s)
    xd = G.up_bf16(x0)
    chain = oracle.widen_bf16(x0)  # the oracle's own chain, fp64
    agree = np.ones(T, dtype=bool)
    total_near = 0
    for layer in range(STACK_LAYERS):
        pk = synth.make_nvfp4_weights(s, layer=layer)
        x_in = G.to_np(xd.view(torch.int16)).view(np.uint16).copy()
        ffn.forward_nvfp4(xd, G.up_nvfp4_weights(pk), xd)
        torch.cuda.synchronize()
        r = {n: G.to_np(v) for n, v in ffn.routing(T).items()}
        rt = oracle.route(x_in, pk["router"], s.top_k)
        near = G.check_routing(r["topk_idx"], r["topk_w"], rt)
        G.check_align(r, r["topk_idx"], s.experts)
        total_near += int(near.sum())
        rc = oracle.route(chain, pk["router"], s.top_k)
        both = np.concatenate([oracle.widen_bf16(x_in), chain])
        sets = np.concatenate([r["topk_idx"], rc["topk_idx"]])
        ref = oracle.moe_ffn(both, pk["router"], pk["gate"], pk["up"], pk["down"], pk["dgate"], pk["dup"],
                             pk["ddown"], top_k=s.top_k, force_routing=sets, intermediates=False)
        got = G.to_f64(xd)
        G.assert_block_close(got, both[:T] + ref["out"][:T], what=f"layer {layer} (teacher-forced)")
        chain = chain + ref["out"][T:]
        agree &= np.all(r["topk_idx"] == rc["topk_idx"], axis=1)
        _, ratio_all = G.block_close(got, chain)
        _, ratio_agree = G.block_close(got[agree], chain[agree])
        rms = np.sqrt(np.mean(chain ** 2))
        rel = float(np.max(np.abs(got - chain)) / rms)
        rel_agree = float(np.max(np.abs(got[agree] - chain[agree])) / rms)
        rms_err = float(np.sqrt(np.mean((got - chain) ** 2)) / rms)
        print(f"stack layer {layer}: near-ties {int(near.sum())}; end-to-end vs the oracle chain: "
              f"worst |err| / (2e-2 (|ref| + rms)) {ratio_all:.3f} over all tokens, {ratio_agree:.3f} over the "
              f"{int(agree.sum())} tokens with identical sets so far; max |err| / rms {rel:.2e} "
              f"({rel_agree:.2e} on those tokens), rms err / rms {rms_err:.2e}", flush=True)
    print(f"stack of {STACK_LAYERS} layers: {total_near} near-tie tokens in total; "
          f"{T - int(agree.sum())} tokens left the oracle chain's routing at some layer")


# ---------------------------------------------------------------------------
# argument validation with a live handle
# ---------------------------------------------------------------------------


def test_validation_with_handle(torch):
    from sparse_moe_transformer_amd import binding as B
    from sparse_moe_transformer_amd import MoeFFN
    s = MID.with_tokens(16)
    ffn = MoeFFN.for_shape(s)
    x, w, _ = G.make_inputs(s)
    xd, wd = G.up_bf16(x), G.up_weights(w)
    out = torch.empty_like(xd)
    p = {k: v.data_ptr() for k, v in wd.items()}
    args = [p["router"], None, p["gate"], p["up"], p["down"], p["dgate"], p["dup"], p["ddown"]]
    st = torch.cuda.current_stream().cuda_stream
    assert B.moe_ffn_forward(ffn.h, 0, xd.data_ptr(), *args, out.data_ptr(), st) == B.MOE_FFN_OK
    assert B.moe_ffn_forward(ffn.h, 17, xd.data_ptr(), *args, out.data_ptr(), st) == B.MOE_FFN_ERR_INVALID_ARG
    assert B.moe_ffn_forward(ffn.h, -1, xd.data_ptr(), *args, out.data_ptr(), st) == B.MOE_FFN_ERR_INVALID_ARG
    assert B.moe_ffn_forward(ffn.h, 16, xd.data_ptr() + 2, *args, out.data_ptr(), st) == B.MOE_FFN_ERR_INVALID_ARG
    assert B.moe_ffn_forward(ffn.h, 16, None, *args, out.data_ptr(), st) == B.MOE_FFN_ERR_INVALID_ARG
    bad = list(args)
    bad[5] = None
    assert B.moe_ffn_forward(ffn.h, 16, xd.data_ptr(), *bad, out.data_ptr(), st) == B.MOE_FFN_ERR_INVALID_ARG
    assert B.moe_ffn_forward(ffn.h, 16, xd.data_ptr(), *args, xd.data_ptr(), st) == B.MOE_FFN_ERR_INVALID_ARG
    assert B.moe_ffn_forward_nvfp4(ffn.h, 16, xd.data_ptr(), p["router"], None, None, None, None,
                                   None, None, None, out.data_ptr(), st) == B.MOE_FFN_ERR_UNSUPPORTED
    assert B.moe_ffn_set_variant(ffn.h, 9) == B.MOE_FFN_ERR_INVALID_ARG
    assert B.moe_ffn_forward(ffn.h, 16, xd.data_ptr(), *args, out.data_ptr(), st) == B.MOE_FFN_OK
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# the sub-block with its sandwich norms and the residual
# ---------------------------------------------------------------------------


def norm_gains(H, seed=0):
    """Seeded per-channel gains around 1 for the pre- and post-norm."""
    rng = np.random.default_rng(1000 + seed)
    return ((1.0 + 0.2 * rng.standard_normal(H)).astype(np.float32),
            (1.0 + 0.2 * rng.standard_normal(H)).astype(np.float32))


def run_block(torch, shape, x, w, pre, post, eps, variant, in_place=False, ffn=None):
    T = x.shape[0]
    ffn = ffn or ffn_for(shape, variant, max_tokens=T)
    xd = G.up_bf16(x)
    out = xd if in_place else torch.empty_like(xd)
    ffn.forward_block(xd, G.up_weights(w), G.up(pre), G.up(post), out, eps=eps)
    torch.cuda.synchronize()
    r = {k: G.to_np(v) for k, v in ffn.routing(T).items()}
    return G.to_f64(out), r


# The pre-normed input is a stored bf16 activation.  Both sides decide its
# rounding in fp32, but their fp32 operation orders differ (the hardware
# reciprocal square root, the order of the two products), so a handful of
# elements per thousand tokens land one bf16 step apart.  One step moves a
# router logit by ~3e-4 (below the 1e-3 near-tie gap, so the sets stay
# bit-exact) and a routing weight by up to ~1e-4: the weights are compared
# to 1e-3 here instead of 1e-5.
BLOCK_W_TOL = 1e-3


def block_check(shape, x, w, pre, post, eps, out, r):
    """Routing of the pre-normed input and every element of the block output
    against oracle.moe_block (run once, on the GPU's sets, after the sets
    are checked against the oracle's own routing of its pre-normed rows)."""
    xn = oracle.round_bf16(oracle.rms_norm(oracle.widen_bf16(x), pre, eps))
    rt = oracle.route(xn, w["router"], shape.top_k)
    near = G.check_routing(r["topk_idx"], r["topk_w"], rt, w_tol=BLOCK_W_TOL)
    G.check_align(r, r["topk_idx"], shape.experts)
    ref = oracle.moe_block(x, pre, post, eps, w["router"], w["gate"], w["up"], w["down"], w.get("dgate"),
                           w.get("dup"), w.get("ddown"), top_k=shape.top_k, force_routing=r["topk_idx"])
    G.assert_block_close(out, ref["out"])
    return int(near.sum())


@pytest.mark.parametrize("variant", [AUTO, STREAM, MFMA])
def test_block_tiny(torch, variant):
    s = synth.TINY
    x, w, _ = G.make_inputs(s)
    pre, post = norm_gains(s.hidden)
    out, r = run_block(torch, s, x, w, pre, post, 1e-6, variant)
    block_check(s, x, w, pre, post, 1e-6, out, r)


@pytest.mark.parametrize("T", [1, 33, 200])
def test_block_ragged(torch, T):
    s = MID.with_tokens(T)
    x, w, _ = G.make_inputs(s, seed=T)
    pre, post = norm_gains(s.hidden, seed=T)
    out, r = run_block(torch, s, x, w, pre, post, 1e-6, AUTO)
    block_check(s, x, w, pre, post, 1e-6, out, r)


def test_block_decode_26b(torch, w26):
    s = synth.DECODE
    x = synth.make_x(s)
    pre, post = norm_gains(s.hidden)
    out, r = run_block(torch, s, x, w26, pre, post, 1e-6, AUTO)
    near = block_check(s, x, w26, pre, post, 1e-6, out, r)
    print(f"block decode near-ties: {near}")


def test_block_prefill_26b(torch, w26):
    s = synth.PREFILL
    x = synth.make_x(s)
    pre, post = norm_gains(s.hidden, seed=1)
    out, r = run_block(torch, s, x, w26, pre, post, 1e-6, AUTO)
    near = block_check(s, x, w26, pre, post, 1e-6, out, r)
    print(f"block prefill near-ties: {near}")


@pytest.mark.parametrize("variant", [STREAM, MFMA])
def test_block_in_place(torch, variant):
    """out = x: the residual stream updated in place."""
    s = MID.with_tokens(16)
    x, w, _ = G.make_inputs(s, seed=5)
    pre, post = norm_gains(s.hidden, seed=5)
    out, r = run_block(torch, s, x, w, pre, post, 1e-6, variant, in_place=True)
    block_check(s, x, w, pre, post, 1e-6, out, r)


def test_block_validation(torch):
    from sparse_moe_transformer_amd import binding as B
    from sparse_moe_transformer_amd import MoeFFN
    s = MID.with_tokens(16)
    x, w, _ = G.make_inputs(s)
    xd, wd = G.up_bf16(x), G.up_weights(w)
    pre, post = (G.up(g) for g in norm_gains(s.hidden))
    out = torch.empty_like(xd)
    p = {k: v.data_ptr() for k, v in wd.items()}
    wargs = [p["gate"], p["up"], p["down"], p["dgate"], p["dup"], p["ddown"]]
    st = torch.cuda.current_stream().cuda_stream
    ffn = MoeFFN.for_shape(s)

    def call(h, T=16, xp=xd.data_ptr(), pp=pre.data_ptr(), qp=post.data_ptr(), eps=1e-6, op=out.data_ptr()):
        return B.moe_ffn_forward_block(h, T, xp, pp, qp, eps, p["router"], None, *wargs, op, st)

    assert call(ffn.h) == B.MOE_FFN_OK
    assert call(ffn.h, T=0) == B.MOE_FFN_OK
    assert call(ffn.h, T=17) == B.MOE_FFN_ERR_INVALID_ARG
    assert call(ffn.h, pp=None) == B.MOE_FFN_ERR_INVALID_ARG
    assert call(ffn.h, qp=post.data_ptr() + 4) == B.MOE_FFN_ERR_INVALID_ARG
    assert call(ffn.h, eps=-1.0) == B.MOE_FFN_ERR_INVALID_ARG
    assert call(ffn.h, eps=float("nan")) == B.MOE_FFN_ERR_INVALID_ARG
    assert call(ffn.h, op=xd.data_ptr()) == B.MOE_FFN_OK  # in place is allowed
    acc = MoeFFN.for_shape(s, accumulate=True)
    assert call(acc.h) == B.MOE_FFN_ERR_UNSUPPORTED
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# HIP graph capture: a forward allocates and clears nothing after create
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("variant,T,block", [(STREAM, 8, False), (MFMA, 200, False), (STREAM, 8, True)])
def test_forward_graph_replays(torch, variant, T, block):
    """A forward captured into a graph and replayed on new inputs (written
    into the captured buffer between replays, with eager forwards in
    between) gives, replay after replay, exactly the eager forward's output;
    the routing hand-off counters are back at zero after each replay."""
    s = MID.with_tokens(T)
    x, w, _ = G.make_inputs(s, seed=11)
    ffn = ffn_for(s, variant, max_tokens=T)
    wd = G.up_weights(w)
    pre, post = (G.up(g) for g in norm_gains(s.hidden, seed=3))
    xd = G.up_bf16(x)
    out = torch.empty_like(xd)

    def fwd(dst):
        if block:
            ffn.forward_block(xd, wd, pre, post, dst, eps=1e-6)
        else:
            ffn.forward(xd, wd, dst)

    fwd(out)  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(out)
    torch.cuda.synchronize()
    for i in range(3):
        xi = synth.make_x(s, seed=30 + i)
        xd.copy_(G.up_bf16(xi))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = torch.empty_like(xd)
        fwd(ref)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {i} differs from the eager forward"
        if not block:
            r = oracle.moe_ffn(xi, w["router"], w["gate"], w["up"], w["down"], w["dgate"], w["dup"], w["ddown"],
                               top_k=s.top_k)
            G.assert_block_close(G.to_f64(got), r["out"])
