"""GPU parity of the FP8 weight-only path (e4m3fn codes with one fp32 scale
per matrix, [K, N] layout) through the C ABI against the oracle, which
decodes the same packed bytes (oracle.fp8).

Rules as for the bf16 block: routing sets bit-exact on tokens whose k-th /
(k+1)-th logit gap exceeds 1e-3 (the router stays bf16), the grouping
bit-exact against the oracle's grouping of the GPU's routing, every output
element within 2e-2 * (|oracle| + rms(oracle)), at every size.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

AUTO, STREAM, MFMA = 0, 1, 2
MID = synth.FFNShape("mid", 0, 512, 32, 4, 128, 192, fp8=True)


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available()
    return _t


def fp8_shape(s, T=None):
    from dataclasses import replace
    s = replace(s, fp8=True)
    return s if T is None else s.with_tokens(T)


def run(torch, shape, x, w, variant, bias=None):
    from sparse_moe_transformer_amd import MoeFFN
    T = x.shape[0]
    ffn = MoeFFN.for_shape(shape, max_tokens=T, variant=variant)
    xd = G.up_bf16(x)
    out = torch.empty_like(xd)
    ffn.forward_fp8(xd, G.up_fp8_weights(w), out, G.up(bias) if bias is not None else None)
    torch.cuda.synchronize()
    r = {k: G.to_np(v) for k, v in ffn.routing(T).items()} if shape.experts else None
    return G.to_f64(out), r


def check(shape, x, w, out, r, tokens=None, bias=None):
    """Routing and grouping of every token; output rows (all, or `tokens`)."""
    rt = oracle.route(x, w["router"], shape.top_k, bias)
    near = G.check_routing(r["topk_idx"], r["topk_w"], rt)
    G.check_align(r, r["topk_idx"], shape.experts)
    ref = oracle.moe_ffn(x, w["router"], w["gate"], w["up"], w["down"], w.get("dgate"), w.get("dup"),
                         w.get("ddown"), top_k=shape.top_k, bias=bias, force_routing=r["topk_idx"],
                         tokens=tokens, intermediates=False)
    G.assert_block_close(out if tokens is None else out[tokens], ref["out"])
    return int(near.sum())


@pytest.mark.parametrize("variant", [AUTO, STREAM, MFMA])
def test_fp8_tiny(torch, variant):
    s = fp8_shape(synth.TINY)
    x, w = synth.make_x(s), synth.make_fp8_weights(s)
    out, r = run(torch, s, x, w, variant)
    assert check(s, x, w, out, r) == 0


@pytest.mark.parametrize("T", [1, 3, 8, 33, 65, 200])
@pytest.mark.parametrize("variant", [STREAM, MFMA])
def test_fp8_ragged(torch, T, variant):
    s = MID.with_tokens(T)
    x, w = synth.make_x(s, seed=T), synth.make_fp8_weights(s, seed=T)
    out, r = run(torch, s, x, w, variant)
    check(s, x, w, out, r)


@pytest.fixture(scope="module")
def w26_fp8():
    return synth.make_fp8_weights(fp8_shape(synth.DECODE))


@pytest.mark.parametrize("variant", [AUTO, MFMA])
def test_fp8_decode_26b(torch, w26_fp8, variant):
    s = fp8_shape(synth.DECODE)
    x = synth.make_x(s)
    out, r = run(torch, s, x, w26_fp8, variant)
    print(f"fp8 decode near-ties: {check(s, x, w26_fp8, out, r)}")


def test_fp8_prefill_26b(torch, w26_fp8):
    s = fp8_shape(synth.PREFILL)
    x = synth.make_x(s)
    out, r = run(torch, s, x, w26_fp8, AUTO)
    print(f"fp8 prefill near-ties: {check(s, x, w26_fp8, out, r)}")


def test_fp8_hot_experts(torch):
    """FP8 B tiles on experts with more than 512 rows (several M-tiles each):
    4 experts picked by nearly every token, 8 more by a large share."""
    s = synth.FFNShape("mid128_fp8", 1200, 512, 128, 8, 128, 128, fp8=True)
    x, w = synth.make_x(s, seed=23), synth.make_fp8_weights(s, seed=23)
    rng = np.random.default_rng(2)
    bias = np.zeros(s.experts, dtype=np.float32)
    hot = rng.choice(s.experts, 12, replace=False)
    bias[hot[:4]], bias[hot[4:]] = 4.0, 1.5
    out, r = run(torch, s, x, w, AUTO, bias=bias)
    check(s, x, w, out, r, bias=bias)
    assert (r["counts"] > 512).sum() >= 4


@pytest.mark.parametrize("T", [8, 300])
def test_fp8_dense_ffn_e4b(torch, T):
    """The E4B dense FFN with FP8 matrices (streaming at T = 8, MFMA at 300)."""
    s = fp8_shape(synth.E4B_DECODE, T)
    x = synth.make_x(s, seed=T)
    w = synth.make_fp8_weights(s, seed=T)
    out, _ = run(torch, s, x, w, AUTO)
    ref = oracle.dense_ffn(x, w["dgate"], w["dup"], w["ddown"])
    G.assert_block_close(out, ref["out"])


def test_fp8_streaming_every_token_count(torch):
    """FP8 streaming at every T from 1 to 64 on one handle (128-column units
    with a ragged last unit at I = 128 + dense 192, the GeGLU pass), each
    forward checked in full."""
    from sparse_moe_transformer_amd import MoeFFN
    ffn = MoeFFN.for_shape(MID, max_tokens=64, variant=STREAM)
    w = synth.make_fp8_weights(MID.with_tokens(64), seed=5)
    wd = G.up_fp8_weights(w)
    for T in range(1, 65):
        s = MID.with_tokens(T)
        x = synth.make_x(s, seed=200 + T)
        xd = G.up_bf16(x)
        out = torch.empty_like(xd)
        ffn.forward_fp8(xd, wd, out)
        torch.cuda.synchronize()
        r = {k: G.to_np(v) for k, v in ffn.routing(T).items()}
        check(s, x, w, G.to_f64(out), r)


def test_fp8_validation(torch):
    from sparse_moe_transformer_amd import MoeFFN, binding as B
    s = MID.with_tokens(16)
    x, w = synth.make_x(s), synth.make_fp8_weights(s)
    xd, wd = G.up_bf16(x), G.up_fp8_weights(w)
    out = torch.empty_like(xd)
    st = torch.cuda.current_stream().cuda_stream
    d = {n: (wd[n]["q8"].data_ptr(), wd[n]["tensor_scale"].data_ptr()) for n in
         ("gate", "up", "down", "dgate", "dup", "ddown")}
    ffn = MoeFFN.for_shape(s)

    def call(h, **kw):
        a = dict(d)
        a.update(kw)
        return B.moe_ffn_forward_fp8(h, 16, xd.data_ptr(), wd["router"].data_ptr(), None, a["gate"], a["up"],
                                     a["down"], a["dgate"], a["dup"], a["ddown"], out.data_ptr(), st)

    assert call(ffn.h) == B.MOE_FFN_OK
    assert call(ffn.h, gate=None) == B.MOE_FFN_ERR_INVALID_ARG
    assert call(ffn.h, up=(d["up"][0], None)) == B.MOE_FFN_ERR_INVALID_ARG
    assert call(ffn.h, down=(d["down"][0] + 8, d["down"][1])) == B.MOE_FFN_ERR_INVALID_ARG
    bf = MoeFFN(s.hidden, s.experts, s.top_k, s.expert_dim, s.dense_dim, 16)
    assert call(bf.h) == B.MOE_FFN_ERR_UNSUPPORTED  # a bf16 handle
    torch.cuda.synchronize()
