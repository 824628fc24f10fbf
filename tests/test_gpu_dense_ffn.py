"""GPU parity of the dense FFN: a config without experts, i.e. the feed-forward
block of the E4B model (gemma-llm API page gm.nn.Gemma4_E4B: embed_dim 2560,
hidden_dim 10240, enable_moe False), through the C ABI against
oracle.dense_ffn / oracle.dense_block.

Rule: every output element within 2e-2 * (|oracle| + rms(oracle)) (bf16
output), at every size.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

AUTO, STREAM, MFMA = 0, 1, 2

# D = 1600: 25 row groups of 64, so the streamed dense-down K-slices are
# uneven (6, 6, 6, 7 groups) and the MFMA gate/up tiles end half-full
E4B_MID = synth.FFNShape("e4b_mid", 0, 512, 0, 0, 0, 1600)


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available()
    return _t


@pytest.fixture(scope="module")
def w_e4b():
    return synth.make_weights(synth.E4B_DECODE)


def ffn_for(shape, variant=AUTO, max_tokens=None, accumulate=False):
    from sparse_moe_transformer_amd import MoeFFN
    return MoeFFN.for_shape(shape, max_tokens=max_tokens or max(shape.tokens, 1), variant=variant,
                            accumulate=accumulate)


def run(torch, shape, x, w, variant, nvfp4=False):
    T = x.shape[0]
    ffn = ffn_for(shape, variant, max_tokens=T)
    xd = G.up_bf16(x)
    out = torch.empty_like(xd)
    if nvfp4:
        ffn.forward_nvfp4(xd, G.up_nvfp4_weights(w), out)
    else:
        ffn.forward(xd, G.up_weights(w), out)
    torch.cuda.synchronize()
    return G.to_f64(out), ffn


def ref_ffn(x, w, tokens=None):
    return oracle.dense_ffn(x, w["dgate"], w["dup"], w["ddown"], tokens=tokens)


@pytest.mark.parametrize("variant", [AUTO, STREAM, MFMA])
def test_dense_tiny(torch, variant):
    s = synth.E4B_TINY
    x, w = synth.make_x(s), synth.make_weights(s)
    out, ffn = run(torch, s, x, w, variant)
    ref = ref_ffn(x, w)
    G.assert_block_close(out, ref["out"])
    if variant == STREAM:
        # the hidden rows and the dense output rows of the streamed forward
        inter = ffn.intermediates(s.tokens)
        torch.cuda.synchronize()
        G.assert_block_close(G.to_f64(inter["h_d"]), ref["h_d"], what="h_d")
        G.assert_block_close(G.to_f64(inter["y_d"]), ref["y_d"], what="y_d")


@pytest.mark.parametrize("T", [1, 2])
def test_dense_tiny_two_rows_per_thread(torch, T):
    """H = 256 in 4 K-slices: each streaming thread owns 2 rows of a slice,
    half of a 4-row activation piece (1-2 tokens read activations directly)."""
    s = synth.E4B_TINY.with_tokens(T)
    x, w = synth.make_x(s, seed=9), synth.make_weights(s, seed=9)
    out, _ = run(torch, s, x, w, STREAM)
    G.assert_block_close(out, ref_ffn(x, w)["out"])


@pytest.mark.parametrize("T", [1, 2, 3, 33, 64, 65, 200])
@pytest.mark.parametrize("variant", [STREAM, MFMA])
def test_dense_ragged(torch, T, variant):
    s = E4B_MID.with_tokens(T)
    x, w = synth.make_x(s, seed=T), synth.make_weights(s, seed=T)
    out, _ = run(torch, s, x, w, variant)
    G.assert_block_close(out, ref_ffn(x, w)["out"])


def test_dense_streaming_every_token_count(torch):
    """The dense-only streaming path at every T from 1 to 64 on one handle
    (uneven K-slices at D = 1600), each forward checked in full."""
    ffn = ffn_for(E4B_MID, STREAM, max_tokens=64)
    w = synth.make_weights(E4B_MID.with_tokens(64), seed=6)
    wd = G.up_weights(w)
    for T in range(1, 65):
        s = E4B_MID.with_tokens(T)
        x = synth.make_x(s, seed=300 + T)
        xd = G.up_bf16(x)
        out = torch.empty_like(xd)
        ffn.forward(xd, wd, out)
        torch.cuda.synchronize()
        G.assert_block_close(G.to_f64(out), ref_ffn(x, w)["out"])


@pytest.mark.parametrize("variant", [AUTO, MFMA])
def test_dense_e4b_decode(torch, w_e4b, variant):
    s = synth.E4B_DECODE
    x = synth.make_x(s)
    out, _ = run(torch, s, x, w_e4b, variant)
    G.assert_block_close(out, ref_ffn(x, w_e4b)["out"])


def test_dense_e4b_prefill(torch, w_e4b):
    s = synth.E4B_PREFILL
    x = synth.make_x(s)
    out, _ = run(torch, s, x, w_e4b, AUTO)
    G.assert_block_close(out, ref_ffn(x, w_e4b)["out"])


@pytest.mark.parametrize("variant", [STREAM, MFMA])
def test_dense_accumulate_in_place(torch, variant):
    """MOE_FFN_ACCUMULATE with out == x: x <- x + FFN(x)."""
    s = E4B_MID.with_tokens(40)
    x, w = synth.make_x(s, seed=3), synth.make_weights(s, seed=3)
    ffn = ffn_for(s, variant, accumulate=True)
    xd = G.up_bf16(x)
    ffn.forward(xd, G.up_weights(w), xd)
    torch.cuda.synchronize()
    G.assert_block_close(G.to_f64(xd), oracle.widen_bf16(x) + ref_ffn(x, w)["out"])


def norm_gains(H, seed=0):
    rng = np.random.default_rng(2000 + seed)
    return ((1.0 + 0.2 * rng.standard_normal(H)).astype(np.float32),
            (1.0 + 0.2 * rng.standard_normal(H)).astype(np.float32))


@pytest.mark.parametrize("shape,variant", [(synth.E4B_TINY, STREAM), (synth.E4B_TINY, MFMA),
                                           (E4B_MID.with_tokens(100), AUTO), (synth.E4B_DECODE, AUTO)])
def test_dense_block(torch, w_e4b, shape, variant):
    """The sandwich sub-block around the dense FFN: x + RMSNorm(FFN(RMSNorm(x)))."""
    x = synth.make_x(shape, seed=4)
    w = w_e4b if shape.name == "e4b_decode" else synth.make_weights(shape, seed=4)
    pre, post = norm_gains(shape.hidden)
    ffn = ffn_for(shape, variant)
    xd = G.up_bf16(x)
    out = torch.empty_like(xd)
    ffn.forward_block(xd, G.up_weights(w), G.up(pre), G.up(post), out, eps=1e-6)
    torch.cuda.synchronize()
    ref = oracle.dense_block(x, pre, post, 1e-6, w["dgate"], w["dup"], w["ddown"])
    G.assert_block_close(G.to_f64(out), ref["out"])


@pytest.mark.parametrize("T", [5, 130])
def test_dense_nvfp4(torch, T):
    """Weight-only NVFP4 dense matrices (decoded in the MFMA tile loads)."""
    s = synth.FFNShape("e4b_mid_fp4", T, 512, 0, 0, 0, 1600, nvfp4=True)
    x = synth.make_x(s, seed=T)
    w = synth.make_nvfp4_weights(s, seed=T)
    out, _ = run(torch, s, x, w, AUTO, nvfp4=True)
    G.assert_block_close(out, ref_ffn(x, w)["out"])


def test_dense_validation(torch):
    from sparse_moe_transformer_amd import binding as B
    s = E4B_MID.with_tokens(16)
    x, w = synth.make_x(s), synth.make_weights(s)
    xd = G.up_bf16(x)
    wd = G.up_weights(w)
    out = torch.empty_like(xd)
    st = torch.cuda.current_stream().cuda_stream
    ffn = ffn_for(s, MFMA)
    p = {k: (v.data_ptr() if v is not None else None) for k, v in wd.items()}
    dense = [p["dgate"], p["dup"], p["ddown"]]

    def call(router=None, gate=None, bias=None):
        return B.moe_ffn_forward(ffn.h, 16, xd.data_ptr(), router, bias, gate, None, None, *dense,
                                 out.data_ptr(), st)

    assert call() == B.MOE_FFN_OK
    assert call(router=xd.data_ptr()) == B.MOE_FFN_ERR_INVALID_ARG
    assert call(gate=xd.data_ptr()) == B.MOE_FFN_ERR_INVALID_ARG
    assert B.moe_ffn_forward(ffn.h, 16, xd.data_ptr(), None, None, None, None, None, None, p["dup"],
                             p["ddown"], out.data_ptr(), st) == B.MOE_FFN_ERR_INVALID_ARG
    # no routing to export; the MFMA dense forward wrote its rows to out only
    assert B.moe_ffn_align_only(ffn.h, 1, xd.data_ptr(), st) == B.MOE_FFN_ERR_UNSUPPORTED
    with pytest.raises(B.MoeFFNError):
        ffn.routing(16)
    with pytest.raises(B.MoeFFNError):
        ffn.intermediates(16)
    torch.cuda.synchronize()
    G.assert_block_close(G.to_f64(out), ref_ffn(x, w)["out"])
