"""GPU: the forward that allocates nothing (moe_ffn_forward_noalloc, whose
workspace is the library's static device array) against moe_ffn_forward on
the same inputs, through the C ABI.

Both run the same kernels, so the outputs must be bit-identical; each is
also held to the bf16 rule against the oracle.  Two calls in a row share the
array: the second, with fewer tokens, must not see anything of the first
(the counters it needs at zero are cleared by the call)."""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

MID = synth.FFNShape("mid", 0, 512, 32, 4, 128, 192)


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available()
    return _t


def noalloc(torch, shape, max_tokens, x, wd, bias=None):
    from sparse_moe_transformer_amd import binding as B
    T = x.shape[0]
    xd = G.up_bf16(x)
    out = torch.full_like(xd, float("nan"))
    cfg = B.make_config(shape.hidden, shape.experts, shape.top_k, shape.expert_dim, shape.dense_dim, max_tokens)
    p = {k: (v.data_ptr() if v is not None else None) for k, v in wd.items()}
    bd = G.up(bias) if bias is not None else None
    st = torch.cuda.current_stream().cuda_stream
    B.check(B.moe_ffn_forward_noalloc(cfg, T, xd.data_ptr(), p["router"], bd.data_ptr() if bd is not None else None,
                                      p["gate"], p["up"], p["down"], p.get("dgate"), p.get("dup"), p.get("ddown"),
                                      out.data_ptr(), st))
    return out


def with_handle(torch, shape, x, wd, bias=None):
    from sparse_moe_transformer_amd import MoeFFN
    T = x.shape[0]
    ffn = MoeFFN.for_shape(shape, max_tokens=T)
    xd = G.up_bf16(x)
    out = torch.empty_like(xd)
    ffn.forward(xd, wd, out, G.up(bias) if bias is not None else None)
    torch.cuda.synchronize()
    ffn.close()
    return out


def oracle_out(x, w, k, bias=None):
    return oracle.moe_ffn(x, w["router"], w["gate"], w["up"], w["down"], w.get("dgate"), w.get("dup"),
                          w.get("ddown"), top_k=k, bias=bias, intermediates=False)["out"]


@pytest.mark.parametrize("shape,Ts", [(synth.DECODE, (8, 3)),       # weight streaming, the 26B layer
                                      (MID, (333, 65)),             # MFMA tiles
                                      (MID, (64, 1))])              # streaming at the largest and smallest T
def test_noalloc_matches_forward(torch, shape, Ts):
    w = synth.make_weights(shape.with_tokens(max(Ts)))
    wd = G.up_weights(w)
    for i, T in enumerate(Ts):
        s = shape.with_tokens(T)
        x = synth.make_x(s, seed=40 + i)
        got = noalloc(torch, s, max(Ts), x, wd)
        torch.cuda.synchronize()
        ref = with_handle(torch, s, x, wd)
        assert torch.equal(got, ref), f"call {i} (T={T}) differs from moe_ffn_forward"
        G.assert_block_close(G.to_f64(got), oracle_out(x, w, s.top_k), what=f"call {i} (T={T})")


def test_noalloc_validation(torch):
    from sparse_moe_transformer_amd import binding as B
    s = MID.with_tokens(16)
    w = synth.make_weights(s)
    wd = G.up_weights(w)
    x = synth.make_x(s)
    xd = G.up_bf16(x)
    out = torch.empty_like(xd)
    p = {k: v.data_ptr() for k, v in wd.items()}
    st = torch.cuda.current_stream().cuda_stream
    args = [p["router"], None, p["gate"], p["up"], p["down"], p["dgate"], p["dup"], p["ddown"]]
    cfg = B.make_config(s.hidden, s.experts, s.top_k, s.expert_dim, s.dense_dim, 16)
    assert B.moe_ffn_forward_noalloc(cfg, 17, xd.data_ptr(), *args, out.data_ptr(), st) == B.MOE_FFN_ERR_INVALID_ARG
    assert B.moe_ffn_forward_noalloc(cfg, 16, None, *args, out.data_ptr(), st) == B.MOE_FFN_ERR_INVALID_ARG
    big = B.make_config(2816, 128, 8, 704, 2112, 4096)
    assert B.moe_ffn_forward_noalloc(big, 4096, xd.data_ptr(), *args, out.data_ptr(), st) == \
        B.MOE_FFN_ERR_UNSUPPORTED
    assert "static scratch" in B.moe_ffn_last_error()
    assert B.moe_ffn_forward_noalloc(cfg, 16, xd.data_ptr(), *args, out.data_ptr(), st) == B.MOE_FFN_OK
    torch.cuda.synchronize()
