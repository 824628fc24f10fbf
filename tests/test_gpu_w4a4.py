"""GPU parity of NVFP4 activations (W4A4) through the C ABI against the
oracle (oracle.quant_act_nvfp4, oracle.moe_ffn_w4a4).

The quantiser's inputs are identical on both sides, so its output (every
scale and code decision, taken in fp32 by one fixed formula) is compared
bit for bit.  The block is compared with the bf16 output rule: routing sets
bit-exact on tokens whose gap exceeds 1e-3, every output element within
2e-2 * (|oracle| + rms(oracle)).  The hidden rows are quantised from the
stored bf16 hidden values, which the two sides may round one step apart
(fp32 vs fp64 accumulation); such a difference can move one code, well
inside the output rule.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

AUTO, STREAM, MFMA = 0, 1, 2


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available()
    return _t


def bf16_bits(v):
    """fp64 values that are exact bf16 values -> uint16 bits."""
    return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def quantise_on_gpu(torch, v, s):
    from sparse_moe_transformer_amd import binding as B
    rows, K = v.shape
    xin = G.up_bf16(synth.bf16_bits(v.astype(np.float32)))
    out = torch.empty_like(xin)
    sd = G.up(np.array([s], dtype=np.float32))
    st = torch.cuda.current_stream().cuda_stream
    assert B.moe_ffn_quant_act_nvfp4(rows, K, xin.data_ptr(), out.data_ptr(), sd.data_ptr(), st) == B.MOE_FFN_OK
    # in place gives the same
    assert B.moe_ffn_quant_act_nvfp4(rows, K, xin.data_ptr(), xin.data_ptr(), sd.data_ptr(), st) == B.MOE_FFN_OK
    torch.cuda.synchronize()
    return (G.to_np(out.view(torch.int16)).view(np.uint16), G.to_np(xin.view(torch.int16)).view(np.uint16))


@pytest.mark.parametrize("scale_mult", [1.0, 1e-3, 1e4])
def test_quantiser_bit_exact(torch, scale_mult):
    """Every group decision equals the oracle's: rows of magnitudes from 1e-6
    to 1e3 and an all-zero row, with the nominal static scale, one that
    saturates many group scales at 448 (x 1e-3) and one that makes them
    subnormal or zero (x 1e4)."""
    rng = np.random.default_rng(21)
    rows, K = 40, 256
    mags = 10.0 ** rng.uniform(-6, 3, size=(rows, K // 16)).repeat(16, axis=1)
    v = rng.standard_normal((rows, K)) * mags
    v[3] = 0.0
    v = oracle.round_bf16(v)
    s = np.float32(np.max(np.abs(v)) / (6 * 448) * scale_mult)
    ref = bf16_bits(oracle.quant_act_nvfp4(v, float(s)))
    got, inplace = quantise_on_gpu(torch, v, s)
    bad = np.flatnonzero(got.reshape(-1) != ref.reshape(-1))
    assert bad.size == 0, f"{bad.size} values differ, e.g. flat index {bad[:5]}"
    assert np.array_equal(inplace, ref)


def test_quantiser_ties_at_unit_scale(torch):
    """With s = fp32(1/6) a group of amax 6 has s_g = 6 and s_g * s = 1, so
    its values are rounded on the e2m1 grid itself: the midpoints between
    grid values go to the even mantissa, values beyond 6 saturate."""
    row = np.array([0, 0.25, 0.3, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6, -1, -2.9, 4.4, 0.5, 1.5, 3.0])
    v = oracle.round_bf16(np.stack([row, -row, np.r_[row[:15], 6.0] * 0.5]))
    s = np.float32(1.0 / 6.0)
    ref = bf16_bits(oracle.quant_act_nvfp4(v, float(s)))
    got, _ = quantise_on_gpu(torch, v, s)
    assert np.array_equal(got, ref)


def static_scales(x, w, pk, k):
    """Static global scales as a min/max observer would set them on this
    input: amax / (6 * 448) of x, of the routed hidden rows and of the dense
    hidden rows (taken from the weight-only oracle forward)."""
    r = oracle.moe_ffn(x, w["router"], pk["gate"], pk["up"], pk["down"], pk.get("dgate"), pk.get("dup"),
                       pk.get("ddown"), top_k=k)
    amax_hd = np.max(np.abs(r["h_d"])) if r["h_d"] is not None else 1.0
    return np.array([np.max(np.abs(oracle.widen_bf16(x))), np.max(np.abs(r["h"])), amax_hd]) / (6 * 448)


def nvfp4_inputs(shape, seed=0):
    x = synth.make_x(shape, seed)
    w = synth.make_weights(shape, seed)
    pk = {"router": w["router"]}
    for n in ("gate", "up", "down"):
        pk[n] = synth.nvfp4_pack_stack(w[n])
    for n in ("dgate", "dup", "ddown"):
        pk[n] = synth.nvfp4_pack_stack(w[n][None]) if w[n] is not None else None
    return x, w, pk


def run(torch, shape, x, pk, scales, variant=AUTO):
    from sparse_moe_transformer_amd import MoeFFN
    T = x.shape[0]
    ffn = MoeFFN.for_shape(shape, max_tokens=T, variant=variant)
    xd = G.up_bf16(x)
    out = torch.empty_like(xd)
    ffn.forward_w4a4(xd, G.up_nvfp4_weights(pk), G.up(np.asarray(scales, dtype=np.float32)), out)
    torch.cuda.synchronize()
    r = {k: G.to_np(v) for k, v in ffn.routing(T).items()}
    return G.to_f64(out), r


def check(shape, x, pk, scales, out, r, tokens=None):
    rt = oracle.route(x, pk["router"], shape.top_k)
    near = G.check_routing(r["topk_idx"], r["topk_w"], rt)
    G.check_align(r, r["topk_idx"], shape.experts)
    ref = oracle.moe_ffn_w4a4(x, pk["router"], pk["gate"], pk["up"], pk["down"], pk.get("dgate"), pk.get("dup"),
                              pk.get("ddown"), np.asarray(scales, dtype=np.float32), top_k=shape.top_k,
                              force_routing=r["topk_idx"], tokens=tokens)
    G.assert_block_close(out if tokens is None else out[tokens], ref["out"])
    return int(near.sum())


def test_w4a4_tiny(torch):
    s = synth.FFNShape("tiny_fp4", 32, 256, 8, 2, 64, 128, nvfp4=True)
    x, w, pk = nvfp4_inputs(s)
    sc = static_scales(x, w, pk, s.top_k)
    out, r = run(torch, s, x, pk, sc)
    assert check(s, x, pk, sc, out, r) == 0


@pytest.mark.parametrize("T", [1, 5, 65, 200])
def test_w4a4_ragged(torch, T):
    s = synth.FFNShape("mid_fp4", T, 512, 32, 4, 128, 192, nvfp4=True)
    x, w, pk = nvfp4_inputs(s, seed=T)
    sc = static_scales(x, w, pk, s.top_k)
    out, r = run(torch, s, x, pk, sc)
    check(s, x, pk, sc, out, r)


def test_w4a4_saturating_scales(torch):
    """Static scales 100x too small: many group scales saturate at 448 and
    many codes at 6; the outputs still follow the oracle."""
    s = synth.FFNShape("mid_fp4", 64, 512, 32, 4, 128, 192, nvfp4=True)
    x, w, pk = nvfp4_inputs(s, seed=3)
    sc = static_scales(x, w, pk, s.top_k) / 100
    out, r = run(torch, s, x, pk, sc)
    check(s, x, pk, sc, out, r)


def test_w4a4_26b(torch):
    s = synth.FFNShape("nvfp4_26b", 256, 2816, 128, 8, 704, 2112, nvfp4=True)
    x = synth.make_x(s)
    pk = synth.make_nvfp4_weights(s)
    # static scales from a sample of tokens (the weight-only oracle forward on 16 tokens)
    xs = x[:16]
    r0 = oracle.moe_ffn(xs, pk["router"], pk["gate"], pk["up"], pk["down"], pk["dgate"], pk["dup"], pk["ddown"],
                        top_k=8)
    sc = np.array([np.max(np.abs(oracle.widen_bf16(x))), np.max(np.abs(r0["h"])), np.max(np.abs(r0["h_d"]))]) / (6 * 448)
    out, r = run(torch, s, x, pk, sc)
    print(f"w4a4 near-ties: {check(s, x, pk, sc, out, r)}")


def test_w4a4_validation(torch):
    from sparse_moe_transformer_amd import MoeFFN, binding as B
    s = synth.FFNShape("mid_fp4", 16, 512, 32, 4, 128, 192, nvfp4=True)
    x, w, pk = nvfp4_inputs(s)
    xd, wd = G.up_bf16(x), G.up_nvfp4_weights(pk)
    out = torch.empty_like(xd)
    sc = G.up(np.ones(3, dtype=np.float32))
    st = torch.cuda.current_stream().cuda_stream
    d = {n: (wd[n]["q"].data_ptr(), wd[n]["scale"].data_ptr(), wd[n]["tensor_scale"].data_ptr())
         for n in ("gate", "up", "down", "dgate", "dup", "ddown")}
    ffn = MoeFFN.for_shape(s)

    def call(h, scale):
        return B.moe_ffn_forward_w4a4(h, 16, xd.data_ptr(), wd["router"].data_ptr(), None, d["gate"], d["up"],
                                      d["down"], d["dgate"], d["dup"], d["ddown"], scale, out.data_ptr(), st)

    assert call(ffn.h, sc.data_ptr()) == B.MOE_FFN_OK
    assert call(ffn.h, None) == B.MOE_FFN_ERR_INVALID_ARG
    assert call(ffn.h, sc.data_ptr() + 2) == B.MOE_FFN_ERR_INVALID_ARG
    bf = MoeFFN(s.hidden, s.experts, s.top_k, s.expert_dim, s.dense_dim, 16)
    assert call(bf.h, sc.data_ptr()) == B.MOE_FFN_ERR_UNSUPPORTED
    assert B.moe_ffn_quant_act_nvfp4(4, 24, xd.data_ptr(), out.data_ptr(), sc.data_ptr(), st) == \
        B.MOE_FFN_ERR_INVALID_ARG
    torch.cuda.synchronize()
