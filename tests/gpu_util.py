"""Helpers shared by the GPU tests: upload seeded inputs, compare with the oracle."""
from __future__ import annotations

import numpy as np

import oracle
import synth

TOL = 2e-2  # |gpu - oracle| <= TOL * (|oracle| + rms(oracle)), bf16 output


def dev():
    import torch
    return torch.device("cuda", 0)


def up_bf16(a):
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return t.to(dev())


def up(a, dtype=None):
    import torch
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def up_weights(w):
    return {k: up_bf16(v) for k, v in w.items()}


def up_nvfp4_weights(w):
    out = {"router": up_bf16(w["router"])}
    for n in ("gate", "up", "down", "dgate", "dup", "ddown"):
        m = w.get(n)
        out[n] = None if m is None else {"q": up(m["q"]), "scale": up(m["scale"]),
                                         "tensor_scale": up(m["tensor_scale"])}
    return out


def up_fp8_weights(w):
    out = {"router": up_bf16(w["router"])}
    for n in ("gate", "up", "down", "dgate", "dup", "ddown"):
        m = w.get(n)
        out[n] = None if m is None else {"q8": up(m["q8"]), "tensor_scale": up(m["tensor_scale"])}
    return out


def to_f64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def to_np(t):
    return t.detach().cpu().numpy()


def block_close(gpu, ref, tol=TOL):
    """Return (ok, worst ratio) for the bf16 output rule."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = tol * (np.abs(ref) + rms)
    err = np.abs(gpu - ref)
    ratio = float(np.max(err / np.maximum(bound, 1e-300))) if ref.size else 0.0
    return bool(np.all(err <= bound)), ratio


def assert_block_close(gpu, ref, tol=TOL, what="output"):
    ok, ratio = block_close(gpu, ref, tol)
    assert ok, f"{what}: worst |gpu-oracle| / bound = {ratio:.3f}"


def check_routing(gpu_idx, gpu_w, ref, w_tol=1e-5):
    """Routing sets bit-exact on every token that is not a near-tie; weights
    within w_tol where the sets agree.  Returns the near-tie mask."""
    near = ref["near_tie"]
    same = np.all(gpu_idx == ref["topk_idx"], axis=1)
    bad = ~same & ~near
    assert not bad.any(), f"routing differs on {int(bad.sum())} non-near-tie tokens, e.g. {np.where(bad)[0][:5]}"
    if same.any():
        err = np.max(np.abs(gpu_w[same] - ref["topk_w"][same]))
        assert err <= w_tol, f"routing weights differ by {err}"
    return near


def check_align(gpu, topk_idx, E):
    """counts, offsets, perm, pos bit-exact against the oracle's grouping of
    the GPU's own routing."""
    a = oracle.align(topk_idx, E)
    for n in ("counts", "offsets", "perm"):
        assert np.array_equal(gpu[n].reshape(-1), a[n].reshape(-1)), n
    assert np.array_equal(gpu["pos"].reshape(-1), a["pos"].reshape(-1)), "pos"
    return a


def make_inputs(shape, seed=0, layer=0):
    x = synth.make_x(shape, seed, layer)
    w = synth.make_weights(shape, seed, layer)
    bias = synth.zipf_bias(shape.experts, seed=seed, layer=layer) if shape.skew else None
    return x, w, bias
