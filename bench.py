#!/usr/bin/env python3
"""Benchmark of the MoE feed-forward block on one MI355X.

One step = one forward of the whole block (router, grouping, gate/up with
GeGLU, down, combine) over one batch of synthetic tokens at the Gemma 4
26B-A4B layer shape.  The headline line is the decode workload (T = 8); the
prefill workload (T = 4096) is reported in the same JSON line.

Inputs are generated on the host from fixed seeds and uploaded before timing;
the weights are replicated into several bit-identical device copies that the
steps rotate through, so each step streams its weights from HBM rather than
from the 256 MB last-level cache.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "MoE-FFN tokens/s per layer (26B-A4B shape, bf16) at T=8 and 4096; % roofline"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--prefill-steps", type=int, default=40)
    p.add_argument("--copies", type=int, default=4, help="weight copies rotated at decode")
    p.add_argument("--graph", action="store_true", help="replay each step from a HIP graph")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-skew", action="store_true")
    p.add_argument("--skew-steps", type=int, default=10)
    p.add_argument("--no-nvfp4", action="store_true")
    p.add_argument("--nvfp4-steps", type=int, default=3, help="timed chains of --nvfp4-layers layers")
    p.add_argument("--nvfp4-layers", type=int, default=30)
    p.add_argument("--no-block", action="store_true", help="skip the sandwich-norm sub-block leg")
    p.add_argument("--block-steps", type=int, default=100)
    p.add_argument("--no-dense", action="store_true", help="skip the E4B dense FFN leg")
    p.add_argument("--no-fp8", action="store_true", help="skip the FP8 weight leg")
    p.add_argument("--no-w4a4", action="store_true", help="skip the NVFP4 W4A4 leg")
    p.add_argument("--dense-steps", type=int, default=100)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-decode-only", action="store_true", help="time the oracle at decode only")
    return p.parse_args()


def to_dev_bf16(torch, a):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda")


# The streaming path runs the first DENSE_ROUTE_EIGHTHS/8 of the dense
# branch's gate/up units (64 columns x one of 4 K-slices of whole 64-row
# groups each, K-slice fastest, then gate/up, then the column block) in the
# router's launch and the rest in the routed gate/up launch.  Mirrors the
# library's split (kDenseRouteEighths in the streaming kernels' source).
DENSE_ROUTE_EIGHTHS = 5
DENSE_UNIT_COLS, DENSE_KSLICES = 64, 4


def dense_units_in_gateup(shape):
    """(weight bytes, output columns) of the dense gate/up units that the
    routed gate/up launch runs."""
    H, D = shape.hidden, shape.dense_dim
    if D == 0:
        return 0, 0
    ks = min(DENSE_KSLICES, H // 64)
    ud = -(-D // DENSE_UNIT_COLS) * 2 * ks
    g64 = H // 64
    wbytes = cols = 0
    for u in range(ud * DENSE_ROUTE_EIGHTHS // 8, ud):
        s, nb = u % ks, u // (2 * ks)
        rows = ((s + 1) * g64 // ks - s * g64 // ks) * 64
        nc = min(DENSE_UNIT_COLS, D - nb * DENSE_UNIT_COLS)
        wbytes += rows * nc * 2
        cols += nc if s == 0 else 0
    return wbytes, cols


def routed_gateup_bytes(shape, n_act):
    """Algorithmic HBM bytes of the routed gate/up weight-streaming launch:
    the gate and up matrices of the n_act experts that have tokens and the
    dense gate/up units it runs, the T input rows, and the T*k hidden rows
    plus the dense units' T output columns at bf16 (the kernel's fp32
    partial sums are an implementation choice, not counted)."""
    H, I, T, k = shape.hidden, shape.expert_dim, shape.tokens, shape.top_k
    dw, dc = dense_units_in_gateup(shape)
    return n_act * 2 * H * I * 2 + dw + T * H * 2 + T * k * I * 2 + T * dc * 2


def step_bytes(shape, n_act):
    """Algorithmic HBM bytes of one whole forward (weights once, activations once)."""
    H, I, D, E, T = shape.hidden, shape.expert_dim, shape.dense_dim, shape.experts, shape.tokens
    return n_act * 3 * H * I * 2 + 3 * H * D * 2 + H * E * 2 + 2 * T * H * 2


def gateup_flops(shape):
    H, I, D, T, k = shape.hidden, shape.expert_dim, shape.dense_dim, shape.tokens, shape.top_k
    return 2 * T * k * H * 2 * I + 2 * T * H * 2 * D


def step_flops(shape):
    H, I, D, E, T, k = (shape.hidden, shape.expert_dim, shape.dense_dim, shape.experts,
                        shape.tokens, shape.top_k)
    return T * (2 * H * E + k * 2 * 3 * H * I + 2 * 3 * H * D)


def upload_nvfp4(torch, pk):
    out = {"router": to_dev_bf16(torch, pk["router"])}
    for n in ("gate", "up", "down", "dgate", "dup", "ddown"):
        m = pk.get(n)
        out[n] = None if m is None else {
            "q": torch.from_numpy(np.ascontiguousarray(m["q"])).cuda(),
            "scale": torch.from_numpy(np.ascontiguousarray(m["scale"])).cuda(),
            "tensor_scale": torch.from_numpy(np.ascontiguousarray(m["tensor_scale"])).cuda()}
    return out


def upload_fp8(torch, pk):
    out = {"router": to_dev_bf16(torch, pk["router"]) if pk["router"] is not None else None}
    for n in ("gate", "up", "down", "dgate", "dup", "ddown"):
        m = pk.get(n)
        out[n] = None if m is None else {
            "q8": torch.from_numpy(np.ascontiguousarray(m["q8"])).cuda(),
            "tensor_scale": torch.from_numpy(np.ascontiguousarray(m["tensor_scale"])).cuda()}
    return out


def clone_fp8(w):
    return {k: (None if v is None else v.clone() if not isinstance(v, dict) else
                {kk: vv.clone() for kk, vv in v.items()}) for k, v in w.items()}


def nvfp4_layer_weight_bytes(shape):
    """Packed bytes of one NVFP4 layer: 0.5 B codes + 1/16 B scales per weight,
    4 B per matrix tensor scale, plus the bf16 router."""
    H, I, D, E = shape.hidden, shape.expert_dim, shape.dense_dim, shape.experts
    nw = E * 3 * H * I + 3 * H * D
    return nw // 2 + nw // 16 + (3 * E + 3) * 4 + H * E * 2


def run_workload(torch, shape, steps, warmup, copies, graph, layers=1, norms=False, w4a4=False):
    """Time `steps` forwards; returns a dict of measurements.

    bf16 workloads rotate `copies` bit-identical weight copies.  The NVFP4
    stack chains `layers` residual layers (x <- x + FFN_l(x), in place) over
    `copies` distinct seeded layers; a step is one layer."""
    import synth
    from sparse_moe_transformer_amd import MoeFFN, binding

    x = synth.make_x(shape)
    xd = to_dev_bf16(torch, x)
    bias = synth.zipf_bias(shape.experts) if shape.skew else None
    bd = torch.from_numpy(bias).cuda() if bias is not None else None
    w = None
    if getattr(shape, "fp8", False):
        base = upload_fp8(torch, synth.make_fp8_weights(shape))
        sets = [base] + [clone_fp8(base) for _ in range(copies - 1)]
        out = torch.empty_like(xd)
        ffn = MoeFFN.for_shape(shape)

        def fwd(i):
            ffn.forward_fp8(xd, sets[i % copies], out, bd)
    elif shape.nvfp4 and w4a4:
        # one NVFP4 layer with NVFP4 activations; static global scales of x,
        # h and h_d as a min/max observer would set them (amax / (6 * 448)),
        # taking amax 4 for the hidden rows; copies are distinct seeded layers
        sets = [upload_nvfp4(torch, synth.make_nvfp4_weights(shape, layer=l)) for l in range(copies)]
        ffn = MoeFFN.for_shape(shape)
        amax_x = float(np.max(np.abs(synth.bf16_bits_to_f32(x))))
        scales = torch.tensor([amax_x, 4.0, 4.0], dtype=torch.float32, device="cuda") / (6 * 448)
        out = torch.empty_like(xd)

        def fwd(i):
            ffn.forward_w4a4(xd, sets[i % copies], scales, out, bd)
    elif shape.nvfp4 and layers == 0:
        # one NVFP4 layer on its own (decode): bit-identical copies rotated
        base = upload_nvfp4(torch, synth.make_nvfp4_weights(shape))
        sets = [base] + [clone_fp8(base) for _ in range(copies - 1)]
        ffn = MoeFFN.for_shape(shape)
        out = torch.empty_like(xd)
        layers = 1

        def fwd(i):
            ffn.forward_nvfp4(xd, sets[i % copies], out, bd)
    elif shape.nvfp4:
        sets = [upload_nvfp4(torch, synth.make_nvfp4_weights(shape, layer=l)) for l in range(copies)]
        ffn = MoeFFN.for_shape(shape, accumulate=True)
        x0 = xd.clone()
        out = xd

        def fwd(i):
            ffn.forward_nvfp4(xd, sets[i % copies], xd, bd)
    else:
        w = synth.make_weights(shape)
        base = {k: to_dev_bf16(torch, v) for k, v in w.items() if v is not None}
        sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]
        out = torch.empty_like(xd)
        ffn = MoeFFN.for_shape(shape)
        if norms:
            # the sub-block with sandwich norms: seeded gains around 1
            rng = np.random.default_rng(1000)
            pre = torch.from_numpy((1.0 + 0.2 * rng.standard_normal(shape.hidden)).astype(np.float32)).cuda()
            post = torch.from_numpy((1.0 + 0.2 * rng.standard_normal(shape.hidden)).astype(np.float32)).cuda()

            def fwd(i):
                ffn.forward_block(xd, sets[i % copies], pre, post, out, 1e-6, bd)
        else:
            def fwd(i):
                ffn.forward(xd, sets[i % copies], out, bd)
    torch.cuda.synchronize()

    graphs = None
    if graph:
        for i in range(copies):  # warm the kernels before capture
            fwd(i)
        torch.cuda.synchronize()
        graphs = []
        for i in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fwd(i)
            graphs.append(g)
        torch.cuda.synchronize()

    def step(i):
        if graphs is not None:
            graphs[i % copies].replay()
        else:
            fwd(i)

    def restart():
        # the stack runs in place: restart each chain of `layers` from x
        if shape.nvfp4 and not w4a4 and layers > 1:
            xd.copy_(x0)

    for i in range(warmup):
        if i % layers == 0:
            restart()
        step(i)
    torch.cuda.synchronize()
    if shape.experts > 0:
        counts = ffn.routing(shape.tokens)["counts"].cpu().numpy()
    else:  # a dense FFN: no routing
        counts = np.zeros(0, dtype=np.int32)
    n_act = int((counts > 0).sum())

    # timed region: `steps` forwards (chains of `layers` for the stack; the
    # restarts copy 2.3 MB and are timed too)
    t0 = time.perf_counter()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        if layers > 1 and i % layers == 0:
            restart()
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / steps

    # per-stage durations: HIP events recorded by the library on the
    # forward's stream around each kernel group, over `steps` eager forwards
    stage_mask = (1 << binding.MOE_FFN_NUM_STAGES) - 1
    binding.check(binding.moe_ffn_profile_begin(ffn.h, stage_mask, steps))
    for i in range(steps):
        if layers > 1 and i % layers == 0:
            restart()
        fwd(i)
    rc, stage_ms, stage_n = binding.moe_ffn_profile_end(ffn.h)
    binding.check(rc)
    stage_avg_us = [1000.0 * m / n if n else 0.0 for m, n in zip(stage_ms, stage_n)]
    ffn.close()
    return {"ms_per_step": ms_step, "wall_s": wall, "n_act": n_act, "counts": counts,
            "stage_avg_us": stage_avg_us, "x": x, "w": w, "bias": bias}


STAGES = ["route", "align", "gateup", "down", "combine", "geglu"]

# HBM traffic of a roofline kernel, from the committed rocprofv3 --pmc summary;
# valid only while the kernel's sources are unchanged (their hash is stored)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "sparse_moe_transformer_amd", "csrc")


def source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_of(kernel):
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if source_hash(rec["sources"]) != rec["source_hash"]:
        return None
    return rec["bytes_per_launch"]


def host_info():
    """CPU model (from /proc/cpuinfo), the BLAS library and its thread count
    (from threadpoolctl) that the oracle's numpy uses."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    from threadpoolctl import threadpool_info
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    vendor = blas[0].get("internal_api", "?") if blas else "none"
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    return {"cpu_model": model, "blas": vendor, "blas_threads": int(threads),
            "affinity_cpus": len(os.sched_getaffinity(0))}


def time_oracle(fn, runs):
    """Median (and every) wall time of `runs` calls of fn."""
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), ts


def cpu_baseline(dec, x, w, bias, legs=True):
    """The oracle (as it stands, fp64 numpy) on the host cores: decode (the
    headline's workload, median of 3 forwards) and, with legs, the tiny
    workload and prefill (median of 3), skew and one NVFP4 stack layer (one
    run each), each as tokens/s of the workload it times."""
    import oracle
    import synth
    info = host_info()

    def ffn(xx, ww, k, b=None):
        return oracle.moe_ffn(xx, ww["router"], ww["gate"], ww["up"], ww["down"], ww["dgate"], ww["dup"],
                              ww["ddown"], top_k=k, bias=b, intermediates=False)

    med, ts = time_oracle(lambda: ffn(x, w, dec.top_k, bias), 3)
    out = {"value": dec.tokens / med, "unit": "tokens/s", "cores": info["blas_threads"], "kind": "oracle",
           "sample": f"median of 3 full fp64 oracle forwards of the decode workload (T={dec.tokens}, "
                     f"{med:.2f} s each); numpy on {info['blas']} with {info['blas_threads']} threads",
           "host": info}
    if not legs:
        return out
    out["legs"] = {}

    def leg(name, shape, runs, ww=None, b=None):
        xx = synth.make_x(shape)
        ww = ww if ww is not None else synth.make_weights(shape)
        m, tt = time_oracle(lambda: ffn(xx, ww, shape.top_k, b), runs)
        out["legs"][name] = {"tokens": shape.tokens, "value": shape.tokens / m, "unit": "tokens/s",
                             "seconds": [round(t, 3) for t in tt], "runs": runs}

    leg("tiny", synth.TINY, 3)
    leg("prefill", synth.PREFILL, 3, ww=w)
    leg("skew", synth.SKEW, 1, ww=w, b=synth.zipf_bias(synth.SKEW.experts))
    leg("nvfp4_stack_layer", synth.NVFP4_STACK, 1, ww=synth.make_nvfp4_weights(synth.NVFP4_STACK))
    return out


def run_nvfp4_stack(torch, shape, n_layers, chains):
    """The NVFP4 residual stack x <- x + FFN_l(x) over n_layers distinct
    layers, in place.  Two layers are generated and quantised on the host
    from their seeds; layer l takes base layer l % 2's packed experts in a
    seeded permutation of the expert axis (copied into memory of its own),
    its own seeded bf16 router and a copy of the base's dense matrices, so
    each layer streams its own 439 MB.  Returns the time per chain."""
    import synth
    from sparse_moe_transformer_amd import MoeFFN, binding
    H, E = shape.hidden, shape.experts
    bases = [upload_nvfp4(torch, synth.make_nvfp4_weights(shape, layer=l)) for l in range(2)]
    layers = []
    for l in range(n_layers):
        b = bases[l % 2]
        perm = torch.from_numpy(np.random.default_rng([0, l, 99]).permutation(E)).cuda()
        lw = {"router": to_dev_bf16(torch, synth.normal_bf16(0, l, synth.TID_ROUTER, (H, E), H ** -0.5))}
        for n in ("gate", "up", "down"):
            lw[n] = {k: v.index_select(0, perm).contiguous() for k, v in b[n].items()}
        for n in ("dgate", "dup", "ddown"):
            lw[n] = {k: v.clone() for k, v in b[n].items()}
        layers.append(lw)
    del bases
    x0 = to_dev_bf16(torch, synth.make_x(shape))
    xd = x0.clone()
    ffn = MoeFFN.for_shape(shape, accumulate=True)

    def chain():
        xd.copy_(x0)
        for lw in layers:
            ffn.forward_nvfp4(xd, lw, xd)

    chain()  # warm up
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(chains):
        chain()
    ev1.record()
    torch.cuda.synchronize()
    ms_chain = ev0.elapsed_time(ev1) / chains
    stage_mask = (1 << binding.MOE_FFN_NUM_STAGES) - 1
    binding.check(binding.moe_ffn_profile_begin(ffn.h, stage_mask, n_layers))
    chain()
    rc, stage_ms, stage_n = binding.moe_ffn_profile_end(ffn.h)
    binding.check(rc)
    ffn.close()
    return ms_chain, [1000.0 * m / n if n else 0.0 for m, n in zip(stage_ms, stage_n)]


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the block shards by tokens with replicated weights; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import synth

    dec = synth.DECODE
    r = run_workload(torch, dec, args.steps, args.warmup, args.copies, args.graph)
    gu_bytes = routed_gateup_bytes(dec, r["n_act"])
    gu_us = r["stage_avg_us"][2]
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": dec.tokens / (r["ms_per_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded x ~ N(0,1), weights ~ N(0,1/fan_in), rounded to bf16",
        "config": {"workload": "Gemma 4 26B-A4B MoE FFN layer, decode T=8 (H=2816, E=128, "
                               "top-8, expert 704, dense 2112)",
                   "tokens": dec.tokens, "hidden": dec.hidden, "experts": dec.experts,
                   "top_k": dec.top_k, "expert_dim": dec.expert_dim, "dense_dim": dec.dense_dim,
                   "weight_copies": args.copies, "graph": bool(args.graph),
                   "active_experts": r["n_act"]},
        "roofline": {"bound": "hbm", "scope": "dominant kernel (the whole step is step_hbm)",
                     "kernel": "k_stream_gateup (routed gate/up + 3/8 of the dense units, weight streaming)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes": gu_bytes, "avg_us": gu_us},
        "step_hbm": {"algorithmic_bytes": step_bytes(dec, r["n_act"]),
                     "GBps": step_bytes(dec, r["n_act"]) / (r["ms_per_step"] * 1e-3) / 1e9,
                     "frac": step_bytes(dec, r["n_act"]) / (r["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "stage_avg_us": dict(zip(STAGES, [round(v, 2) for v in r["stage_avg_us"]])),
    }
    line["roofline"]["traffic"] = traffic_of("k_stream_gateup")
    if not args.no_block:
        rb = run_workload(torch, dec, args.block_steps, args.warmup, args.copies, args.graph, norms=True)
        line["sandwich_block"] = {
            "workload": "same layer, decode T=8, the sub-block x + RMSNorm(FFN(RMSNorm(x))) "
                        "(pre-norm kernel, post-norm and residual in the combine)",
            "tokens": dec.tokens,
            "value": dec.tokens / (rb["ms_per_step"] * 1e-3),
            "unit": "tokens/s",
            "ms_per_step": rb["ms_per_step"],
            "steps": args.block_steps,
            "us_over_plain_ffn": (rb["ms_per_step"] - r["ms_per_step"]) * 1000.0,
            "stage_avg_us": dict(zip(STAGES, [round(v, 2) for v in rb["stage_avg_us"]])),
        }
    if not args.no_prefill:
        pre = synth.PREFILL
        rp = run_workload(torch, pre, args.prefill_steps, max(3, args.warmup // 4), 2, args.graph)
        gu_us = rp["stage_avg_us"][2]
        tf = gateup_flops(pre) / (gu_us * 1e-6) / 1e12
        step_tf = step_flops(pre) / (rp["ms_per_step"] * 1e-3) / 1e12
        line["prefill"] = {
            "workload": "same layer, prefill T=4096", "tokens": pre.tokens,
            "value": pre.tokens / (rp["ms_per_step"] * 1e-3), "unit": "tokens/s",
            "ms_per_step": rp["ms_per_step"], "steps": args.prefill_steps,
            "step_tflops": step_tf, "step_mfma_frac": step_tf / BF16_PEAK_TFLOPS,
            "roofline": {"bound": "mfma", "kernel": "k_gemm<2,0,true> (gate/up MFMA GEMM: routed + dense, GeGLU)",
                         "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / BF16_PEAK_TFLOPS, "traffic": traffic_of("k_gemm<2, 0>"),
                         "algorithmic_flops": gateup_flops(pre), "avg_us": gu_us},
            "stage_avg_us": dict(zip(STAGES, [round(v, 2) for v in rp["stage_avg_us"]])),
        }
    if not args.no_skew:
        sk = synth.SKEW
        rs = run_workload(torch, sk, args.skew_steps, 2, 2, args.graph)
        c = rs["counts"]
        line["skew"] = {
            "workload": "same layer, T=16384, Zipf(1.2) expert loads via a router logit bias",
            "tokens": sk.tokens, "value": sk.tokens / (rs["ms_per_step"] * 1e-3), "unit": "tokens/s",
            "ms_per_step": rs["ms_per_step"], "steps": args.skew_steps,
            "step_mfma_frac": step_flops(sk) / (rs["ms_per_step"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "load_max": int(c.max()), "load_min": int(c.min()),
            "load_max_over_mean": float(c.max() / c.mean()),
            "stage_avg_us": dict(zip(STAGES, [round(v, 2) for v in rs["stage_avg_us"]])),
        }
    if not args.no_nvfp4:
        st = synth.NVFP4_STACK
        L = args.nvfp4_layers
        ms_chain, stage_us = run_nvfp4_stack(torch, st, L, args.nvfp4_steps)
        us = ms_chain * 1e3 / L
        wbytes = nvfp4_layer_weight_bytes(st)
        line["nvfp4_stack"] = {
            "workload": f"residual stack of {L} distinct NVFP4 weight-only layers, T=1024 (x <- x + FFN_l(x) in "
                        f"place; layers built from 2 seeded quantised layers by seeded expert permutations, each "
                        f"with its own seeded router and its own copy of every matrix)",
            "tokens": st.tokens, "layers": L, "stack_ms": ms_chain, "chains_timed": args.nvfp4_steps,
            "value": st.tokens / (us * 1e-6), "unit": "tokens/s per layer", "us_per_layer": us,
            "layer_weight_bytes": wbytes, "hbm_frac": wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "mfma_frac": step_flops(st) / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
            "stage_avg_us": dict(zip(STAGES, [round(v, 2) for v in stage_us])),
        }
    if not args.no_nvfp4:
        # one NVFP4 layer at decode (T = 8): weights streamed into registers
        sd = synth.NVFP4_STACK.with_tokens(8)
        rd = run_workload(torch, sd, args.steps, args.warmup, args.copies, args.graph, layers=0)
        H, I, D, E = sd.hidden, sd.expert_dim, sd.dense_dim, sd.experts
        per_w = 0.5 + 1.0 / 16  # packed bytes per weight: the code nibble and its share of a group scale
        nb = int(rd["n_act"] * 3 * H * I * per_w + 3 * H * D * per_w + H * E * 2 + 2 * sd.tokens * H * 2)
        line["nvfp4_decode"] = {
            "workload": "one NVFP4 weight-only layer at decode, T=8 (packed weights rotated over bit-identical copies)",
            "tokens": sd.tokens, "value": sd.tokens / (rd["ms_per_step"] * 1e-3), "unit": "tokens/s",
            "ms_per_step": rd["ms_per_step"], "steps": args.steps, "active_experts": rd["n_act"],
            "algorithmic_bytes": nb, "hbm_frac": nb / (rd["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "stage_avg_us": dict(zip(STAGES, [round(v, 2) for v in rd["stage_avg_us"]])),
        }
    if not args.no_dense:
        # the dense GeGLU FFN of the E4B model (2560 -> 10240 -> 2560, no experts)
        dd, dp = synth.E4B_DECODE, synth.E4B_PREFILL
        H, D = dd.hidden, dd.dense_dim
        rd = run_workload(torch, dd, args.dense_steps, args.warmup, args.copies, args.graph)
        dbytes = 3 * H * D * 2 + 2 * dd.tokens * H * 2
        dense = {
            "workload": "Gemma 4 E4B dense GeGLU FFN (H=2560, D=10240, no experts)",
            "decode": {"tokens": dd.tokens, "value": dd.tokens / (rd["ms_per_step"] * 1e-3),
                       "unit": "tokens/s", "ms_per_step": rd["ms_per_step"], "steps": args.dense_steps,
                       "algorithmic_bytes": dbytes,
                       "hbm_frac": dbytes / (rd["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "stage_avg_us": dict(zip(STAGES, [round(v, 2) for v in rd["stage_avg_us"]]))},
        }
        if not args.no_prefill:
            rq = run_workload(torch, dp, args.prefill_steps, max(3, args.warmup // 4), 2, args.graph)
            fl = 2 * dp.tokens * 3 * H * D
            gu_us = rq["stage_avg_us"][2]
            dense["prefill"] = {
                "tokens": dp.tokens, "value": dp.tokens / (rq["ms_per_step"] * 1e-3), "unit": "tokens/s",
                "ms_per_step": rq["ms_per_step"], "steps": args.prefill_steps,
                "step_mfma_frac": fl / (rq["ms_per_step"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                "gateup_mfma_frac": (2 * dp.tokens * 2 * H * D) / (gu_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
                "stage_avg_us": dict(zip(STAGES, [round(v, 2) for v in rq["stage_avg_us"]]))}
        line["e4b_dense"] = dense
    if not args.no_fp8:
        # FP8 weight-only (e4m3fn codes + per-matrix scale): one byte per weight
        from dataclasses import replace
        f8 = replace(dec, fp8=True)
        rf = run_workload(torch, f8, args.steps, args.warmup, args.copies, args.graph)
        H, I = f8.hidden, f8.expert_dim
        gu8 = rf["n_act"] * 2 * H * I + f8.tokens * H * 2 + f8.tokens * f8.top_k * I * 2
        step8 = rf["n_act"] * 3 * H * I + 3 * H * f8.dense_dim + H * f8.experts * 2 + 2 * f8.tokens * H * 2
        gu_us8 = rf["stage_avg_us"][2]
        fp8 = {
            "workload": "same layer with FP8 e4m3fn expert and dense weights (per-matrix scale), router bf16",
            "decode": {"tokens": f8.tokens, "value": f8.tokens / (rf["ms_per_step"] * 1e-3), "unit": "tokens/s",
                       "ms_per_step": rf["ms_per_step"], "steps": args.steps, "active_experts": rf["n_act"],
                       "gateup_hbm_frac": gu8 / (gu_us8 * 1e-6) / 1e9 / HBM_PEAK_GBS,
                       "step_hbm_frac": step8 / (rf["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "stage_avg_us": dict(zip(STAGES, [round(v, 2) for v in rf["stage_avg_us"]]))},
        }
        if not args.no_prefill:
            fp = replace(synth.PREFILL, fp8=True)
            rq = run_workload(torch, fp, args.prefill_steps, max(3, args.warmup // 4), 2, args.graph)
            fp8["prefill"] = {
                "tokens": fp.tokens, "value": fp.tokens / (rq["ms_per_step"] * 1e-3), "unit": "tokens/s",
                "ms_per_step": rq["ms_per_step"], "steps": args.prefill_steps,
                "step_mfma_frac": step_flops(fp) / (rq["ms_per_step"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                "stage_avg_us": dict(zip(STAGES, [round(v, 2) for v in rq["stage_avg_us"]]))}
        line["fp8"] = fp8
    if not args.no_w4a4:
        from dataclasses import replace
        st = replace(synth.NVFP4_STACK, layers=1)
        rw = run_workload(torch, st, 40, 8, 2, False, w4a4=True)
        us = rw["ms_per_step"] * 1e3
        line["w4a4"] = {
            "workload": "one NVFP4 layer with NVFP4 activations (W4A4), T=1024, 2 distinct seeded layers rotated",
            "tokens": st.tokens, "value": st.tokens / (us * 1e-6), "unit": "tokens/s per layer",
            "us_per_layer": us, "steps": 40,
            "mfma_frac": step_flops(st) / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
            "stage_avg_us": dict(zip(STAGES, [round(v, 2) for v in rw["stage_avg_us"]])),
        }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(dec, r["x"], r["w"], r["bias"], legs=not args.cpu_decode_only)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
