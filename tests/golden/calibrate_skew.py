"""Calibrate the logit-bias scale of the skewed-load workload.

The workload adds b_e = lambda * ln p_e to the router logits, with
p_e ∝ (pi_e + 1)^-1.2 over a seeded permutation pi of the experts
(``synth.zipf_bias``), and asks for expert loads whose sorted log-log slope
over ranks 9..128 is -1.2 (ranks 1..8 saturate near T because a token picks
an expert at most once).  The loads come from the CPU oracle's router.

Run ``python tests/golden/calibrate_skew.py`` to print the bisection result;
the value is stored as ``synth.SKEW_LAMBDA`` and re-checked by
``tests/test_oracle_pins.py::test_skew_lambda_gives_zipf_slope``.
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import oracle  # noqa: E402
import synth  # noqa: E402

_CACHE = {}


def _inputs(seed):
    if seed not in _CACHE:
        s = synth.SKEW
        x = synth.make_x(s, seed)
        wr = synth.normal_bf16(seed, 0, synth.TID_ROUTER, (s.hidden, s.experts), s.hidden ** -0.5)
        _CACHE[seed] = (x, wr)
    return _CACHE[seed]


def load_slope(lam, seed=0):
    """(slope over ranks 9..128, per-expert loads) at bias scale ``lam``."""
    s = synth.SKEW
    x, wr = _inputs(seed)
    b = synth.zipf_bias(s.experts, lam, synth.ZIPF_S, seed)
    r = oracle.route(x, wr, s.top_k, bias=b)
    loads = np.bincount(r["topk_idx"].ravel(), minlength=s.experts)
    srt = np.sort(loads)[::-1].astype(np.float64)
    ranks = np.arange(1, s.experts + 1)
    sel = (ranks >= 9) & (srt > 0)
    slope = np.polyfit(np.log(ranks[sel]), np.log(srt[sel]), 1)[0]
    return slope, loads


def calibrate(seed=0, lo=0.0, hi=2.0, steps=20):
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        slope, _ = load_slope(mid, seed)
        if slope > -synth.ZIPF_S:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


if __name__ == "__main__":
    lam = calibrate()
    slope, loads = load_slope(lam)
    print(f"lambda={lam:.7f} slope={slope:.4f} max={loads.max()} min={loads.min()} "
          f"max/mean={loads.max() / loads.mean():.2f}")
