"""Fit the correction-bias slope of the skewed-routing workload (test infrastructure).

The skewed workload keeps the layer's weights and sets the correction bias to
b_e = -beta * ln(rank_e), with rank a seeded permutation of 1..E, so that
expert popularity is Zipf-like.  beta is chosen so that the expert loads,
sorted in decreasing order, fall with a log-log slope of -1.1 over ranks
2..200 (rank 1, the hottest expert, is left out of the fit).  The routing is
the oracle's own (RMSNorm, router logits, sigmoid, biased top-8), evaluated on
inputs drawn on the CPU from the workload's seed; the bias only enters after
the logits, so the logits are computed once and beta is found by bisection.

    python -m oracle.fit_zipf_beta            # prints the fitted beta

The printed value is the constant frozen in the skewed workload's shape.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np

from .adapt import to_f32
from .moe_ref import rmsnorm, router_logits, select_topk, sigmoid_scores

TARGET_SLOPE = -1.1
RANKS = (2, 200)


def load_slope(loads: np.ndarray) -> float:
    """Least-squares slope of log(load) over log(rank), ranks RANKS (1-based)."""
    srt = np.sort(loads)[::-1].astype(np.float64)
    r = np.arange(RANKS[0], RANKS[1] + 1)
    y = np.log(np.maximum(srt[r - 1], 0.5))          # an empty expert counts as half a token
    return float(np.polyfit(np.log(r), y, 1)[0])


def fit(shape, seed: int = 0, lo: float = 0.0, hi: float = 0.2, iters: int = 30,
        log=print) -> float:
    import synth

    x, norm_w, w_router = synth.generate_router_inputs(shape, seed, device="cpu")
    h = rmsnorm(to_f32(x), to_f32(norm_w), shape.rms_eps, round_bf16=True)
    s = sigmoid_scores(router_logits(h, to_f32(w_router)))
    log(f"logits of {s.shape[0]} tokens x {s.shape[1]} experts computed")

    def slope(beta):
        bias = to_f32(synth.bias_vector(dataclasses.replace(shape, zipf_beta=beta), seed, "cpu"))
        ids, _ = select_topk((s + bias[None, :]).astype(np.float32), shape.top_k)
        return load_slope(np.bincount(ids.ravel(), minlength=shape.n_experts))

    # the slope falls monotonically (steeper) as beta grows
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if slope(mid) > TARGET_SLOPE:
            lo = mid
        else:
            hi = mid
    beta = 0.5 * (lo + hi)
    log(f"beta {beta:.4f}: slope {slope(beta):.3f}")
    return beta


if __name__ == "__main__":
    sys.path.insert(0, ".")
    import synth

    print(f"{fit(synth.K2_SKEWED):.4f}")
