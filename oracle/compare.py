"""Parity criteria between the HIP layer and the oracle.

TEST INFRASTRUCTURE ONLY.

* Expert ids: bit-exact, except tokens whose oracle gap between the k-th and
  (k+1)-th biased score is below 1e-5 ("flagged"); for those any set is
  accepted whose every member scores at least the oracle's k-th score minus
  1e-5.
* Permutation: bit-exact against the oracle's grouping applied to the GPU's
  own ids.
* Outputs of a token are compared only where the GPU chose the oracle's
  expert set (every unflagged token; a flagged token with another valid set
  has no unique output and is reported, not compared).
* Floating-point outputs: max |gpu - ref| <= 2e-2 * RMS(ref) and
  mean |gpu - ref| / mean |ref| <= 5e-3, both in fp64 over the compared set.
  The fp32 MoE output y is held to this as is.  The bf16 layer output
  out = bf16(x + y) too, with one relief in its max-abs part: where the two
  fp32 values round to different bf16 neighbours the results differ by one
  bf16 step, which is not counted (at |out| >= 8 one step, 2^-4, exceeds
  2e-2 * RMS(out) by itself); its mean-relative part is on the raw difference.
"""
from __future__ import annotations

import numpy as np

MAX_ABS_FRAC = 2e-2
MEAN_REL = 5e-3
GAP_FLAG = 1e-5



def bf16_ulp(r: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |r| (8 significant bits)."""
    a = np.maximum(np.abs(r), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def close_report(gpu, ref, max_abs_frac: float = MAX_ABS_FRAC, bf16_out: bool = False) -> dict:
    """Tolerance report.  bf16_out: the compared values were each rounded once
    to bf16 from fp32, so one bf16 step of difference is the rounding decision
    falling the other way; it is not counted against the max-abs bound (the
    mean-relative figure is taken on the raw difference)."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    diff = np.abs(g - r)
    dmax = np.maximum(diff - bf16_ulp(r), 0.0) if bf16_out else diff
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    max_abs = float(dmax.max()) if r.size else 0.0
    mean_ref = float(np.mean(np.abs(r))) if r.size else 0.0
    mean_rel = float(diff.mean() / mean_ref) if mean_ref > 0 else float(diff.mean() if r.size else 0.0)
    finite = bool(np.all(np.isfinite(g)))
    ok = finite and max_abs <= max_abs_frac * rms and mean_rel <= MEAN_REL
    return dict(max_abs=max_abs, rms=rms, mean_rel=mean_rel, finite=finite, ok=ok)


def assert_close(gpu, ref, what: str, max_abs_frac: float = MAX_ABS_FRAC,
                 bf16_out: bool = False) -> dict:
    rep = close_report(gpu, ref, max_abs_frac, bf16_out)
    assert rep["ok"], f"{what}: {rep}"
    return rep


def check_routing(gpu_ids, gpu_w, ref: dict, w_rtol: float = 2e-5) -> dict:
    """Compare GPU top-k ids / weights with the oracle's routing of every token."""
    gpu_ids = np.asarray(gpu_ids)
    gpu_w = np.asarray(gpu_w, dtype=np.float64)
    ids, w, gap, sb = ref["ids"], ref["w"].astype(np.float64), ref["gap"], ref.get("sb")
    T, k = ids.shape
    flagged = gap < GAP_FLAG
    same = np.all(gpu_ids == ids, axis=1)
    bad = np.flatnonzero(~same & ~flagged)
    assert bad.size == 0, f"ids differ on unflagged tokens {bad[:10]} (of {T})"
    for t in np.flatnonzero(flagged & ~same):
        assert sb is not None
        kth = np.sort(sb[t])[::-1][k - 1]
        assert len(set(gpu_ids[t].tolist())) == k
        assert np.all(sb[t][gpu_ids[t]] >= kth - GAP_FLAG), f"token {t}"
    assert np.all(np.diff(gpu_ids, axis=1) > 0), "ids not ascending"
    np.testing.assert_allclose(gpu_w[same], w[same], rtol=w_rtol, atol=0)
    return dict(tokens=T, flagged=int(flagged.sum()), differing_flagged=int((flagged & ~same).sum()),
                agree=same)
