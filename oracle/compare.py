"""Parity criteria between the HIP layer and the oracle.

TEST INFRASTRUCTURE ONLY.

* Expert ids: bit-exact, except tokens whose oracle gap between the k-th and
  (k+1)-th biased score is below 1e-5 ("flagged"); for those any set is
  accepted whose every member scores at least the oracle's k-th score minus
  1e-5.
* Permutation: bit-exact against the oracle's grouping applied to the GPU's
  own ids.
* Floating-point outputs: max |gpu - ref| <= 2e-2 * RMS(ref) and
  mean |gpu - ref| / mean |ref| <= 5e-3, both in fp64 over the compared set.
"""
from __future__ import annotations

import numpy as np

MAX_ABS_FRAC = 2e-2
MEAN_REL = 5e-3
GAP_FLAG = 1e-5


def close_report(gpu, ref) -> dict:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    diff = np.abs(g - r)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    max_abs = float(diff.max()) if r.size else 0.0
    mean_ref = float(np.mean(np.abs(r))) if r.size else 0.0
    mean_rel = float(diff.mean() / mean_ref) if mean_ref > 0 else float(diff.mean())
    finite = bool(np.all(np.isfinite(g)))
    ok = finite and max_abs <= MAX_ABS_FRAC * rms and mean_rel <= MEAN_REL
    return dict(max_abs=max_abs, rms=rms, mean_rel=mean_rel, finite=finite, ok=ok)


def assert_close(gpu, ref, what: str) -> dict:
    rep = close_report(gpu, ref)
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
    ok_w = same
    np.testing.assert_allclose(gpu_w[ok_w], w[ok_w], rtol=w_rtol, atol=0)
    return dict(tokens=T, flagged=int(flagged.sum()), differing_flagged=int((flagged & ~same).sum()))
