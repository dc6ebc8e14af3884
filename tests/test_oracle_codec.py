"""Pins for the oracle's number formats (OCP E4M3FN and bfloat16).

The pages name the format only ("e4m3"); the scale rule amax/448 fixes the
OCP E4M3FN variant.  Pins: values the OCP definition fixes, brute-force
nearest-value search, and torch's own float8_e4m3fn / bfloat16 casts as
library routines.
"""
import numpy as np
import pytest
import torch

from oracle.fp8 import E4M3_TABLE, bf16_round, e4m3_decode, e4m3_encode


def test_decode_fixed_points():
    t = E4M3_TABLE
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x38] == 1.0                # exponent field 7 = bias
    assert t[0x7E] == 448.0              # largest finite
    assert t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2      # no infinities, one NaN pattern per sign
    assert np.all(np.isfinite(t[~np.isnan(t)]))


def test_decode_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = e4m3_decode(np.arange(256, dtype=np.uint8))
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.all(both_nan | (ref == mine))


def test_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), codes)


def _brute_force(v: np.ndarray) -> np.ndarray:
    finite = [c for c in range(0x7F)]
    vals = E4M3_TABLE[finite]
    out = np.empty(v.shape, np.uint8)
    for i, x in enumerate(v.astype(np.float64)):
        a = abs(x)
        dist = np.abs(vals - a)
        best = np.flatnonzero(dist == dist.min())
        if len(best) > 1:                     # tie: the code with an even mantissa
            best = [b for b in best if (finite[b] & 1) == 0]
        c = finite[best[0]]
        out[i] = c | (0x80 if np.signbit(x) else 0)
    return out


def test_encode_matches_brute_force_nearest_even():
    rng = np.random.default_rng(1)
    # random magnitudes over the whole range, plus exact midpoints between codes
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 3000)).astype(np.float32)
    pos = E4M3_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    v = np.concatenate([mags, -mags, mids, -mids, [0.0, 448.0, -448.0, 2.0 ** -10, 2.0 ** -11]])
    v = v.astype(np.float32)
    assert np.array_equal(e4m3_encode(v), _brute_force(v))


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.normal(0, 50, 20000), rng.normal(0, 0.01, 5000),
                        rng.uniform(-448, 448, 5000)]).astype(np.float32)
    v = np.clip(v, -448, 448)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(v), ref)


def test_encode_monotone():
    v = np.sort(np.random.default_rng(3).uniform(-448, 448, 5000).astype(np.float32))
    dec = e4m3_decode(e4m3_encode(v))
    assert np.all(np.diff(dec) >= 0)


def test_encode_rejects_unclamped():
    with pytest.raises(ValueError):
        e4m3_encode(np.array([449.0], np.float32))


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e-3, 2000)]).astype(np.float32)
    # exact ties: bf16 value + half an ulp
    base = torch.from_numpy(v[:1000]).to(torch.bfloat16).to(torch.float32).numpy()
    ties = (base.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf16_round(v), ref)
