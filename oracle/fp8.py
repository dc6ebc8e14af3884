"""Number formats used by the layer: OCP FP8 E4M3FN and bfloat16.

The released configuration ("Kimi K2 · Architecture", Sources, config.json
quantization_config) names the weight format ``fp8`` / ``e4m3`` and
"Kimi-K2-Base" (Pretraining recipe, Training precision) names FP8-E4M3.  The
scale rule amax/448 fixes the OCP E4M3FN variant: exponent bias 7, largest
finite value 448, no infinities, S.1111.111 is NaN, subnormals m * 2^-9.

Encoding rounds to nearest, ties to even, keeps subnormals, and expects the
caller to have clamped the input to [-448, 448].
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _decode_one(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# decode table: code -> float64 value (exact)
E4M3_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
# the 127 non-negative finite values, ascending (codes 0x00 .. 0x7E)
_POS_VALUES = E4M3_TABLE[:0x7F].copy()
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (exact)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float32 values in [-448, 448] -> uint8 codes, round to nearest even."""
    v = np.asarray(v, dtype=np.float32)
    if np.any(np.isnan(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("e4m3_encode expects finite inputs clamped to +-448")
    a = np.abs(v).astype(np.float64)
    _, ex = np.frexp(a)                    # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)             # unbiased exponent; below 2^-6 the 2^-9 grid
    quantum = np.ldexp(1.0, e - 3)         # 3 mantissa bits
    n = np.rint(a / quantum)               # exact division by a power of two; rint = half-even
    q = n * quantum                        # a representable value (may carry to next binade)
    idx = np.searchsorted(_POS_VALUES, q)
    assert np.all(_POS_VALUES[idx] == q)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (idx.astype(np.uint8) | sign).astype(np.uint8)


def f32(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float32)


def bf16_round(v: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    bits = v.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """raw bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint32) << 16).astype(np.uint32).view(np.float32)
