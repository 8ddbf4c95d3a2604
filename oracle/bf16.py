"""Exact rounding of float64 to bfloat16 (oracle) — TEST INFRASTRUCTURE ONLY.

bfloat16 keeps 8 significant bits and float32's exponent range. Rounding is to
nearest, ties to even, applied once to the exact fp64 value (no intermediate
float32 step), with gradual underflow below 2^-126 and overflow to infinity.
"""
from __future__ import annotations

import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x):
    """fp64 array -> fp64 array holding the nearest bfloat16 values."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)                       # xf = m * 2**e, 0.5 <= |m| < 1
    qexp = np.maximum(e - 8, -133)            # quantum: 8 significant bits
    quantum = np.ldexp(1.0, qexp)
    r = np.rint(xf / quantum) * quantum       # rint is round-half-even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def bf16_bits(x):
    """Bit patterns (uint16) of round_bf16(x)."""
    r = round_bf16(x).astype(np.float32)      # exact: bf16 values fit fp32
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f64(bits):
    """uint16 bfloat16 bit patterns -> fp64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
